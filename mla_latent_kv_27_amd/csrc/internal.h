// Host-side launch interfaces between the C ABI (mla_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

enum class DType { F32 = 0, BF16 = 1 };

inline size_t dsize(DType t) { return t == DType::BF16 ? 2 : 4; }

// RoPE frequencies: theta_k = base^(-2k/d_hr), or their YaRN form when scale > 1 (turns counted
// over orig_ctx positions, ramp from alpha to beta turns).
struct RopeFreq {
  double base = 10000.0;
  double scale = 1.0;
  double orig_ctx = 0.0, alpha = 1.0, beta = 32.0;
};
// Entry i = r * half + k of the RoPE table: (cos, sin)(pos[r] * theta_k), the angle formed and
// reduced in fp64 (positions up to 1.3e5 keep full fp32 accuracy in cos/sin).
__device__ inline float2 rope_table_entry(const int32_t* pos, int half, const RopeFreq& f, int64_t i) {
  const int r = (int)(i / half), k = (int)(i % half);
  const double two_pi = 6.283185307179586476925286766559;
  double theta = exp(-(2.0 * k / (2.0 * half)) * log(f.base));
  if (f.scale > 1.0) {
    const double turns = f.orig_ctx * theta / two_pi;
    const double g = fmin(fmax((turns - f.alpha) / (f.beta - f.alpha), 0.0), 1.0);
    theta = g * theta + (1.0 - g) * (theta / f.scale);
  }
  double a = (double)pos[r] * theta;
  a = a - floor(a / two_pi) * two_pi;
  double sn, cs;
  sincos(a, &sn, &cs);
  return make_float2((float)cs, (float)sn);
}

// A RoPE table for n positions that a GEMM fills on the side (in extra workgroups of its first
// kernel) when its epilogue runs in a later split-K pass; otherwise gemm_run fills it first.
struct RopeJob {
  const int32_t* pos = nullptr;
  int n = 0, half = 0;
  RopeFreq f;
  float2* tab = nullptr;  // null: no job
};

// Where a GEMM result element (row, col) of batch z is stored, and what happens on the way.
//   address = z*batch_stride + rowbase(row) + (col/group)*group_stride + group_off + col%group
//   rowbase = row*ldc, or, when block_table is set, slot(row)*ldc with
//             slot = block_table[seq][row_pos[row]/block_size]*block_size
//                    + row_pos[row] % block_size    (paged cache rows),
//             seq = row_seq[row], or row itself when row_seq is null
//   columns >= rope_col0 are rotated as interleaved pairs in groups of d_hr by the angles
//   rope_tab[row][k] = (cos, sin) of pair k.
struct Epilogue {
  void* C = nullptr;
  bool c_f32 = false;  // C holds fp32 instead of the GEMM's element type
  int64_t ldc = 0, batch_stride = 0;
  int group = 1 << 30;
  int64_t group_stride = 0, group_off = 0;
  // the 4-column pieces of every 16 columns of a group are stored in the order 0, 2, 1, 3 (the
  // pipelined prefill attention's V^T rows: a lane's 8 keys of a 16-key step then lie together)
  bool perm16 = false;
  int rope_col0 = 1 << 30;
  int d_hr = 0;
  const float2* rope_tab = nullptr;
  const int32_t* row_seq = nullptr;
  const int32_t* row_pos = nullptr;
  const int32_t* block_table = nullptr;
  int max_blocks = 0, block_size = 1;
  float* C2 = nullptr;  // optional fp32 copy at the same indices
};

// C[z] (M x N) = A[z] (M x K) * op(B[z]),  op(B) = B^T with B [N][K] ("NT", weights in y = W x
// form) or B with B [K][N] ("NN").  For NT the rows of B may come from up to three matrices
// stacked along N: rows n < N0 from B0, N0 <= n < N1 from B1 (row n - N0), n >= N1 from B2
// (row n - N1).  Output columns col >= E0 go through epi2 as column col - E0 (two products that
// share the input A in one launch); E0 is even, so RoPE pairs never straddle it.
struct GemmParams {
  const void* A = nullptr;
  int64_t lda = 0, strideA = 0;
  const void* B0 = nullptr;
  const void* B1 = nullptr;
  const void* B2 = nullptr;
  int N0 = 1 << 30, N1 = 1 << 30;
  int64_t ldb = 0, strideB = 0;
  bool nn = false;
  int M = 0, N = 0, K = 0, batch = 1;
  Epilogue epi;
  Epilogue epi2;
  int E0 = 1 << 30;
  RopeJob side_rope;  // the table the epilogues read, filled before they run
};

struct GemmPlan {
  int cfg = 0;      // tile configuration id
  int bm = 0, bn = 0;
  int splits = 1;   // split-K factor
  int k_per_split = 0;
  size_t partial_bytes = 0;  // workspace for fp32 partials (0 when splits == 1)
};

// skinny_ok: the product is bf16, "NT" and 16-byte aligned, so rows M <= 64 may take the
// weight-streaming kernel and products with enough 256 x 256 tiles the large-tile kernel.
GemmPlan gemm_plan(int M, int N, int K, int batch, int cus, bool skinny_ok);
// W_UK absorption for bf16 (d_h == 128, d_c a multiple of 128):
// qhat[b*out_ld + h*out_hs + c] = sum_k qc[(b*n_h + h)*d_h + k] * w_uk[(h*d_h + k)*d_c + c].
bool absorb_ok(DType t, int d_h, int d_c);
struct QuantJob;
struct DecodeAttnParams;
// With qj (a decode step over the fp8 cache), the same launch also quantises the step's new entries
// (qj->n rows) in workgroups of its own, which saves the quantiser its launch.  With units (a decode
// attention's parameters with a balanced-units table, B <= 64), one workgroup of the launch builds
// that table, which saves the table builder its launch (the attention is then told units_ready).
hipError_t absorb_run(const void* qc, const void* w_uk, void* qhat, int B, int n_h, int d_h, int d_c,
                      int64_t out_ld, int64_t out_hs, hipStream_t s, const QuantJob* qj = nullptr,
                      const DecodeAttnParams* units = nullptr);
// o = W_UV per head for bf16 (d_c == 512, d_h a multiple of 64):
// o[(b*n_h + h)*d_h + d] = sum_c w_uv[(h*d_h + d)*512 + c] * ohat[(b*n_h + h)*512 + c]; o32 (may be
// null) receives the same values in fp32.
// With `parts` (split-KV decode's per-partition outputs, bf16 O_s / l_s, uv_parts_ok: d_h == 128)
// o_hat is not read: its rows are combined from the partitions by the log-sum-exp rule on the way.
struct UvPartials {
  const float* m = nullptr;  // [B][splits][n_h] partition max (log2 domain)
  const float* l = nullptr;  // [B][splits][n_h] partition normaliser
  const void* o = nullptr;   // [B][splits][n_h][512] bf16 O_s / l_s
  int splits = 0;
};
bool uv_ok(DType t, int d_h, int d_c);
bool uv_parts_ok(DType t, int d_h, int d_c);
// Workgroups of the W_UV kernel that combines the partitions itself, for B rows of n_h heads.
int uv_parts_workgroups(int B, int n_h);
hipError_t uv_run(const void* ohat, const void* w_uv, void* o, float* o32, int B, int n_h, int d_h,
                  hipStream_t s, const UvPartials* parts = nullptr);
// fp8 cache quantiser (latent_fp8.hip).  Destination of entry row r: dense row r of `codes` /
// `scales` when block_table is null, else the paged slot of (row_seq ? row_seq[r] : r, row_pos[r]).
struct QuantDst {
  uint8_t* codes = nullptr;  // [..][576] e4m3 codes
  float* scales = nullptr;   // [..][2] (s_c, s_r)
  const int32_t* block_table = nullptr;
  int max_blocks = 0, block_size = 1;
  const int32_t* row_seq = nullptr;
  const int32_t* row_pos = nullptr;
};
bool fp8_cache_ok(int d_c, int d_hr);
// n staged bf16 entries (rows src_ld elements apart) to quantise into dst, with the arguments of
// quantize_entries_run, for a launch that does it on the side (absorb_run).
struct QuantJob {
  void* src = nullptr;
  int64_t src_ld = 0;
  int n = 0;
  QuantDst dst;
  const void* gain = nullptr;
  float eps = 0.f;
  bool writeback = false;
};
// Quantises n bf16 entries (rows src_ld elements apart) into dst; with gain, their latent part is
// RMS-normalised first (and written back into src when writeback).
hipError_t quantize_entries_run(const void* src, int64_t src_ld, int n, const QuantDst& dst, hipStream_t s,
                                const void* gain = nullptr, float eps = 0.f, bool writeback = false);
// Largest partial_bytes of gemm_plan(m, ...) over 1 <= m <= M (workspace sized for M then also
// serves every smaller call).
size_t gemm_partial_bound(int M, int N, int K, int batch, int cus, bool skinny_ok);
// Launches the GEMM (and its split-K reduction).  `partial` must hold plan.partial_bytes.
hipError_t gemm_run(DType t, const GemmParams& p, const GemmPlan& plan, float* partial,
                    hipStream_t s);

// rope_tab[r][k] = (cos, sin)(pos[r] * theta_k), r < n; angles formed in fp64.
hipError_t rope_table(const int32_t* pos, int n, int d_hr, const RopeFreq& f, float2* tab, hipStream_t s);
// x[r][0..W) <- gain * x / sqrt(mean(x^2) + eps) for rows r < n, ld elements apart, in place
// (the RMSNorm of the compressed latents).
hipError_t rmsnorm_rows(DType t, void* x, int n, int W, int64_t ld, const void* gain, float eps, hipStream_t s);
// One launch for the latent norms of new tokens: entries[r] (r < n_e, E values, rows E apart) get
// their first d_c values normalised with g_ckv (if not null), in place, and are copied to their
// cache pages (slot of (seq[r] or r, pos[r])); cq[r] (r < n_q, d_cq values) is normalised in place
// with g_cq.
struct LatentFinish {
  void* entries = nullptr;
  int n_e = 0, E = 0, d_c = 0;
  const void* g_ckv = nullptr;
  void* pool = nullptr;
  const int32_t* block_table = nullptr;
  int max_blocks = 0, block_size = 1;
  const int32_t* seq = nullptr;
  const int32_t* pos = nullptr;
  void* cq = nullptr;
  int n_q = 0, d_cq = 0;
  const void* g_cq = nullptr;
  float eps = 1e-6f;
};
hipError_t latent_finish(DType t, const LatentFinish& f, hipStream_t s);
// seq[r] = r / T, pos[r] = r % T (+ start[seq[r]] when start != nullptr) for r < n.
hipError_t prefill_rows(int n, int T, int32_t* seq, int32_t* pos, hipStream_t s, const int32_t* start = nullptr);
// Dense key rows of a chunked prefill, out[b][j] for sequences b < S and j < Tk (entries of E
// values): the cached prefix j < start[b] from the pages (an fp8 pool, scales != nullptr, is
// dequantised, value(code) * s, to bf16), then the chunk's own rows fresh[b][0..T) as computed,
// then zeros.
hipError_t gather_entries(DType t, const void* pool, const float* scales, const int32_t* block_table, int max_blocks,
                          int block_size, const int32_t* start, const void* fresh, int T, int S, int Tk, int E, int d_c,
                          void* out, hipStream_t s);
// Copies dense rows src[r][0..width) into paged cache slots (row_seq/row_pos/block_table;
// row_seq == nullptr: row r belongs to sequence r).
hipError_t scatter_rows(DType t, const void* src, int n, int width, void* pool,
                        const int32_t* row_seq, const int32_t* row_pos, const int32_t* block_table,
                        int max_blocks, int block_size, hipStream_t s);

struct DecodeAttnParams {
  const void* q;          // [B][n_h][d_c + d_hr]
  const void* pool;       // [num_blocks][block_size][d_c + d_hr]
  const int32_t* block_table;
  int max_blocks, block_size;
  const int32_t* lens;    // [B] entries to attend over (or ctx_lens when lens_plus_one)
  bool lens_plus_one;
  int B, n_h, d_c, d_hr;
  float scale_log2;       // softmax scale * log2(e)
  int splits;
  int tokens_per_split;   // a multiple of 64
  float* part_m;          // [B][splits][n_h]   (log2 domain running max)
  float* part_l;          // [B][splits][n_h]
  void* part_o;           // [B][splits][n_h][d_c]: O_s / l_s (fp32, or bf16 for the tiled kernel)
  void* o_hat;            // [B][n_h][d_c] output (element type)
  float* lse;             // optional [B][n_h], natural log
  bool fp8 = false;       // pool holds e4m3 codes, with per-token (s_c, s_r) in scales
  const float* scales = nullptr;  // [num_blocks][block_size][2]
  bool leave_partials = false;    // write the partitions' (m, l, O_s / l_s) even with one partition,
                                  // and skip the combine (needs decode_bf16_partials); o_hat and
                                  // lse are not written
  int4* units = nullptr;          // set: balanced work units for the tiled kernels (scratch of
                                  // B * (splits + 1) entries, filled by decode_attention); null:
                                  // fixed partitions of tokens_per_split
  int cus = 256;                  // compute units, for the balanced units' finish time
  bool units_ready = false;       // the table is already built (by an earlier launch on the stream)
};

// true when the kernel decode_attention picks writes bf16 partition outputs
bool decode_bf16_partials(DType t, const DecodeAttnParams& p);

bool decode_supported(int d_c, int d_hr);
hipError_t decode_attention(DType t, const DecodeAttnParams& p, hipStream_t s);

// T queries per sequence at positions q_off[s] .. q_off[s] + T - 1 (q_off == nullptr: 0), each
// attending to keys 0 .. its position; a sequence's keys sit in a slot of Tk >= max q_off + T rows,
// of which the first q_off[s] + T are valid.  Every operand is the plain output of a projection:
// queries and keys token-major, the rope half of the query not yet rotated (the kernels rotate it
// with the position table as they load it), values token-contiguous.
struct PrefillAttnParams {
  const void* qc;     // [S*T][n_h*d_h]           q^C
  const float* qr;    // [S*T][n_h*d_hr] fp32     q^R, un-rotated
  const float2* rope; // [S*T][d_hr/2]            (cos, sin) of each query row's position
  const void* k;      // [S*Tk][k_ld]             k^C: head h at columns h*d_h
  int64_t k_ld;
  const void* kr;     // [S*Tk] rows of ld_kr elements; k^R at column kr_off
  int64_t ld_kr;
  int kr_off;
  const void* vt;     // [n_h][d_h][S][Tkp]       (W_UV_i c^KV, token-contiguous; Tkp = Tk rounded up to 64;
                      //  for the pipelined kernel with the key pieces of Epilogue::perm16)
  void* o;            // [S*T][n_h][d_h]
  float* o_f32;       // optional fp32 copy
  int S, T, n_h, d_h, d_hr;
  int Tk = 0;                     // 0: T
  const int32_t* q_off = nullptr;
  float scale_log2;
};
bool prefill_supported(int d_h, int d_hr);
// Whether prefill_attention takes the pipelined kernel for these sizes (its V^T rows then carry the
// key order of Epilogue::perm16).
bool prefill_pipelined(DType t, int d_h, int d_hr, int64_t S, int64_t Tk, int64_t ld_kr, int64_t k_ld);
hipError_t prefill_attention(DType t, const PrefillAttnParams& p, hipStream_t s);

}  // namespace mla
