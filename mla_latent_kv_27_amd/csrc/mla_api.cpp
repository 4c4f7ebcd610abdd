// C ABI of libmla: argument validation, workspace carving and the launch sequence of each
// entry point.  The operations are those of App. C ("Full Formulas of MLA") on the DeepSeek-V2
// summary page; see include/mla.h for the contract of every call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <vector>

#include "mla.h"
#include "internal.h"

using namespace mla;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Bump allocator over the caller's workspace (or a null base, for sizing).
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(reinterpret_cast<char*>(b)) {}
  template <typename P>
  P* take(size_t bytes) {
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += align_up(bytes);
    return p;
  }
};

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

int validate_dims(const mla_dims* d) {
  if (!d) return MLA_ERR_INVALID_ARG;
  if (d->d_model <= 0 || d->n_h <= 0 || d->d_h <= 0 || d->d_c <= 0 || d->d_hr <= 0 || d->d_cq < 0)
    return MLA_ERR_INVALID_ARG;
  if (d->d_hr % 2 != 0) return MLA_ERR_INVALID_ARG;
  if (d->dtype != MLA_F32 && d->dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (!(d->softmax_scale >= 0.f) || !std::isfinite(d->softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (!(d->rope_base > 0.f) || !std::isfinite(d->rope_base)) return MLA_ERR_INVALID_ARG;
  if (!(d->rope_scale >= 0.f) || !std::isfinite(d->rope_scale)) return MLA_ERR_INVALID_ARG;
  if (!(d->rms_eps >= 0.f) || !std::isfinite(d->rms_eps)) return MLA_ERR_INVALID_ARG;
  if (d->rope_scale > 1.f) {
    if (d->rope_orig_ctx <= 0 || !(d->yarn_alpha >= 0.f) || !std::isfinite(d->yarn_beta) ||
        !(d->yarn_beta > d->yarn_alpha) || !(d->yarn_mscale >= 0.f) || !std::isfinite(d->yarn_mscale))
      return MLA_ERR_INVALID_ARG;
  }
  // every contraction and row is moved in 16-byte chunks
  const int epc = d->dtype == MLA_BF16 ? 8 : 4;
  if (d->d_model % epc || d->d_h % epc || d->d_c % epc || d->d_cq % epc || d->d_hr % 8)
    return MLA_ERR_UNSUPPORTED;
  if (d->cache_dtype != 0 && d->cache_dtype != d->dtype) {
    if (d->cache_dtype != MLA_FP8_E4M3 || d->dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
    if (!fp8_cache_ok(d->d_c, d->d_hr)) return MLA_ERR_UNSUPPORTED;
  }
  return MLA_OK;
}

bool fp8_cache(const mla_dims* d) { return d->cache_dtype == MLA_FP8_E4M3; }

inline DType dt(const mla_dims* d) { return d->dtype == MLA_BF16 ? DType::BF16 : DType::F32; }
inline int q_in(const mla_dims* d) { return d->d_cq > 0 ? d->d_cq : d->d_model; }
inline int entry(const mla_dims* d) { return d->d_c + d->d_hr; }
// bf16 "NT" products may take the weight-streaming kernel for small row counts
inline bool sk(const mla_dims* d) { return d->dtype == MLA_BF16; }
inline bool yarn_on(const mla_dims* d) { return d->rope_scale > 1.f; }
inline float eps_of(const mla_dims* d) { return d->rms_eps > 0.f ? d->rms_eps : 1e-6f; }
// The gain of the c^q norm exists only with query compression.
inline bool weights_norm_ok(const mla_dims* d, const mla_weights* w) { return !w->g_cq || d->d_cq > 0; }
// The logit scale: the layer's own, else 1/sqrt(d_h + d_hr) times YaRN's t = (c ln s + 1)^2.
inline float scale_of(const mla_dims* d) {
  if (d->softmax_scale > 0.f) return d->softmax_scale;
  double sc = 1.0 / std::sqrt((double)(d->d_h + d->d_hr));
  if (yarn_on(d)) {
    const double root_t = (double)d->yarn_mscale * std::log((double)d->rope_scale) + 1.0;
    sc *= root_t * root_t;
  }
  return (float)sc;
}
inline RopeFreq freq_of(const mla_dims* d) {
  RopeFreq f;
  f.base = d->rope_base;
  if (yarn_on(d)) {
    f.scale = d->rope_scale;
    f.orig_ctx = d->rope_orig_ctx;
    f.alpha = d->yarn_alpha;
    f.beta = d->yarn_beta;
  }
  return f;
}

int validate_cache(const mla_dims* d, const mla_paged_cache* c) {
  if (!c || !c->pool || !c->block_table) return MLA_ERR_INVALID_ARG;
  if (c->num_blocks <= 0 || c->block_size <= 0 || c->max_blocks_per_seq <= 0) return MLA_ERR_INVALID_ARG;
  if (fp8_cache(d) && !c->scales) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

// ----------------------------------------------------------------------------- debug builds
// Built with -DMLA_DEBUG (build.py --variant debug), the library also checks the preconditions
// that a release build leaves to the caller, because checking them means reading device memory
// on the host: every context length inside its bound and its block table row, and every block id
// that a sequence's tokens use inside the pool.  The tables are copied to the host (synchronously)
// before anything is launched; a violation prints what it found and returns MLA_ERR_INVALID_ARG.
// Every launch group is followed by a device synchronisation, so that a kernel that fails is
// reported (MLA_ERR_HIP) by the call that launched it.
#ifdef MLA_DEBUG
constexpr bool kDebug = true;
#else
constexpr bool kDebug = false;
#endif

// Sequence b (of batch) uses tokens 0 .. len_b - 1, len_b = (lens ? lens[b] : 0) + extra
// (+ start[b] for a chunk); lens (device, may be null) each in [0, max_len].
[[maybe_unused]] int debug_check_tokens(const mla_paged_cache* c, const int32_t* lens, int batch, int extra, int max_len,
                       const int32_t* start = nullptr) {
  std::vector<int32_t> len(batch, 0), st(batch, 0), row(c->max_blocks_per_seq);
  if (lens && hipMemcpy(len.data(), lens, sizeof(int32_t) * batch, hipMemcpyDeviceToHost) != hipSuccess)
    return MLA_ERR_HIP;
  if (start && hipMemcpy(st.data(), start, sizeof(int32_t) * batch, hipMemcpyDeviceToHost) != hipSuccess)
    return MLA_ERR_HIP;
  for (int b = 0; b < batch; ++b) {
    if (len[b] < 0 || (lens && len[b] > max_len) || st[b] < 0) {
      std::fprintf(stderr, "mla debug: sequence %d: length %d (bound %d), start %d\n", b, len[b], max_len, st[b]);
      return MLA_ERR_INVALID_ARG;
    }
    const int64_t tokens = (int64_t)st[b] + len[b] + extra;
    const int64_t blocks = (tokens + c->block_size - 1) / c->block_size;
    if (blocks > c->max_blocks_per_seq) {
      std::fprintf(stderr, "mla debug: sequence %d: %lld tokens need %lld blocks, the table row has %d\n", b,
                   (long long)tokens, (long long)blocks, c->max_blocks_per_seq);
      return MLA_ERR_INVALID_ARG;
    }
    if (blocks == 0) continue;
    if (hipMemcpy(row.data(), c->block_table + (int64_t)b * c->max_blocks_per_seq, sizeof(int32_t) * blocks,
                  hipMemcpyDeviceToHost) != hipSuccess)
      return MLA_ERR_HIP;
    for (int64_t k = 0; k < blocks; ++k)
      if (row[k] < 0 || row[k] >= c->num_blocks) {
        std::fprintf(stderr, "mla debug: sequence %d: logical block %lld maps to block %d of %d\n", b, (long long)k,
                     row[k], c->num_blocks);
        return MLA_ERR_INVALID_ARG;
      }
  }
  return MLA_OK;
}

// Appended token i goes to position pos[i] of sequence seq_idx[i] (both device).
[[maybe_unused]] int debug_check_slots(const mla_paged_cache* c, const int32_t* seq_idx, const int32_t* pos, int n) {
  std::vector<int32_t> sq(n), ps(n);
  if (hipMemcpy(sq.data(), seq_idx, sizeof(int32_t) * n, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(ps.data(), pos, sizeof(int32_t) * n, hipMemcpyDeviceToHost) != hipSuccess)
    return MLA_ERR_HIP;
  for (int i = 0; i < n; ++i) {
    if (sq[i] < 0 || ps[i] < 0 || ps[i] / c->block_size >= c->max_blocks_per_seq) {
      std::fprintf(stderr, "mla debug: token %d: sequence %d position %d outside the table\n", i, sq[i], ps[i]);
      return MLA_ERR_INVALID_ARG;
    }
    int32_t blk = 0;
    if (hipMemcpy(&blk, c->block_table + (int64_t)sq[i] * c->max_blocks_per_seq + ps[i] / c->block_size,
                  sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
      return MLA_ERR_HIP;
    if (blk < 0 || blk >= c->num_blocks) {
      std::fprintf(stderr, "mla debug: token %d: position %d of sequence %d maps to block %d of %d\n", i, ps[i],
                   sq[i], blk, c->num_blocks);
      return MLA_ERR_INVALID_ARG;
    }
  }
  return MLA_OK;
}

// KV partitions are whole multiples of 64 tokens (a common multiple of every decode kernel's
// tile), so the partition count, and with it the workspace, does not depend on which kernel
// runs.
constexpr int kSplitQuantum = 64;

int auto_splits(const mla_dims* d, int batch, int max_ctx_len, int cus) {
  const int hg = (d->n_h + 127) / 128;  // workgroups per (sequence, partition)
  const int chunks = (max_ctx_len + 1 + kSplitQuantum - 1) / kSplitQuantum;
  const int units = batch * hg;
  int s = (cus + units - 1) / units;
  s = std::min(s, std::max(1, chunks / 4));  // at least 256 tokens per partition
  return std::max(1, std::min(s, 64));
}

// Small batches (fewer than 16 workgroups per partition slot) take the balanced work units of
// the tiled kernels, with twice the automatic slots so that long sequences can spread over more
// compute units than short ones.
bool balanced_units(const mla_dims* d, int batch) { return batch * ((d->n_h + 127) / 128) < 16; }
int auto_request(const mla_dims* d, int batch, int max_ctx_len, int cus) {
  const int s = auto_splits(d, batch, max_ctx_len, cus);
  return balanced_units(d, batch) ? std::min(128, 2 * s) : s;
}

// ----------------------------------------------------------------------------- workspace plans
struct AppendWs {
  float2* rope;
  float* partial;
  void* staged;  // entries before their latent norm and/or quantisation [n][entry]
  GemmPlan plan;
};
AppendWs carve_append(Carve& cv, const mla_dims* d, int n, int cus) {
  AppendWs w;
  w.plan = gemm_plan(n, entry(d), d->d_model, 1, cus, sk(d));
  w.rope = cv.take<float2>((size_t)n * (d->d_hr / 2) * sizeof(float2));
  w.partial = cv.take<float>(gemm_partial_bound(n, entry(d), d->d_model, 1, cus, sk(d)));
  // the workspace size does not know whether the weights carry a c^KV norm: always room to stage
  w.staged = cv.take<char>((size_t)n * entry(d) * dsize(dt(d)));
  return w;
}

// Decode products; those sharing an input run as one launch with stacked weights:
//   kvq = h [W_DQ; W_DKV; W_KR]   (c^q and the new cache entry; W_DKV; W_KR alone when d_cq == 0)
//   q   = q_in [W_UQ; W_QR]       (q^C and the rotated q^R)
struct DecodeGemms {
  GemmPlan kvq, q, absorb, uv, out;
};
inline int kvq_cols(const mla_dims* d) { return d->d_cq + entry(d); }
inline int q_cols(const mla_dims* d) { return d->n_h * (d->d_h + d->d_hr); }
// partial workspace serving every batch <= B
size_t decode_partial_bound(const mla_dims* d, int B, int cus) {
  return std::max({gemm_partial_bound(B, kvq_cols(d), d->d_model, 1, cus, sk(d)),
                   gemm_partial_bound(B, q_cols(d), q_in(d), 1, cus, sk(d)),
                   gemm_partial_bound(B, d->d_c, d->d_h, d->n_h, cus, false),
                   gemm_partial_bound(B, d->d_h, d->d_c, d->n_h, cus, sk(d)),
                   gemm_partial_bound(B, d->d_model, d->n_h * d->d_h, 1, cus, sk(d))});
}
DecodeGemms decode_gemms(const mla_dims* d, int B, int cus) {
  DecodeGemms g;
  g.kvq = gemm_plan(B, kvq_cols(d), d->d_model, 1, cus, sk(d));
  g.q = gemm_plan(B, q_cols(d), q_in(d), 1, cus, sk(d));
  g.absorb = gemm_plan(B, d->d_c, d->d_h, d->n_h, cus, false);
  g.uv = gemm_plan(B, d->d_h, d->d_c, d->n_h, cus, sk(d));
  g.out = gemm_plan(B, d->d_model, d->n_h * d->d_h, 1, cus, sk(d));
  return g;
}

struct AttnWs {
  float *pm, *pl, *po;
  int4* units;    // the tiled kernels' work-unit table
  bool balanced;  // automatic splits for a small batch: use the table
  int splits, tps;
};
// Partition count for a request of `splits`; *tps = tokens per partition.
int split_count(int max_kv_len, int splits, int* tps) {
  const int chunks = (max_kv_len + kSplitQuantum - 1) / kSplitQuantum;
  const int per = std::max(1, (chunks + splits - 1) / splits);
  *tps = per * kSplitQuantum;
  return std::max(1, (chunks + per - 1) / per);
}
// Partial rows serving every batch <= B and context <= max_kv_len.  split_count never exceeds
// the requested count, and the automatic count grows with the context, so the request at
// max_kv_len bounds every smaller call.  splits_raw == 0: automatic choice.
size_t attn_rows_bound(const mla_dims* d, int B, int max_kv_len, int splits_raw, int cus) {
  size_t best = 0;
  for (int b = 1; b <= B; ++b) {
    const int req = splits_raw > 0 ? splits_raw : auto_request(d, b, max_kv_len - 1, cus);
    if (req > 1) best = std::max(best, (size_t)b * req * d->n_h);
  }
  return best;
}
AttnWs carve_attn(Carve& cv, const mla_dims* d, int B, int max_kv_len, int splits_raw, int cus) {
  AttnWs a;
  const int req = splits_raw > 0 ? splits_raw : auto_request(d, B, max_kv_len - 1, cus);
  a.splits = split_count(max_kv_len, req, &a.tps);
  a.balanced = splits_raw == 0 && balanced_units(d, B);
  const size_t n = attn_rows_bound(d, B, max_kv_len, splits_raw, cus);
  a.pm = cv.take<float>(n * sizeof(float));
  a.pl = cv.take<float>(n * sizeof(float));
  a.po = cv.take<float>(n * d->d_c * sizeof(float));
  // B * (splits + 1) entries: n bounds b * splits * n_h over every call when splits > 1
  a.units = cv.take<int4>((std::max<size_t>(n / std::max(1, d->n_h), B) + B) * sizeof(int4));
  return a;
}

struct DecodeWs {
  float2* rope;
  void *cq, *qc, *qcat, *ohat, *o;
  void* staged;  // the new tokens' entries before their latent norm and/or quantisation
  AttnWs attn;
  float* partial;
  DecodeGemms gm;
};
// splits: the caller's num_splits (0 = automatic)
DecodeWs carve_decode(Carve& cv, const mla_dims* d, int B, int max_ctx_len, int splits, int cus) {
  DecodeWs w;
  const size_t es = dsize(dt(d));
  w.gm = decode_gemms(d, B, cus);
  w.rope = cv.take<float2>((size_t)B * (d->d_hr / 2) * sizeof(float2));
  w.cq = cv.take<char>((size_t)B * d->d_cq * es);
  w.qc = cv.take<char>((size_t)B * d->n_h * d->d_h * es);
  w.qcat = cv.take<char>((size_t)B * d->n_h * entry(d) * es);
  w.staged = cv.take<char>((size_t)B * entry(d) * es);
  w.ohat = cv.take<char>((size_t)B * d->n_h * d->d_c * es);
  w.o = cv.take<char>((size_t)B * d->n_h * d->d_h * es);
  w.attn = carve_attn(cv, d, B, max_ctx_len + 1, splits, cus);
  w.partial = cv.take<float>(decode_partial_bound(d, B, cus));
  return w;
}

struct PrefillWs {
  int32_t *seq, *pos;
  float2* rope;
  void *cq, *qc, *kvd, *kva, *kp, *vt, *o;  // kva: chunked prefill's gathered keys (else kvd)
  float* qr;                               // [M][n_h*d_hr] un-rotated q^R, fp32
  float* partial;
  GemmPlan kvq_p, q_p, kv_p, k_p, v_p, out_p;  // kvq_p: [W_DQ; W_DKV; W_KR] (d_cq > 0), else kv_p
  int Tk, Tp;  // key rows per sequence (T, or max_start + T when chunked), rounded up to 64
};
// Every intermediate is the plain output of one product: q^C and q^R token-major (q^R in fp32,
// rotated by the attention kernel as it loads it), k^C token-major, v^T token-contiguous.
// chunked: keys are the cached prefix plus the new rows, max_start + T per sequence
PrefillWs carve_prefill(Carve& cv, const mla_dims* d, int S, int T, int cus, bool chunked = false,
                        int max_start = 0) {
  PrefillWs w;
  const size_t es = dsize(dt(d));
  const int M = S * T;
  w.Tk = chunked ? max_start + T : T;
  const int Mk = S * w.Tk;
  w.Tp = (w.Tk + 63) / 64 * 64;
  const int qw = d->n_h * (d->d_h + d->d_hr);
  w.kvq_p = d->d_cq > 0 ? gemm_plan(M, d->d_cq + entry(d), d->d_model, 1, cus, sk(d)) : GemmPlan{};
  w.q_p = gemm_plan(M, qw, q_in(d), 1, cus, sk(d));
  w.kv_p = d->d_cq > 0 ? GemmPlan{} : gemm_plan(M, entry(d), d->d_model, 1, cus, sk(d));
  w.k_p = gemm_plan(Mk, d->n_h * d->d_h, d->d_c, 1, cus, sk(d));
  w.v_p = gemm_plan(d->n_h * d->d_h, Mk, d->d_c, 1, cus, sk(d));
  w.out_p = gemm_plan(M, d->d_model, d->n_h * d->d_h, 1, cus, sk(d));
  w.seq = cv.take<int32_t>((size_t)M * 4);
  w.pos = cv.take<int32_t>((size_t)M * 4);
  w.rope = cv.take<float2>((size_t)M * (d->d_hr / 2) * sizeof(float2));
  w.cq = cv.take<char>((size_t)M * d->d_cq * es);
  w.qc = cv.take<char>((size_t)M * d->n_h * d->d_h * es);
  w.qr = cv.take<float>((size_t)M * d->n_h * d->d_hr * sizeof(float));
  w.kvd = cv.take<char>((size_t)M * entry(d) * es);
  w.kva = chunked ? cv.take<char>((size_t)Mk * entry(d) * es) : w.kvd;
  w.kp = cv.take<char>((size_t)Mk * d->n_h * d->d_h * es);
  w.vt = cv.take<char>((size_t)d->n_h * d->d_h * S * w.Tp * es);
  w.o = cv.take<char>((size_t)M * d->n_h * d->d_h * es);
  size_t mp = std::max({gemm_partial_bound(M, qw, q_in(d), 1, cus, sk(d)),
                        gemm_partial_bound(M, entry(d), d->d_model, 1, cus, sk(d)),
                        gemm_partial_bound(Mk, d->n_h * d->d_h, d->d_c, 1, cus, sk(d)),
                        gemm_partial_bound(d->n_h * d->d_h, Mk, d->d_c, 1, cus, sk(d)),
                        gemm_partial_bound(M, d->d_model, d->n_h * d->d_h, 1, cus, sk(d))});
  if (d->d_cq > 0) mp = std::max(mp, gemm_partial_bound(M, d->d_cq + entry(d), d->d_model, 1, cus, sk(d)));
  w.partial = cv.take<float>(mp);
  return w;
}

#define MLA_HIP(x)                                                                      \
  do {                                                                                  \
    if ((x) != hipSuccess) return MLA_ERR_HIP;                                          \
    if (kDebug && (hipDeviceSynchronize() != hipSuccess || hipGetLastError() != hipSuccess)) \
      return MLA_ERR_HIP;                                                               \
  } while (0)

// Plain row-major output epilogue.
Epilogue dense(void* C, int64_t ldc) {
  Epilogue e;
  e.C = C;
  e.ldc = ldc;
  return e;
}

// Stores rows of [c^KV | k^R] into their paged cache slots, rotating the k^R columns.
Epilogue cache_epilogue(const mla_dims* d, const mla_paged_cache* c, const float2* rope, const int32_t* seq,
                        const int32_t* pos) {
  Epilogue e;
  e.C = c->pool;
  e.ldc = entry(d);
  e.rope_col0 = d->d_c;
  e.d_hr = d->d_hr;
  e.rope_tab = rope;
  e.row_seq = seq;
  e.row_pos = pos;
  e.block_table = c->block_table;
  e.max_blocks = c->max_blocks_per_seq;
  e.block_size = c->block_size;
  return e;
}

// Dense rows [c^KV | RoPE'd k^R] for the latent norm and/or the fp8 quantiser.
Epilogue staged_epilogue(const mla_dims* d, void* staged, const float2* rope) {
  Epilogue e;
  e.C = staged;
  e.ldc = entry(d);
  e.rope_col0 = d->d_c;
  e.d_hr = d->d_hr;
  e.rope_tab = rope;
  return e;
}
QuantDst quant_dst(const mla_paged_cache* c, const int32_t* seq, const int32_t* pos) {
  QuantDst q;
  q.codes = reinterpret_cast<uint8_t*>(c->pool);
  q.scales = c->scales;
  q.block_table = c->block_table;
  q.max_blocks = c->max_blocks_per_seq;
  q.block_size = c->block_size;
  q.row_seq = seq;
  q.row_pos = pos;
  return q;
}

// Entries are staged (dense rows) when they need a pass after the projection: the c^KV norm and/or
// the fp8 quantiser.
inline bool staged_entries(const mla_dims* d, const mla_weights* w) { return fp8_cache(d) || w->g_ckv; }

// Staged rows -> their cache slots (seq == nullptr: row r belongs to sequence r): the c^KV norm
// in place, then quantised (fp8) or copied into the pages.  cq (n_q rows), when given, gets the
// c^q norm in the same launch on the bf16/fp32 path.
// quant_later: the fp8 quantisation is left to a later launch (the decode step's W_UK absorption).
int finish_entries(const mla_dims* d, const mla_weights* w, const mla_paged_cache* c, void* staged, int n,
                   const int32_t* seq, const int32_t* pos, hipStream_t s, void* cq = nullptr, int n_q = 0,
                   bool quant_later = false) {
  const bool q_norm = cq && w->g_cq;
  if (fp8_cache(d)) {
    if (!quant_later)
      MLA_HIP(quantize_entries_run(staged, entry(d), n, quant_dst(c, seq, pos), s, w->g_ckv, eps_of(d), true));
    if (q_norm) MLA_HIP(rmsnorm_rows(dt(d), cq, n_q, d->d_cq, d->d_cq, w->g_cq, eps_of(d), s));
    return MLA_OK;
  }
  if (!w->g_ckv && !q_norm) {
    MLA_HIP(scatter_rows(dt(d), staged, n, entry(d), c->pool, seq, pos, c->block_table, c->max_blocks_per_seq,
                         c->block_size, s));
    return MLA_OK;
  }
  LatentFinish f;
  f.entries = staged; f.n_e = n; f.E = entry(d); f.d_c = d->d_c; f.g_ckv = w->g_ckv;
  f.pool = c->pool; f.block_table = c->block_table; f.max_blocks = c->max_blocks_per_seq;
  f.block_size = c->block_size; f.seq = seq; f.pos = pos;
  if (q_norm) { f.cq = cq; f.n_q = n_q; f.d_cq = d->d_cq; f.g_cq = w->g_cq; }
  f.eps = eps_of(d);
  MLA_HIP(latent_finish(dt(d), f, s));
  return MLA_OK;
}

int run_cache_writer(const mla_dims* d, const mla_weights* w, const mla_paged_cache* c, const void* h, int n,
                     const int32_t* seq, const int32_t* pos, const float2* rope, const GemmPlan& plan,
                     float* partial, void* staged, hipStream_t s) {
  GemmParams g;
  g.A = h;
  g.lda = d->d_model;
  g.B0 = w->W_DKV;
  g.B1 = w->W_KR;
  g.N0 = d->d_c;
  g.ldb = d->d_model;
  g.M = n;
  g.N = entry(d);
  g.K = d->d_model;
  if (staged_entries(d, w)) {  // entries to the staging rows, then normalised / quantised into their slots
    g.epi = staged_epilogue(d, staged, rope);
    MLA_HIP(gemm_run(dt(d), g, plan, partial, s));
    return finish_entries(d, w, c, staged, n, seq, pos, s);
  }
  g.epi = cache_epilogue(d, c, rope, seq, pos);
  MLA_HIP(gemm_run(dt(d), g, plan, partial, s));
  return MLA_OK;
}

// mla_prefill (start == nullptr) and mla_prefill_chunk (the new rows start at start[b]; the keys
// are the cached prefix gathered back from the pages plus the new rows).
int prefill_impl(const mla_dims* d, const mla_weights* w, const mla_paged_cache* c, const void* h, int32_t batch,
                 int32_t T, const int32_t* start, int32_t max_start, void* u, float* o_heads, void* workspace,
                 size_t ws_bytes, void* stream) {
  int st = validate_dims(d);
  if (st != MLA_OK) return st;
  if ((st = validate_cache(d, c)) != MLA_OK) return st;
  if (!w || !w->W_UQ || !w->W_QR || !w->W_DKV || !w->W_KR || !w->W_UK || !w->W_UV || !w->W_O)
    return MLA_ERR_INVALID_ARG;
  if ((d->d_cq > 0) != (w->W_DQ != nullptr) || !weights_norm_ok(d, w)) return MLA_ERR_INVALID_ARG;
  if (!h || !u || batch <= 0 || T <= 0) return MLA_ERR_INVALID_ARG;
  const bool chunked = start != nullptr;
  if ((int64_t)max_start + T > (int64_t)c->max_blocks_per_seq * c->block_size) return MLA_ERR_INVALID_ARG;
  if ((int64_t)batch * (max_start + T) > (1LL << 30)) return MLA_ERR_UNSUPPORTED;
  if (!prefill_supported(d->d_h, d->d_hr)) return MLA_ERR_UNSUPPORTED;
  const int cus = device_cus();
  Carve sz(nullptr);
  carve_prefill(sz, d, batch, T, cus, chunked, max_start);
  if (!workspace || ws_bytes < sz.off) return MLA_ERR_WORKSPACE;
  if (kDebug && (st = debug_check_tokens(c, nullptr, batch, T, 0, start)) != MLA_OK) return st;
  Carve cv(workspace);
  PrefillWs ws = carve_prefill(cv, d, batch, T, cus, chunked, max_start);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const DType t = dt(d);
  const int M = batch * T, E = entry(d), qw = q_in(d), QD = d->d_h + d->d_hr;
  const int Mk = batch * ws.Tk;  // key rows

  MLA_HIP(prefill_rows(M, T, ws.seq, ws.pos, s, start));
  MLA_HIP(rope_table(ws.pos, M, d->d_hr, freq_of(d), ws.rope, s));
  const void* qin = h;
  // dense [c^KV | RoPE(k^R)] rows (then normalised and copied into the paged cache), and c^q
  // when the query is compressed: one product [W_DQ; W_DKV; W_KR] h
  Epilogue kv_epi = dense(ws.kvd, E);
  kv_epi.rope_col0 = d->d_c; kv_epi.d_hr = d->d_hr; kv_epi.rope_tab = ws.rope;
  if (d->d_cq > 0) {
    GemmParams g;
    g.A = h; g.lda = d->d_model; g.ldb = d->d_model;
    g.B0 = w->W_DQ; g.N0 = d->d_cq; g.B1 = w->W_DKV; g.N1 = d->d_cq + d->d_c; g.B2 = w->W_KR;
    g.M = M; g.N = d->d_cq + E; g.K = d->d_model;
    g.epi = dense(ws.cq, d->d_cq);
    g.E0 = d->d_cq;
    g.epi2 = kv_epi;
    MLA_HIP(gemm_run(t, g, ws.kvq_p, ws.partial, s));
    if (w->g_cq) MLA_HIP(rmsnorm_rows(t, ws.cq, M, d->d_cq, d->d_cq, w->g_cq, eps_of(d), s));
    qin = ws.cq;
  } else {
    GemmParams g;
    g.A = h; g.lda = d->d_model; g.B0 = w->W_DKV; g.B1 = w->W_KR; g.N0 = d->d_c; g.ldb = d->d_model;
    g.M = M; g.N = E; g.K = d->d_model;
    g.epi = kv_epi;
    MLA_HIP(gemm_run(t, g, ws.kv_p, ws.partial, s));
  }
  {  // [q^C | q^R] = [W_UQ; W_QR] c^q in one launch: q^C token-major in the layer's type, q^R
     // token-major in fp32 and not yet rotated (the attention kernel rotates it as it loads it)
    GemmParams g;
    g.A = qin; g.lda = qw; g.ldb = qw;
    g.B0 = w->W_UQ; g.N0 = d->n_h * d->d_h; g.B1 = w->W_QR;
    g.M = M; g.N = d->n_h * QD; g.K = qw;
    g.epi = dense(ws.qc, (int64_t)d->n_h * d->d_h);
    g.E0 = d->n_h * d->d_h;
    g.epi2 = dense(ws.qr, (int64_t)d->n_h * d->d_hr);
    g.epi2.c_f32 = true;
    MLA_HIP(gemm_run(t, g, ws.q_p, ws.partial, s));
  }
  {
    {  // c^KV norm in place (the K/V products below read it), then into the pages
      const int rc = finish_entries(d, w, c, ws.kvd, M, ws.seq, ws.pos, s);
      if (rc != MLA_OK) return rc;
    }
    if (chunked)  // key rows: the cached prefix read back from the pages, then the chunk's rows
      MLA_HIP(gather_entries(t, c->pool, fp8_cache(d) ? c->scales : nullptr, c->block_table, c->max_blocks_per_seq,
                             c->block_size, start, ws.kvd, T, batch, ws.Tk, E, d->d_c, ws.kva, s));
  }
  {  // k^C = [W_UK_1; ...; W_UK_n_h] c^KV, token-major [Mk][n_h*d_h]
    GemmParams g;
    g.A = ws.kva; g.lda = E; g.B0 = w->W_UK; g.ldb = d->d_c;
    g.M = Mk; g.N = d->n_h * d->d_h; g.K = d->d_c;
    g.epi = dense(ws.kp, (int64_t)d->n_h * d->d_h);
    MLA_HIP(gemm_run(t, g, ws.k_p, ws.partial, s));
  }
  {  // v^T: rows (head, dim) of W_UV times c^KV^T, token-contiguous [n_h][d_h][S][Tp]
    GemmParams g;
    g.A = w->W_UV; g.lda = d->d_c; g.B0 = ws.kva; g.ldb = E;
    g.M = d->n_h * d->d_h; g.N = Mk; g.K = d->d_c;
    g.epi = dense(ws.vt, (int64_t)batch * ws.Tp);
    g.epi.group = ws.Tk; g.epi.group_stride = ws.Tp;
    g.epi.perm16 = prefill_pipelined(t, d->d_h, d->d_hr, batch, ws.Tk, E, (int64_t)d->n_h * d->d_h);
    MLA_HIP(gemm_run(t, g, ws.v_p, ws.partial, s));
  }
  {
    PrefillAttnParams a{};
    a.qc = ws.qc; a.qr = ws.qr; a.rope = ws.rope;
    a.k = ws.kp; a.k_ld = (int64_t)d->n_h * d->d_h;
    a.kr = ws.kva; a.ld_kr = E; a.kr_off = d->d_c; a.vt = ws.vt;
    a.o = ws.o; a.o_f32 = o_heads;
    a.S = batch; a.T = T; a.n_h = d->n_h; a.d_h = d->d_h; a.d_hr = d->d_hr;
    a.Tk = ws.Tk; a.q_off = start;
    a.scale_log2 = scale_of(d) * 1.4426950408889634f;
    MLA_HIP(prefill_attention(t, a, s));
  }
  {  // u = W_O [o_1; ...; o_n_h]
    const int64_t K = (int64_t)d->n_h * d->d_h;
    GemmParams g;
    g.A = ws.o; g.lda = K; g.B0 = w->W_O; g.ldb = K;
    g.M = M; g.N = d->d_model; g.K = (int)K;
    g.epi = dense(u, d->d_model);
    MLA_HIP(gemm_run(t, g, ws.out_p, ws.partial, s));
  }
  return MLA_OK;
}

// ----------------------------------------------------------------------------- allocation-free decode
// mla_decode_noalloc's scratch: one array per device, reserved when the code object loads there and
// held until the process ends.  In host code `scratch` only names the symbol; its device address is
// looked up once per device (with that device current) and used everywhere after that.
constexpr size_t kNoAllocBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MLA_ERR_HIP;
  if (dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

int decode_impl(const mla_dims* d, const mla_weights* w, const mla_paged_cache* c, const void* h, int32_t batch,
                const int32_t* ctx_lens, int32_t max_ctx_len, int32_t num_splits, void* u, float* o_heads,
                void* workspace, size_t ws_bytes, void* stream);

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: null pointer, non-positive or inconsistent size";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: sizes the library has no kernel for";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP call or kernel launch failed";
    default: return "unknown mla_status";
  }
}

int32_t mla_decode_auto_splits(const mla_dims* d, int32_t batch, int32_t max_ctx_len) {
  if (validate_dims(d) != MLA_OK || batch <= 0 || max_ctx_len < 0) return -1;
  return auto_splits(d, batch, max_ctx_len, device_cus());
}

int mla_workspace_size(const mla_dims* d, int op, int32_t batch, int32_t max_tokens, int32_t max_ctx_len,
                       int32_t num_splits, size_t* bytes) {
  int st = validate_dims(d);
  if (st != MLA_OK) return st;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  const int cus = device_cus();
  Carve cv(nullptr);
  switch (op) {
    case MLA_OP_CACHE_APPEND:
      if (max_tokens < 0) return MLA_ERR_INVALID_ARG;
      carve_append(cv, d, max_tokens, cus);
      break;
    case MLA_OP_PREFILL:
      if (batch <= 0 || max_tokens <= 0) return MLA_ERR_INVALID_ARG;
      carve_prefill(cv, d, batch, max_tokens, cus);
      break;
    case MLA_OP_DECODE: {
      if (batch <= 0 || max_ctx_len < 0 || num_splits < 0) return MLA_ERR_INVALID_ARG;
      carve_decode(cv, d, batch, max_ctx_len, num_splits, cus);
      break;
    }
    case MLA_OP_PREFILL_CHUNK:
      if (batch <= 0 || max_tokens <= 0 || max_ctx_len < 0) return MLA_ERR_INVALID_ARG;
      carve_prefill(cv, d, batch, max_tokens, cus, true, max_ctx_len);
      break;
    default: return MLA_ERR_INVALID_ARG;
  }
  *bytes = cv.off;
  return MLA_OK;
}

int mla_cache_append(const mla_dims* d, const mla_weights* w, const mla_paged_cache* c, const void* h, int32_t n,
                     const int32_t* seq_idx, const int32_t* pos, void* workspace, size_t ws_bytes, void* stream) {
  int st = validate_dims(d);
  if (st != MLA_OK) return st;
  if ((st = validate_cache(d, c)) != MLA_OK) return st;
  if (!w || !w->W_DKV || !w->W_KR || n < 0 || !weights_norm_ok(d, w)) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (!h || !seq_idx || !pos) return MLA_ERR_INVALID_ARG;
  const int cus = device_cus();
  Carve sz(nullptr);
  carve_append(sz, d, n, cus);
  if (!workspace || ws_bytes < sz.off) return MLA_ERR_WORKSPACE;
  if (kDebug && (st = debug_check_slots(c, seq_idx, pos, n)) != MLA_OK) return st;
  Carve cv(workspace);
  AppendWs ws = carve_append(cv, d, n, cus);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  MLA_HIP(rope_table(pos, n, d->d_hr, freq_of(d), ws.rope, s));
  return run_cache_writer(d, w, c, h, n, seq_idx, pos, ws.rope, ws.plan, ws.partial, ws.staged, s);
}

int mla_quantize_entries(const mla_dims* d, const void* entries, int32_t n, uint8_t* codes, float* scales,
                         void* stream) {
  int st = validate_dims(d);
  if (st != MLA_OK) return st;
  if (!fp8_cache(d) || n < 0) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (!entries || !codes || !scales) return MLA_ERR_INVALID_ARG;
  QuantDst q;
  q.codes = codes;
  q.scales = scales;
  MLA_HIP(quantize_entries_run(entries, entry(d), n, q, reinterpret_cast<hipStream_t>(stream)));
  return MLA_OK;
}

int mla_decode_attention(const mla_dims* d, const mla_paged_cache* c, const void* q, int32_t batch,
                         const int32_t* kv_lens, int32_t max_kv_len, int32_t num_splits, void* o_hat, float* lse,
                         void* workspace, size_t ws_bytes, void* stream) {
  int st = validate_dims(d);
  if (st != MLA_OK) return st;
  if ((st = validate_cache(d, c)) != MLA_OK) return st;
  if (!q || !kv_lens || !o_hat || batch <= 0 || max_kv_len <= 0 || num_splits < 0) return MLA_ERR_INVALID_ARG;
  if ((int64_t)max_kv_len > (int64_t)c->max_blocks_per_seq * c->block_size) return MLA_ERR_INVALID_ARG;
  if (!decode_supported(d->d_c, d->d_hr)) return MLA_ERR_UNSUPPORTED;
  const int cus = device_cus();
  Carve sz(nullptr);
  carve_decode(sz, d, batch, max_kv_len - 1, num_splits, cus);
  if (!workspace || ws_bytes < sz.off) return MLA_ERR_WORKSPACE;
  if (kDebug && (st = debug_check_tokens(c, kv_lens, batch, 0, max_kv_len)) != MLA_OK) return st;
  Carve cv(workspace);
  DecodeWs ws = carve_decode(cv, d, batch, max_kv_len - 1, num_splits, cus);
  DecodeAttnParams a{};
  a.q = q;
  a.pool = c->pool;
  a.fp8 = fp8_cache(d);
  a.scales = c->scales;
  a.block_table = c->block_table;
  a.max_blocks = c->max_blocks_per_seq;
  a.block_size = c->block_size;
  a.lens = kv_lens;
  a.lens_plus_one = false;
  a.B = batch;
  a.n_h = d->n_h;
  a.d_c = d->d_c;
  a.d_hr = d->d_hr;
  a.scale_log2 = scale_of(d) * 1.4426950408889634f;
  a.splits = ws.attn.splits;
  a.tokens_per_split = ws.attn.tps;
  a.part_m = ws.attn.pm;
  a.part_l = ws.attn.pl;
  a.part_o = ws.attn.po;
  a.units = ws.attn.balanced ? ws.attn.units : nullptr;
  a.cus = cus;
  a.o_hat = o_hat;
  a.lse = lse;
  MLA_HIP(decode_attention(dt(d), a, reinterpret_cast<hipStream_t>(stream)));
  return MLA_OK;
}

int mla_decode_attention_partials(const mla_dims* d, const mla_paged_cache* c, const void* q, int32_t batch,
                                  const int32_t* kv_lens, int32_t max_kv_len, int32_t num_splits, float* part_m,
                                  float* part_l, void* part_o, int32_t* splits_out, void* stream) {
  int st = validate_dims(d);
  if (st != MLA_OK) return st;
  if ((st = validate_cache(d, c)) != MLA_OK) return st;
  if (!q || !kv_lens || !part_m || !part_l || !part_o || !splits_out || batch <= 0 || max_kv_len <= 0 ||
      num_splits <= 0)
    return MLA_ERR_INVALID_ARG;
  if ((int64_t)max_kv_len > (int64_t)c->max_blocks_per_seq * c->block_size) return MLA_ERR_INVALID_ARG;
  if (!decode_supported(d->d_c, d->d_hr)) return MLA_ERR_UNSUPPORTED;
  DecodeAttnParams a{};
  a.q = q;
  a.pool = c->pool;
  a.fp8 = fp8_cache(d);
  a.scales = c->scales;
  a.block_table = c->block_table;
  a.max_blocks = c->max_blocks_per_seq;
  a.block_size = c->block_size;
  a.lens = kv_lens;
  a.lens_plus_one = false;
  a.B = batch;
  a.n_h = d->n_h;
  a.d_c = d->d_c;
  a.d_hr = d->d_hr;
  a.scale_log2 = scale_of(d) * 1.4426950408889634f;
  a.splits = split_count(max_kv_len, num_splits, &a.tokens_per_split);
  a.part_m = part_m;
  a.part_l = part_l;
  a.part_o = part_o;
  a.units = nullptr;
  a.cus = device_cus();
  a.leave_partials = true;
  if (!decode_bf16_partials(dt(d), a)) return MLA_ERR_UNSUPPORTED;
  if (kDebug && (st = debug_check_tokens(c, kv_lens, batch, 0, max_kv_len)) != MLA_OK) return st;
  *splits_out = a.splits;
  MLA_HIP(decode_attention(dt(d), a, reinterpret_cast<hipStream_t>(stream)));
  return MLA_OK;
}

int mla_decode(const mla_dims* d, const mla_weights* w, const mla_paged_cache* c, const void* h, int32_t batch,
               const int32_t* ctx_lens, int32_t max_ctx_len, int32_t num_splits, void* u, float* o_heads,
               void* workspace, size_t ws_bytes, void* stream) {
  return decode_impl(d, w, c, h, batch, ctx_lens, max_ctx_len, num_splits, u, o_heads, workspace, ws_bytes, stream);
}

int mla_decode_noalloc(const mla_dims* d, const mla_weights* w, const mla_paged_cache* c, const void* h,
                       int32_t batch, const int32_t* ctx_lens, int32_t max_ctx_len, int32_t num_splits, void* u,
                       float* o_heads, void* stream) {
  void* ws = nullptr;
  const int st = noalloc_scratch(&ws);
  if (st != MLA_OK) return st;
  return decode_impl(d, w, c, h, batch, ctx_lens, max_ctx_len, num_splits, u, o_heads, ws, kNoAllocBytes, stream);
}

}  // extern "C"

namespace {

int decode_impl(const mla_dims* d, const mla_weights* w, const mla_paged_cache* c, const void* h, int32_t batch,
                const int32_t* ctx_lens, int32_t max_ctx_len, int32_t num_splits, void* u, float* o_heads,
                void* workspace, size_t ws_bytes, void* stream) {
  int st = validate_dims(d);
  if (st != MLA_OK) return st;
  if ((st = validate_cache(d, c)) != MLA_OK) return st;
  if (!w || !w->W_UQ || !w->W_QR || !w->W_DKV || !w->W_KR || !w->W_UK || !w->W_UV || !w->W_O)
    return MLA_ERR_INVALID_ARG;
  if ((d->d_cq > 0) != (w->W_DQ != nullptr) || !weights_norm_ok(d, w)) return MLA_ERR_INVALID_ARG;
  if (!h || !ctx_lens || !u || batch <= 0 || max_ctx_len < 0 || num_splits < 0) return MLA_ERR_INVALID_ARG;
  if ((int64_t)max_ctx_len + 1 > (int64_t)c->max_blocks_per_seq * c->block_size) return MLA_ERR_INVALID_ARG;
  if (!decode_supported(d->d_c, d->d_hr)) return MLA_ERR_UNSUPPORTED;
  const int cus = device_cus();
  Carve sz(nullptr);
  carve_decode(sz, d, batch, max_ctx_len, num_splits, cus);
  if (!workspace || ws_bytes < sz.off) return MLA_ERR_WORKSPACE;
  // the new token goes to position ctx_lens[b]: ctx_lens[b] + 1 tokens per sequence
  if (kDebug && (st = debug_check_tokens(c, ctx_lens, batch, 1, max_ctx_len)) != MLA_OK) return st;
  Carve cv(workspace);
  DecodeWs ws = carve_decode(cv, d, batch, max_ctx_len, num_splits, cus);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const DType t = dt(d);
  const int B = batch, E = entry(d), qw = q_in(d);

  const void* qin = h;
  // over the fp8 cache the new entries are quantised by the W_UK absorption's launch (workgroups of
  // its own; the attention, which reads them, comes after it)
  const bool quant_in_absorb = fp8_cache(d) && absorb_ok(t, d->d_h, d->d_c);
  {  // [c^q | c^KV | k^R] = [W_DQ; W_DKV; W_KR] h: c^q to the workspace, the new token's cache
     // entry to position ctx_lens[b] of its sequence
    GemmParams g;
    g.A = h; g.lda = d->d_model; g.ldb = d->d_model;
    // the RoPE table of the new tokens' positions ctx_lens[b] (rows are sequences 0..B-1), read
    // by this product's epilogue and the next one's
    g.side_rope.pos = ctx_lens; g.side_rope.n = B; g.side_rope.half = d->d_hr / 2;
    g.side_rope.f = freq_of(d); g.side_rope.tab = ws.rope;
    g.M = B; g.N = kvq_cols(d); g.K = d->d_model;
    if (d->d_cq > 0) {
      g.B0 = w->W_DQ; g.N0 = d->d_cq;
      g.B1 = w->W_DKV; g.N1 = d->d_cq + d->d_c;
      g.B2 = w->W_KR;
      g.epi = dense(ws.cq, d->d_cq);
      g.E0 = d->d_cq;
      g.epi2 = staged_entries(d, w) ? staged_epilogue(d, ws.staged, ws.rope)
                                    : cache_epilogue(d, c, ws.rope, nullptr, ctx_lens);
      qin = ws.cq;
    } else {
      g.B0 = w->W_DKV; g.N0 = d->d_c;
      g.B1 = w->W_KR;
      g.epi = staged_entries(d, w) ? staged_epilogue(d, ws.staged, ws.rope)
                                   : cache_epilogue(d, c, ws.rope, nullptr, ctx_lens);
    }
    MLA_HIP(gemm_run(t, g, ws.gm.kvq, ws.partial, s));
    if (staged_entries(d, w)) {  // entries to their pages; the c^q norm rides along
      const int rc = finish_entries(d, w, c, ws.staged, B, nullptr, ctx_lens, s, d->d_cq > 0 ? ws.cq : nullptr, B,
                                    quant_in_absorb);
      if (rc != MLA_OK) return rc;
    } else if (w->g_cq) {
      MLA_HIP(rmsnorm_rows(t, ws.cq, B, d->d_cq, d->d_cq, w->g_cq, eps_of(d), s));
    }
  }
  {  // [q^C | q^R] = [W_UQ; W_QR] c^q: q^C to the workspace, RoPE'd q^R into columns
     // [d_c, d_c + d_hr) of each head's absorbed query row
    GemmParams g;
    g.A = qin; g.lda = qw; g.ldb = qw;
    g.B0 = w->W_UQ; g.N0 = d->n_h * d->d_h;
    g.B1 = w->W_QR;
    g.M = B; g.N = q_cols(d); g.K = qw;
    g.epi = dense(ws.qc, (int64_t)d->n_h * d->d_h);
    g.E0 = d->n_h * d->d_h;
    g.epi2 = dense(ws.qcat, (int64_t)d->n_h * E);
    g.epi2.group = d->d_hr; g.epi2.group_stride = E; g.epi2.group_off = d->d_c;
    g.epi2.rope_col0 = 0; g.epi2.d_hr = d->d_hr; g.epi2.rope_tab = ws.rope;
    MLA_HIP(gemm_run(t, g, ws.gm.q, ws.partial, s));
  }
  // the latent attention's parameters (over ctx_lens[b] + 1 entries); with balanced work units the
  // absorption launch builds their table
  DecodeAttnParams a{};
  a.q = ws.qcat; a.pool = c->pool; a.block_table = c->block_table;
  a.fp8 = fp8_cache(d); a.scales = c->scales;
  a.max_blocks = c->max_blocks_per_seq; a.block_size = c->block_size;
  a.lens = ctx_lens; a.lens_plus_one = true;
  a.B = B; a.n_h = d->n_h; a.d_c = d->d_c; a.d_hr = d->d_hr;
  a.scale_log2 = scale_of(d) * 1.4426950408889634f;
  a.splits = ws.attn.splits; a.tokens_per_split = ws.attn.tps;
  a.part_m = ws.attn.pm; a.part_l = ws.attn.pl; a.part_o = ws.attn.po;
  a.units = ws.attn.balanced ? ws.attn.units : nullptr; a.cus = cus;
  a.o_hat = ws.ohat; a.lse = nullptr;
  if (absorb_ok(t, d->d_h, d->d_c)) {  // q_hat_i = W_UK_i^T q^C_i -> columns [0, d_c) of each head's row
    QuantJob qj;
    if (quant_in_absorb) {
      qj.src = ws.staged; qj.src_ld = E; qj.n = B;
      qj.dst = quant_dst(c, nullptr, ctx_lens);
      qj.gain = w->g_ckv; qj.eps = eps_of(d); qj.writeback = true;
    }
    const bool units_here = a.units && B <= 64;
    MLA_HIP(absorb_run(ws.qc, w->W_UK, ws.qcat, B, d->n_h, d->d_h, d->d_c, (int64_t)d->n_h * E, E, s,
                       quant_in_absorb ? &qj : nullptr, units_here ? &a : nullptr));
    a.units_ready = units_here;
  } else {
    GemmParams g;
    g.A = ws.qc; g.lda = (int64_t)d->n_h * d->d_h; g.strideA = d->d_h;
    g.B0 = w->W_UK; g.ldb = d->d_c; g.strideB = (int64_t)d->d_h * d->d_c; g.nn = true;
    g.M = B; g.N = d->d_c; g.K = d->d_h; g.batch = d->n_h;
    g.epi = dense(ws.qcat, (int64_t)d->n_h * E);
    g.epi.batch_stride = E;
    MLA_HIP(gemm_run(t, g, ws.gm.absorb, ws.partial, s));
  }
  UvPartials parts;
  {  // latent attention over ctx_lens[b] + 1 entries
    // with several partitions and the W_UV kernel that combines them, the combine pass is skipped;
    // not when many partitions meet few workgroups of that kernel (a small batch with few heads):
    // the combine kernel's workgroup per row then spreads the partition reads over the chip
    // (measured: V2-Lite, batch 8, up to 128 partitions: 69.4 against 77.7 us per step; the
    // 128-head long-context batch keeps the fused combine, 192.5 against 209.2 us)
    const bool fused_combine = a.splits < 16 || uv_parts_workgroups(B, d->n_h) >= cus / 2;
    a.leave_partials = a.splits > 1 && fused_combine && uv_parts_ok(t, d->d_h, d->d_c) && decode_bf16_partials(t, a);
    MLA_HIP(decode_attention(t, a, s));
    parts.m = a.part_m; parts.l = a.part_l; parts.o = a.part_o;
    parts.splits = a.leave_partials ? a.splits : 0;
  }
  if (parts.splits > 0) {  // o_i = W_UV_i o_hat_i, o_hat_i combined from the partitions
    MLA_HIP(uv_run(nullptr, w->W_UV, ws.o, o_heads, B, d->n_h, d->d_h, s, &parts));
  } else if (uv_ok(t, d->d_h, d->d_c)) {  // o_i = W_UV_i o_hat_i
    MLA_HIP(uv_run(ws.ohat, w->W_UV, ws.o, o_heads, B, d->n_h, d->d_h, s));
  } else {
    GemmParams g;
    g.A = ws.ohat; g.lda = (int64_t)d->n_h * d->d_c; g.strideA = d->d_c;
    g.B0 = w->W_UV; g.ldb = d->d_c; g.strideB = (int64_t)d->d_h * d->d_c;
    g.M = B; g.N = d->d_h; g.K = d->d_c; g.batch = d->n_h;
    g.epi = dense(ws.o, (int64_t)d->n_h * d->d_h);
    g.epi.batch_stride = d->d_h;
    g.epi.C2 = o_heads;
    MLA_HIP(gemm_run(t, g, ws.gm.uv, ws.partial, s));
  }
  {  // u = W_O [o_1; ...; o_n_h] (the weight-streaming kernel: faster than hipBLASLt at M <= 64)
    GemmParams g;
    g.A = ws.o; g.lda = (int64_t)d->n_h * d->d_h; g.B0 = w->W_O; g.ldb = (int64_t)d->n_h * d->d_h;
    g.M = B; g.N = d->d_model; g.K = d->n_h * d->d_h;
    g.epi = dense(u, d->d_model);
    MLA_HIP(gemm_run(t, g, ws.gm.out, ws.partial, s));
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_prefill(const mla_dims* d, const mla_weights* w, const mla_paged_cache* c, const void* h, int32_t batch,
                int32_t T, void* u, float* o_heads, void* workspace, size_t ws_bytes, void* stream) {
  return prefill_impl(d, w, c, h, batch, T, nullptr, 0, u, o_heads, workspace, ws_bytes, stream);
}

int mla_prefill_chunk(const mla_dims* d, const mla_weights* w, const mla_paged_cache* c, const void* h,
                      int32_t batch, int32_t T, const int32_t* start_pos, int32_t max_start, void* u, float* o_heads,
                      void* workspace, size_t ws_bytes, void* stream) {
  if (!start_pos || max_start < 0) return MLA_ERR_INVALID_ARG;
  return prefill_impl(d, w, c, h, batch, T, start_pos, max_start, u, o_heads, workspace, ws_bytes, stream);
}

}  // extern "C"
