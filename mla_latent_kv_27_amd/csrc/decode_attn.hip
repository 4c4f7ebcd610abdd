// Decode latent attention over the paged MLA cache, split-KV, on gfx950 matrix cores.
//
// With W_UK folded into the query and W_UV applied after the softmax (the associativity
// argument of App. C, "Full Formulas of MLA", DeepSeek-V2 summary page), every head of a
// sequence attends over the same cached entries [c^KV_j | k^R_j]:
//   s_ij = scale * (q_hat_i . c^KV_j + q^R_i . k^R_j),   o_hat_i = sum_j softmax_j(s_ij) c^KV_j.
// So one streamed cache tile serves all the heads of a workgroup, and both contractions are
// dense: S^T = K Q^T over d_c + d_hr and O^T = V^T P^T over the tile's tokens, where K is the
// tile itself and V is its first d_c columns.
//
// Layout of the work:
//   * a workgroup = (sequence b, group of 16*NW heads, KV partition); each wave owns 16 heads;
//   * a tile of 32 tokens is gathered through the block table into LDS twice: token-major
//     (the A operand of S^T) and latent-major (the A operand of O^T);
//   * S^T accumulators give each lane one head and 8 tokens, which is exactly the B operand
//     that O^T needs for those 8 tokens, so probabilities never leave registers;
//   * the online softmax (running max and sum per head) uses exp2 with the scale pre-multiplied
//     by log2(e) and cross-lane shuffles over the 4 lane groups that share a head;
//   * partitions write (max, sum, unnormalised o_hat) and a second kernel combines them with
//     the log-sum-exp rule; with one partition the kernel writes o_hat directly.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "units.h"

namespace mla {

constexpr int kTile = 32;  // tokens per LDS tile

template <int DC, int DR, typename T>
struct DecodeShape {
  static constexpr int D = DC + DR;                       // cache entry width
  static constexpr int DP = (D + 31) / 32 * 32;           // contraction padded to 32
  static constexpr int KCH = DP / 32;                     // 32-wide k chunks
  static constexpr int EPC = 16 / sizeof(T);              // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                     // chunks per cache row
  static constexpr int LDK = DP + EPC;                    // Ks row (elements), padded
  static constexpr int LDV = kTile + (sizeof(T) == 2 ? 4 : 4);  // Vt row (elements), padded
  static constexpr int DB = DC / 16;                      // 16-row latent blocks
};

template <typename T, int DC, int DR, int NW>
__global__ void __launch_bounds__(64 * NW) decode_attn_kernel(DecodeAttnParams p, int HG) {
  using Sh = DecodeShape<DC, DR, T>;
  constexpr int NT = 64 * NW;
  __shared__ __attribute__((aligned(16))) T Ks[kTile * Sh::LDK];
  __shared__ __attribute__((aligned(16))) T Vt[DC * Sh::LDV];

  // blockIdx -> (unit = (b, split), head group); all head groups of a unit get the same
  // blockIdx % 8 so that they run on the same XCD and share its L2 for the cache tiles.
  const int units = p.B * p.splits;
  const int i = blockIdx.x;
  const int grp = i / (8 * HG), rem = i % (8 * HG);
  const int hg = rem / 8;
  const int unit = grp * 8 + (rem % 8);
  if (unit >= units) return;
  const int b = unit / p.splits, split = unit % p.splits;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, hl = lane & 15;
  const int head = hg * 16 * NW + w * 16 + hl;
  const bool valid_head = head < p.n_h;

  const int kv_len = p.lens[b] + (p.lens_plus_one ? 1 : 0);
  const int ntiles = (kv_len + kTile - 1) / kTile;
  const int tps = p.tokens_per_split / kTile;
  const int t_begin = split * tps;
  const int t_end = min(ntiles, t_begin + tps);

  // Q^T fragments (B operand): head = hl, k = 8g..8g+7 of every 32-chunk.
  Frag8<T> q[Sh::KCH];
  {
    const T* qrow = reinterpret_cast<const T*>(p.q) + ((int64_t)b * p.n_h + (valid_head ? head : 0)) * Sh::D;
#pragma unroll
    for (int kc = 0; kc < Sh::KCH; ++kc) {
      const int k = kc * 32 + 8 * g;
      if (valid_head && k < Sh::D) load8(q[kc], qrow + k);
      else zero8(q[kc]);
    }
  }
  // zero the padded contraction columns once (never overwritten by tile loads)
  if (Sh::DP > Sh::D) {
    for (int c = tid; c < kTile * (Sh::DP - Sh::D); c += NT) {
      const int r = c / (Sh::DP - Sh::D), k = Sh::D + c % (Sh::DP - Sh::D);
      Ks[r * Sh::LDK + k] = from_f32<T>(0.f);
    }
  }

  floatx4 o[Sh::DB];
#pragma unroll
  for (int d = 0; d < Sh::DB; ++d) o[d] = floatx4{0, 0, 0, 0};
  float m_run = -INFINITY, l_run = 0.f;

  const char* pool = reinterpret_cast<const char*>(p.pool);
  const int32_t* bt = p.block_table + (int64_t)b * p.max_blocks;

  for (int t = t_begin; t < t_end; ++t) {
    __syncthreads();
    for (int c = tid; c < kTile * Sh::CPR; c += NT) {
      const int tok = c / Sh::CPR, cc = c % Sh::CPR;
      const int abs_tok = t * kTile + tok;
      Chunk16 v = zero16();
      if (abs_tok < kv_len) {
        const int64_t slot = (int64_t)bt[abs_tok / p.block_size] * p.block_size + abs_tok % p.block_size;
        v = ld16(pool + (slot * Sh::D + cc * Sh::EPC) * (int64_t)sizeof(T));
      }
      st16(&Ks[tok * Sh::LDK + cc * Sh::EPC], v);
      if (cc * Sh::EPC < DC) {
        const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
        for (int x = 0; x < Sh::EPC; ++x) Vt[(cc * Sh::EPC + x) * Sh::LDV + tok] = e[x];
      }
    }
    __syncthreads();

    // S^T (tokens x heads): lane holds head hl, tokens tb*16 + 4g + j
    floatx4 s[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      s[tb] = floatx4{0, 0, 0, 0};
#pragma unroll
      for (int kc = 0; kc < Sh::KCH; ++kc) {
        Frag8<T> a;
        load8(a, &Ks[(tb * 16 + hl) * Sh::LDK + kc * 32 + 8 * g]);
        s[tb] = mma16(a, q[kc], s[tb]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int abs_tok = t * kTile + tb * 16 + 4 * g + j;
        const float x = abs_tok < kv_len ? s[tb][j] * p.scale_log2 : -INFINITY;
        s[tb][j] = x;
        mx = fmaxf(mx, x);
      }
    mx = wave_max_xor(mx, 16);
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float sum = 0.f;
    Frag8<T> pf;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // the sum uses the probabilities as rounded for the PV product, so the weights applied
        // to the latent rows sum to exactly the normaliser
        const float e = to_f32(from_f32<T>(exp2f(s[tb][j] - m_new)));
        sum += e;
        set8(pf, tb * 4 + j, e);
      }
    sum = wave_sum_xor(sum, 16);
    sum = wave_sum_xor(sum, 32);
    l_run = l_run * alpha + sum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < Sh::DB; ++d) {
      o[d] *= alpha;
      Frag8<T> a;
      const T* vr = &Vt[(d * 16 + hl) * Sh::LDV + 4 * g];
      load4x2(a, vr, vr + 16);
      o[d] = mma16(a, pf, o[d]);
    }
  }

  if (!valid_head) return;
  if (p.splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    T* out = reinterpret_cast<T*>(p.o_hat) + ((int64_t)b * p.n_h + head) * DC;
#pragma unroll
    for (int d = 0; d < Sh::DB; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) out[d * 16 + 4 * g + j] = from_f32<T>(o[d][j] * inv);
    if (p.lse && g == 0) p.lse[(int64_t)b * p.n_h + head] = (m_run + log2f(l_run)) * 0.69314718055994531f;
    return;
  }
  const int64_t pi = ((int64_t)b * p.splits + split) * p.n_h + head;
  if (g == 0) {
    p.part_m[pi] = m_run;
    p.part_l[pi] = l_run;
  }
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* po = reinterpret_cast<float*>(p.part_o) + pi * DC;
#pragma unroll
  for (int d = 0; d < Sh::DB; ++d) *reinterpret_cast<floatx4*>(po + d * 16 + 4 * g) = o[d] * inv;
}

// ----------------------------------------------------------------------------- balanced units
// (the table builder is in units.h: the W_UK absorption launch can run it as well)
__global__ void __launch_bounds__(256) decode_units_kernel(DecodeAttnParams p) { build_decode_units(p); }

// ----------------------------------------------------------------------------- tiled kernel
// The DeepSeek-V2-sized cases (d_c = 512, d_hr = 64; the bf16 kernel and, with its own tiles, the
// fp8 one).  A workgroup is eight waves (two per SIMD, hiding each other's LDS and copy latency)
// and one (sequence, KV partition, group of 128 heads); with more than 128 heads the other head
// groups' workgroups read the same tiles and get block ids on the same XCD, so their repeat reads
// come from its L2.
//   * Tiles of 32 tokens arrive by direct global->LDS copies into a ring of four buffers.
//   * LDS row of a token = its 1152-byte cache entry as 72 16-byte chunks; chunk c of token t is
//     stored at chunk slot t*72 + (c ^ (t & 7)) so that the 16 tokens of an MFMA operand read
//     fall on different banks.
//   * S^T = K Q^T with 16x16x32 MFMA: A = 16 tokens x 32 latent dims (ds_read_b128),
//     B = Q^T held in registers for the whole kernel (18 k-chunks x 8 values).
//   * O^T = V^T P^T: the A operand (16 latent dims x 32 tokens) is read straight from the
//     token-major tile with the gfx950 LDS transpose read (ds_read_b64_tr_b16): within each
//     16-lane group, source lane s supplies 4 consecutive dims of token 4j + s/4 and lane i
//     receives dim i of those four tokens.
//   * The softmax keeps a per-head reference max that every lane of the head shares, so the common
//     tile needs no cross-lane exchange; every lane keeps a partial sum combined once at the end.
namespace tiled {
constexpr int kT = 32;                    // tokens per tile
constexpr int kNBuf = 4;                  // ring buffers
constexpr int kD = 576, kDC = 512;        // entry width, latent width
constexpr int kCPR = kD * 2 / 16;         // 72 chunks per entry
constexpr int kRow = kCPR * 16;           // 1152 bytes per entry
constexpr int kBytes = kT * kRow;         // 36864 per buffer
constexpr int kWaves = 8;
constexpr int kDmaTotal = kT * kCPR / 64;  // 36 one-KiB copies per tile, nine from each of waves 0-3
constexpr int kDmaPerWave = kDmaTotal / 4;
constexpr float kLazy = 8.f;              // log2 headroom before a rescale
}  // namespace tiled

__shared__ __attribute__((aligned(1024))) char g_kv0[tiled::kBytes];
__shared__ __attribute__((aligned(1024))) char g_kv1[tiled::kBytes];
__shared__ __attribute__((aligned(1024))) char g_kv2[tiled::kBytes];
__shared__ __attribute__((aligned(1024))) char g_kv3[tiled::kBytes];


template <int BUF>
__device__ __forceinline__ char* kv_buf() {
  return BUF == 0 ? g_kv0 : (BUF == 1 ? g_kv1 : (BUF == 2 ? g_kv2 : g_kv3));
}

struct TiledCtx {
  const char* pool;
  const float* scales;  // the fp8 cache's (s_c, s_r) per slot
  const int32_t* bt;
  int bs, kv_len;
  uint32_t dma_off[5];  // this lane's byte offsets of its copies (bf16: nine, fp8: five) in a tile, 16 bits each
};

// The copy itself, written as one asm statement (M0 = the LDS destination): the compiler then does
// not treat the ring's fragment reads as possibly waiting on these copies (with more copies in
// flight than it tracks it would wait for most of them before every read).  The waits on them are
// the kernel's own: a tile is read only after every wave has waited for its own copies of it and
// passed a barrier, and every copy is waited for before the workgroup ends.
__device__ __forceinline__ void dma16_ring(__amdgpu_buffer_rsrc_t span, uint32_t off, const void* lds_dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_dst;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(span), "s"(m0)
               : "memory", "m0");
}

// This wave's share of the 36 direct-to-LDS copies of tile `tile` into buffer BUF: waves 0-3 copy
// nine 1-KiB pieces each (rows 8w .. 8w+7), waves 4-7 none.  Issued all by half of the waves, the
// copies hold up only those (measured: 169.5 against 175.6 us with every wave issuing its share,
// and slower again with the copies spread through the multiply): the other wave of each SIMD
// starts its products at once and has the matrix core to itself meanwhile.  block_size is a multiple of the tile size, so a tile lies
// inside one block: one uniform block-table lookup.  The buffer resource spans only the tile's rows
// inside the context: rows past it read as zeros (an out-of-range buffer read returns zero, and the
// copy writes those zeros), so a partial last tile needs no clearing.  A tile past the partition
// (live == false) reads nothing at all; its copies are still issued so that every step of a wave
// issues the same number.  The lane's nine byte offsets within a tile are the same for every tile:
// they are worked out once, before the loop, and kept as 16-bit halves of five registers (working
// them out in every phase, ten vector instructions per copy, cost the copying waves ~90 vector
// instructions a phase: V2-Lite attention 18.5 against 20.1 us, the V2 batch 1% faster).
template <int BUF>
__device__ __forceinline__ void issue_tile(const TiledCtx& c, int tile, bool live, int w, int lane) {
  using namespace tiled;
  char* dst = kv_buf<BUF>();
  const int tok0 = tile * kT;
  const int blk = tok0 / c.bs;
  const char* base = c.pool + ((int64_t)c.bt[live ? blk : 0] * c.bs + (tok0 - blk * c.bs)) * kRow;
  const int first = kDmaPerWave * w;
  const int rows = live ? min(kT, c.kv_len - tok0) : 0;
  const __amdgpu_buffer_rsrc_t span = dma_span(base, (uint32_t)rows * kRow);
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    if (w < 4) {
      const uint32_t off = (c.dma_off[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      dma16_ring(span, off, dst + (first + i) * 1024);
    }
  }
}

// ---- the bf16 kernel: S by head, P.V by latent column, one barrier per tile
// The S^T = K Q^T product stays with the head's wave (Q is register-resident), but P.V is split by
// latent columns: wave w accumulates O^T for dims 64w .. 64w+63 of all the workgroup's heads.  Its
// A operand (V^T, 16 dims x 32 tokens) is then read once per tile and feeds one MFMA per 16-head
// block, and each B operand (P^T, 32 tokens x 16 heads) one MFMA per 16-dim block, instead of every
// wave reading the whole tile for its own 16 heads.  The probabilities cross waves through LDS, in
// the B-operand layout: the S^T accumulators of lane (g, l16) hold head l16 at tokens
// 16 (s/4) + 4g + s%4, which is exactly that lane's B fragment, so a wave stores its 16-byte
// fragment at [g][head] and the P.V waves read it back with one 16-byte read per head block.
//
// Software pipeline: between two barriers a wave multiplies P.V of tile t-1 and then S of tile t, so
// one barrier per tile publishes tile t's probabilities, retires tile t-1's buffer and makes tile
// t+1 visible.  The probabilities alternate between two LDS buffers; the ring holds tiles t-1 (P.V),
// t (S) and the copies of t+1 and t+2 in flight.
//
// The softmax reference of a head is fixed by the partition's first tile.  A later score more than
// 2^kHeadroom above it (rare: P and O stay far from overflow below that) raises the reference, which
// would leave O rows summed over two references in every wave; the partition then restarts from its
// first tile with the raised references.  O therefore never passes through the vector ALU inside the
// loop.  The restart request travels with the probabilities themselves: a wave that raised a
// reference writes the value -1 (bf16 0xBF80) as the first probability of each of its fragments, a
// value no probability takes (2^x is never negative, and a NaN from a corrupt cache entry has an
// all-ones exponent, so it cannot pose as a request and restart the partition forever).  Every wave,
// reading every head block's fragments for its P.V, sees the request in the next phase; its O is
// discarded by the restart, so the replaced values do no harm.  Nothing else in LDS carries it, so no
// copy into the ring can overwrite a request before every wave has read it.
namespace sp {
constexpr float kHeadroom = 64.f;  // log2 units a score may exceed its head's reference by
}  // namespace sp

__shared__ __attribute__((aligned(1024))) char g_pex0[4 * 128 * 16];  // [lane group][head][8 bf16]
__shared__ __attribute__((aligned(1024))) char g_pex1[4 * 128 * 16];
template <int PB>
__device__ __forceinline__ char* pex_buf() { return PB == 0 ? g_pex0 : g_pex1; }

struct SplitState {
  floatx4 o[4][8];  // O^T: latent dims 16 (4w + db) + 4g + j of head 16 hb + l16
  float m_ref;      // S side: reference max of head 16w + l16 (log2 domain), shared by its lanes
  float l_part;     // S side: this lane's partial normaliser
};

// S^T for this wave's 16 heads over the tile in buffer BUF, the softmax against the fixed
// references and the probabilities into P buffer PB.  Returns 1 when a reference had to be raised
// (the same in every lane).
template <int BUF, int PB>
__device__ __forceinline__ unsigned char sp_scores(const Frag8<bf16> (&q)[18], SplitState& st, int t, int kv_len,
                                          float scale_log2, int w, int lane) {
  using namespace tiled;
  const char* buf = kv_buf<BUF>();
  // the lane's LDS offsets are recomputed in every step (a few integer ops) rather than kept live
  // for all four ring buffers across the loop
  asm volatile("" : "+v"(lane));
  const int g = lane >> 4, l16 = lane & 15;
  // ---- S^T = K Q^T : two 16-token blocks; lane holds head l16, tokens 16*tb + 4g + j
  floatx4 sc[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
  {
    // chunk (4kc + g) of token l16 sits at slot (4kc + g) ^ (l16 & 7): two lane-constant bases
    // (kc parity); 128 bytes per kc pair and 16 rows per token block are immediates
    const int x = l16 & 7;
    const char* rb0 = buf + l16 * kRow + ((g) ^ x) * 16;
    const char* rb1 = buf + l16 * kRow + ((4 + g) ^ x) * 16;
    Frag8<bf16> a[2][2];  // [stage][tb]: the next k-chunk's fragments are in flight
    a[0][0].v = *reinterpret_cast<const bf16x8*>(rb0);
    a[0][1].v = *reinterpret_cast<const bf16x8*>(rb0 + 16 * kRow);
#pragma unroll
    for (int kc = 0; kc < 18; ++kc) {
      if (kc + 1 < 18) {
        const char* pn = ((kc + 1) & 1 ? rb1 : rb0) + 128 * ((kc + 1) >> 1);
        a[(kc + 1) & 1][0].v = *reinterpret_cast<const bf16x8*>(pn);
        a[(kc + 1) & 1][1].v = *reinterpret_cast<const bf16x8*>(pn + 16 * kRow);
      }
      sc[0] = mma16(a[kc & 1][0], q[kc], sc[0]);
      sc[1] = mma16(a[kc & 1][1], q[kc], sc[1]);
    }
  }
  // ---- softmax against the head's reference (masked past the context on a partial tile)
  float lmax = -INFINITY;
  const bool full = (t + 1) * kT <= kv_len;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = sc[tb][j] * scale_log2;
      if (!full && t * kT + tb * 16 + 4 * g + j >= kv_len) v = -INFINITY;
      sc[tb][j] = v;
      lmax = fmaxf(lmax, v);
    }
  unsigned char restart = 0;
  if (__builtin_amdgcn_ballot_w64(lmax > st.m_ref + sp::kHeadroom) != 0) {  // the first tile, or rare
    float hmax = wave_max_xor(lmax, 16);
    hmax = wave_max_xor(hmax, 32);
    // a head whose reference was set already: its O rows hold sums over the old reference
    if (__builtin_amdgcn_ballot_w64(st.m_ref != -INFINITY && lmax > st.m_ref + sp::kHeadroom) != 0) restart = 1;
    st.m_ref = fmaxf(st.m_ref, hmax);
  }
  bf16x8 pf;  // slot s = token 16 (s/4) + 4g + s%4
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pf[tb * 4 + j] = (bf16)__builtin_amdgcn_exp2f(sc[tb][j] - st.m_ref);  // argument <= kHeadroom
  // the normaliser sums the probabilities as P.V multiplies them (rounded to bf16): one bf16 dot
  // product with (1, 1) per pair instead of a widening and an add per value
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
#pragma unroll
  for (int i = 0; i < 8; i += 2)
    st.l_part = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[i], pf[i + 1]}, one, st.l_part, false);
  if (restart) pf[0] = (bf16)-1.f;  // the request: a value no probability takes
  *reinterpret_cast<bf16x8*>(pex_buf<PB>() + ((g * 128) + 16 * w + l16) * 16) = pf;
  return restart;
}

// S of tile t in buffer BUF by the waves that own heads, probabilities into P buffer PB.
template <int BUF, int PB>
__device__ __forceinline__ void sp_scores_wave(const Frag8<bf16> (&q)[18], SplitState& st, int t, int kv_len,
                                               float scale_log2, bool s_wave, int w, int lane) {
  if (s_wave) sp_scores<BUF, PB>(q, st, t, kv_len, scale_log2, w, lane);
}

// ---- the same kernel over the fp8 cache (per-token-scaled e4m3 codes, one scale per part of the
// entry): a tile is 32 tokens x 576 code bytes plus their 32 (s_c, s_r) pairs, half the bytes.
//   * S^T = K Q^T runs on fp8 MFMAs straight from the codes: the query of each head is split into
//     two e4m3 parts sharing one scale, q / s_q = hi + lo (hi the nearest code, lo the code of the
//     remainder), which keeps about bf16 precision;
//     s_tj = scale s_q (s_c,j (q . code_c,j) + s_r,j (q^R . code_r,j)).  The latent part uses the
//     16x16x128 f8f6f4 MFMA (twice the rate of the 16x16x32 fp8 form), the rope part the
//     16x16x32 fp8 one.
//   * P.V is the bf16 one, split by latent column: the V^T fragment comes from the codes by an
//     8-bit LDS transpose read and an exact conversion in registers, and the token's s_c is folded
//     into its probability.
namespace tiled8 {
constexpr int kT = 32;
constexpr int kRow = 576;                   // code bytes per entry (36 chunks)
constexpr int kCodes = kT * kRow;           // 18432
constexpr int kScales = kT * 8;             // 256: (s_c, s_r) per token
constexpr int kBuf = kCodes + kScales;
constexpr int kCodeCopies = kCodes / 1024;  // 18 one-KiB copies per tile
constexpr int kDmaPerWave = 5;              // waves 0-2: five code copies; wave 3: three and the scales
// Chunk c of token row t sits at slot c ^ swz_lat(t) for the 32 latent chunks and c ^ swz_rope(t) for
// the 4 rope chunks (each a permutation within its part of the row).  LDS serves a 16-byte read 8
// lanes at a time and an 8-byte read 16 lanes at a time over 32 banks (128 bytes); rows are 576
// bytes = 16 banks apart, so a chunk's bank group (of 4) is (4 (t & 1) + slot) mod 8.  With these
// swizzles every read of the kernel takes its minimum number of passes: a K fragment read
// (8 consecutive rows, one chunk: u(t) = swz_lat(t) ^ 4 (t & 1) takes 8 distinct values on them), a
// rope read (8 consecutive rows, one chunk: (t & 1, (t >> 1) & 3) distinct) and a V^T transpose read
// (the tokens 4g .. 4g+3 and 16 + 4g .. +3 of a lane group: u distinct on them as well).
__device__ __forceinline__ int swz_lat(int t) { return (t & 3) | ((((t >> 4) ^ (t >> 2) ^ t) & 1) << 2); }
__device__ __forceinline__ int swz_rope(int t) { return (t >> 1) & 3; }
}  // namespace tiled8

typedef int intx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) intx2 lds_intx2_t;

__shared__ __attribute__((aligned(1024))) char g_kv8_0[tiled8::kBuf];
__shared__ __attribute__((aligned(1024))) char g_kv8_1[tiled8::kBuf];
__shared__ __attribute__((aligned(1024))) char g_kv8_2[tiled8::kBuf];
__shared__ __attribute__((aligned(1024))) char g_kv8_3[tiled8::kBuf];
template <int BUF>
__device__ __forceinline__ char* kv8_buf() {
  return BUF == 0 ? g_kv8_0 : (BUF == 1 ? g_kv8_1 : (BUF == 2 ? g_kv8_2 : g_kv8_3));
}

// A 4-byte-per-lane copy (lane i's word lands at the LDS destination + 4 i), the form of dma16_ring.
__device__ __forceinline__ void dma4_ring(__amdgpu_buffer_rsrc_t span, uint32_t off, const void* lds_dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_dst;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(span), "s"(m0)
               : "memory", "m0");
}

// This wave's share of the copies of fp8 tile `tile` into buffer BUF: the 18 one-KiB code copies
// go five each to waves 0-2 and three to wave 3, which also copies the tile's 256 bytes of scales;
// waves 4-7 copy nothing (as in the bf16 kernel).  Rows past the context read as zeros (codes and
// scales), and a tile past the partition (live == false) reads nothing.
template <int BUF>
__device__ __forceinline__ void issue_tile8(const TiledCtx& c, int tile, bool live, int w, int lane) {
  using namespace tiled8;
  char* dst = kv8_buf<BUF>();
  const int tok0 = tile * kT;
  const int blk = tok0 / c.bs;
  const int64_t slot0 = (int64_t)c.bt[live ? blk : 0] * c.bs + (tok0 - blk * c.bs);
  const uint32_t rows = live ? (uint32_t)min(kT, c.kv_len - tok0) : 0u;
  const __amdgpu_buffer_rsrc_t codes = dma_span(c.pool + slot0 * kRow, rows * kRow);
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    if (w < 4) {
      const int P = kDmaPerWave * w + i;
      const uint32_t off = (c.dma_off[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      if (P < kCodeCopies) dma16_ring(codes, off, dst + P * 1024);
      else if (P == kCodeCopies) dma4_ring(dma_span(c.scales + 2 * slot0, rows * 8), off, dst + kCodes);
    }
  }
}

struct QBf16 {
  Frag8<bf16> v[18];  // k-chunk kc: dims 32 kc + 8 g .. +7 of the lane's head
};
struct QFp8 {
  intx8 c_hi[4], c_lo[4];  // latent part, chunk kc: codes of dims 128 kc + 32 g .. +31
  long r_hi[2], r_lo[2];   // rope part, MFMA kr: codes of rope dims 16 g + 8 kr .. +7
  float s;                 // the head's query scale
};

// The head's query as hi + lo e4m3 codes with one scale: s = amax / 448 over the head's 576 values
// (its four lane groups), hi = e4m3(q / s), lo = e4m3(q / s - hi).
__device__ __forceinline__ void load_q_fp8(QFp8& q, const bf16* qrow, bool live, int g) {
  Frag8<bf16> qv[18];  // 0..15: latent dims 128 (i / 4) + 32 g + 8 (i % 4); 16, 17: rope dims 16 g + 8 kr
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 18; ++i) {
    const int off = i < 16 ? 128 * (i >> 2) + 32 * g + 8 * (i & 3) : 512 + 16 * g + 8 * (i - 16);
    if (live) load8(qv[i], qrow + off);
    else zero8(qv[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)qv[i].v[e]));
  }
  amax = wave_max_xor(amax, 16);
  amax = wave_max_xor(amax, 32);
  q.s = amax / 448.f;
  const float inv = amax > 0.f ? 448.f / amax : 0.f;
  // 4 values -> one word of hi codes and one of lo codes
  auto split4 = [&](const Frag8<bf16>& v, int h, uint32_t& hw, uint32_t& lw) {
    float x[4], r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = fminf(fmaxf((float)v.v[4 * h + e] * inv, -448.f), 448.f);
    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], pk, true);
    const floatx2 b0 = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
    const floatx2 b1 = __builtin_amdgcn_cvt_pk_f32_fp8(pk, true);
    r[0] = x[0] - b0[0];
    r[1] = x[1] - b0[1];
    r[2] = x[2] - b1[0];
    r[3] = x[3] - b1[1];
    int pl = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
    pl = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], pl, true);
    hw = (uint32_t)pk;
    lw = (uint32_t)pl;
  };
#pragma unroll
  for (int i = 0; i < 18; ++i) {
    uint32_t h0, l0, h1, l1;
    split4(qv[i], 0, h0, l0);
    split4(qv[i], 1, h1, l1);
    if (i < 16) {
      q.c_hi[i >> 2][2 * (i & 3)] = (int)h0;
      q.c_hi[i >> 2][2 * (i & 3) + 1] = (int)h1;
      q.c_lo[i >> 2][2 * (i & 3)] = (int)l0;
      q.c_lo[i >> 2][2 * (i & 3) + 1] = (int)l1;
    } else {
      q.r_hi[i - 16] = (long)(((uint64_t)h1 << 32) | h0);
      q.r_lo[i - 16] = (long)(((uint64_t)l1 << 32) | l0);
    }
  }
}

// S^T for this wave's 16 heads over the fp8 tile in buffer BUF, the softmax against the fixed
// references (as sp_scores) and the probabilities times the tokens' s_c into P buffer PB.
template <int BUF, int PB>
__device__ __forceinline__ void sp8_scores(const QFp8& q, SplitState& st, int t, int kv_len, float scale_log2, int w,
                                           int lane) {
  using namespace tiled8;
  const char* buf = kv8_buf<BUF>();
  asm volatile("" : "+v"(lane));
  const int g = lane >> 4, l16 = lane & 15;
  // ---- S^T = K Q^T per part: lane holds head l16, tokens 16 tb + 4 g + j.  The k split of a
  // 16x16x128 MFMA only has to match between its operands: lane group g gives 32 consecutive
  // dims of the chunk for both K (two 16-byte slots of the row) and Q.
  floatx4 scc[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
  floatx4 scr[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
  {
    const char* rows[2] = {buf + l16 * kRow, buf + (16 + l16) * kRow};
    const int sw[2] = {swz_lat(l16), swz_lat(16 + l16)};
    auto kfrag = [&](int kc, int tb) {
      const int ch = 8 * kc + 2 * g;
      const intx4 x = *reinterpret_cast<const intx4*>(rows[tb] + ((ch ^ sw[tb]) << 4));
      const intx4 y = *reinterpret_cast<const intx4*>(rows[tb] + (((ch + 1) ^ sw[tb]) << 4));
      return intx8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    };
    intx8 a[2];
    a[0] = kfrag(0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // (chunk, token block) = (i / 2, i % 2)
      if (i + 1 < 8) a[(i + 1) & 1] = kfrag((i + 1) >> 1, (i + 1) & 1);
      floatx4& acc = scc[i & 1];
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i & 1], q.c_hi[i >> 1], acc, 0, 0, 0, 127, 0, 127);
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i & 1], q.c_lo[i >> 1], acc, 0, 0, 0, 127, 0, 127);
    }
    // rope part: the k split of the two 16x16x32 MFMAs is again free as long as both operands
    // follow it: lane group g takes rope dims 16 g + 8 kr .. +7 in MFMA kr, so one 16-byte read of
    // chunk 32 + g serves both
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int r = 16 * tb + l16;
      const intx4 k16 = *reinterpret_cast<const intx4*>(rows[tb] + (((32 + g) ^ swz_rope(r)) << 4));
#pragma unroll
      for (int kr = 0; kr < 2; ++kr) {
        const long k8 = (long)(((uint64_t)(uint32_t)k16[2 * kr + 1] << 32) | (uint32_t)k16[2 * kr]);
        scr[tb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(k8, q.r_hi[kr], scr[tb], 0, 0, 0);
        scr[tb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(k8, q.r_lo[kr], scr[tb], 0, 0, 0);
      }
    }
  }
  // ---- per-token and per-head scales; softmax against the head's reference (masked past the
  // context on a partial tile)
  float lmax = -INFINITY;
  float s_lat[2][4];
  const bool full = (t + 1) * kT <= kv_len;
  const float qs = q.s * scale_log2;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const float4* sp = reinterpret_cast<const float4*>(buf + kCodes + (16 * tb + 4 * g) * 8);
    const float4 u0 = sp[0], u1 = sp[1];  // (s_c, s_r) of tokens +0 .. +3
    s_lat[tb][0] = u0.x;
    s_lat[tb][1] = u0.z;
    s_lat[tb][2] = u1.x;
    s_lat[tb][3] = u1.z;
    const float srs[4] = {u0.y, u0.w, u1.y, u1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = (s_lat[tb][j] * scc[tb][j] + srs[j] * scr[tb][j]) * qs;
      if (!full && t * kT + tb * 16 + 4 * g + j >= kv_len) v = -INFINITY;
      scc[tb][j] = v;
      lmax = fmaxf(lmax, v);
    }
  }
  bool restart = false;
  if (__builtin_amdgcn_ballot_w64(lmax > st.m_ref + sp::kHeadroom) != 0) {  // the first tile, or rare
    float hmax = wave_max_xor(lmax, 16);
    hmax = wave_max_xor(hmax, 32);
    if (__builtin_amdgcn_ballot_w64(st.m_ref != -INFINITY && lmax > st.m_ref + sp::kHeadroom) != 0) restart = true;
    st.m_ref = fmaxf(st.m_ref, hmax);
  }
  bf16x8 pf;  // slot s = token 16 (s/4) + 4g + s%4: the weight times the token's s_c
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = __builtin_amdgcn_exp2f(scc[tb][j] - st.m_ref);  // argument <= kHeadroom
      st.l_part += e;
      pf[tb * 4 + j] = (bf16)(e * fabsf(s_lat[tb][j]));
    }
  // the request: no product takes this value (a scale is never negative; taking its magnitude
  // keeps a corrupt negative one from posing as a request and restarting the partition forever)
  if (restart) pf[0] = (bf16)-1.f;
  *reinterpret_cast<bf16x8*>(pex_buf<PB>() + ((g * 128) + 16 * w + l16) * 16) = pf;
}

// O^T += V^T P^T for this wave's 64 latent dims and the head blocks present, over the tile in
// buffer BUF with the probabilities in P buffer PB.  Returns nonzero (the same in every wave) when
// one of those probabilities carries a restart request.
template <int BUF, int PB, bool FULL, bool F8>
__device__ __forceinline__ uint64_t sp_pv(SplitState& st, int nhb_rt, int w, int lane) {
  const int nhb = FULL ? 8 : nhb_rt;  // FULL: every head block of the group is present
  asm volatile("" : "+v"(lane));
  const int g = lane >> 4, l16 = lane & 15;
  Frag8<bf16> va[4];
  if constexpr (!F8) {
    using namespace tiled;
    const char* buf = kv_buf<BUF>();
    // V^T fragments of dim blocks 4w .. 4w+3 (16 dims x 32 tokens each): lane group g reads tokens
    // 4g + s/4 (+16 for the second read); source lane s supplies dims 16 d + 4 (s % 4) .. +3 = chunk
    // 2d + (s%4)/2, byte (s % 2) * 8 of its token row, stored at slot chunk ^ (token & 7)
    const int x = (4 * g + (l16 >> 2)) & 7;
    const int clo = (l16 & 3) >> 1;
    const char* row = buf + (4 * g + (l16 >> 2)) * kRow + (l16 & 1) * 8;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const char* pv = row + ((2 * (4 * w + db) + clo) ^ x) * 16;
      const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)pv);
      const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(pv + 16 * kRow));
      va[db].v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  } else {
    using namespace tiled8;
    const char* buf = kv8_buf<BUF>();
    // one 8-bit transpose read per dim block: lane (g, l16) supplies dims 8 (l16 % 2) .. +7 of the
    // 16-byte piece of token 16 (l16 / 8) + 4g + (l16 / 2) % 4, the token of probability slot
    // l16 / 2, so lane i of group g receives dim i of exactly the tokens its P fragment holds; the
    // codes (exact in bf16) are converted in registers, the token's s_c being folded into P
    const int tok = 16 * (l16 >> 3) + 4 * g + ((l16 >> 1) & 3);
    const int sw = swz_lat(tok);
    const char* row = buf + tok * kRow + 8 * (l16 & 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const intx2 c8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2_t*)(row + 16 * ((4 * w + db) ^ sw)));
      const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8[0], 1.f, false);
      const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8[0], 1.f, true);
      const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8[1], 1.f, false);
      const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8[1], 1.f, true);
      va[db].v = bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
  }
  // P^T fragments four head blocks at a time (the scheduler barrier keeps the second group's reads
  // from being hoisted, which would need registers the queries and O occupy)
  const char* pb = pex_buf<PB>() + (g * 128 + l16) * 16;
  bool req = false;  // a fragment's first value is the request value
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
    Frag8<bf16> pf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (FULL || 4 * hq + i < nhb) pf[i].v = *reinterpret_cast<const bf16x8*>(pb + 256 * (4 * hq + i));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (FULL || 4 * hq + i < nhb) {
#pragma unroll
        for (int db = 0; db < 4; ++db) st.o[db][4 * hq + i] = mma16(va[db], pf[i], st.o[db][4 * hq + i]);
        req |= ((uint32_t)__builtin_bit_cast(intx4, pf[i].v)[0] & 0xFFFFu) == 0xBF80u;
      }
    __builtin_amdgcn_sched_barrier(0);
  }
  return __builtin_amdgcn_ballot_w64(req);
}

// Waits until this wave's copies of the next tile have landed, with those of the one after it (issued
// at the end of this phase) still in flight (waves 0-3 issue nine copies per tile, 4-7 none), and
// until its LDS writes (the probabilities it publishes) have completed; then the workgroup barrier.
template <bool F8>
__device__ __forceinline__ void sp_barrier_next(int w) {
  if constexpr (!F8) {
    if (w < 4) MLA_TILE_BARRIER(waitcnt_vm_lgkm0(tiled::kDmaPerWave));
    else MLA_TILE_BARRIER(waitcnt_vm_lgkm0(0));
  } else {
    if (w < 3) MLA_TILE_BARRIER(waitcnt_vm_lgkm0(tiled8::kDmaPerWave));
    else if (w == 3) MLA_TILE_BARRIER(waitcnt_vm_lgkm0(tiled8::kDmaPerWave - 1));
    else MLA_TILE_BARRIER(waitcnt_vm_lgkm0(0));
  }
}

// The phase of tile t (buffer B = (t - t_begin) % 4; t == t_end: only tile t-1's P.V): P.V of tile
// t-1, S of tile t, then the copies of tile t+2 into the buffer tile t-2 left.  The copies go out
// at the end of the phase: the copying waves (0-3) finish their products before the others, which
// share their SIMDs, so the issue overlaps the others' last products instead of delaying the
// copying waves' first ones (measured: 174.5 against 177.0 us); tile t+2 still has a whole phase
// to land.  Returns nonzero, the same in every wave, when tile t-1's probabilities carry a restart
// request.
template <int B, bool FULL, bool F8, typename QT>
__device__ __forceinline__ uint64_t sp_phase(const TiledCtx& c, const QT& q, SplitState& st, int t, int t_end,
                                             float scale_log2, bool s_wave, int nhb, int w, int lane) {
  using namespace tiled;
  constexpr int BPREV = (B + 3) % kNBuf, BNEXT2 = (B + 2) % kNBuf;
  const uint64_t req = sp_pv<BPREV, (B + 1) & 1, FULL, F8>(st, nhb, w, lane);
  if constexpr (F8) {
    if (t < t_end && s_wave) sp8_scores<B, B & 1>(q, st, t, c.kv_len, scale_log2, w, lane);
    issue_tile8<BNEXT2>(c, t + 2, t + 2 < t_end, w, lane);
  } else {
    if (t < t_end) sp_scores_wave<B, B & 1>(q.v, st, t, c.kv_len, scale_log2, s_wave, w, lane);
    issue_tile<BNEXT2>(c, t + 2, t + 2 < t_end, w, lane);
  }
  sp_barrier_next<F8>(w);
  return req;
}

template <bool FULL, bool F8>
__global__ void __launch_bounds__(512)
    decode_attn_tiled_kernel(DecodeAttnParams p, int HG, const int32_t* __restrict__ block_table) {
  using namespace tiled;
  // block id -> (unit = (sequence, partition), head group): the HG head groups of a unit sit 8
  // ids apart, i.e. on the same XCD (ids are dealt to the 8 XCDs round robin)
  const int units = p.B * p.splits + (p.units ? p.B : 0);
  const int grp = blockIdx.x / (8 * HG), rem = blockIdx.x % (8 * HG);
  const int hg = rem / 8, unit = grp * 8 + rem % 8;
  if (unit >= units) return;
  int b, split, t_begin, t_end;
  if (p.units) {  // the balanced table: (sequence, partition slot, first tile, end tile)
    const int4 ue = p.units[unit];
    if (ue.x < 0) return;
    b = ue.x, split = ue.y, t_begin = ue.z, t_end = ue.w;
  } else {  // fixed partitions of tokens_per_split
    b = unit / p.splits, split = unit % p.splits;
    const int ntiles = (p.lens[b] + (p.lens_plus_one ? 1 : 0) + kT - 1) / kT;
    t_begin = split * (p.tokens_per_split / kT);
    t_end = min(ntiles, t_begin + p.tokens_per_split / kT);
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int h0 = hg * (16 * kWaves);                    // the head group's first head
  const int nhb = min(kWaves, (p.n_h - h0 + 15) / 16);  // its 16-head blocks
  const bool s_wave = w < nhb;                          // this wave computes S for heads h0 + 16w ..
  const int head = h0 + w * 16 + l16;
  const bool valid_head = head < p.n_h;
  const bool partial = p.splits > 1 || p.leave_partials;  // else o_hat (and lse) directly

  if (t_begin >= t_end) {  // an empty partition: only its max (-inf), which the combines skip
    if (s_wave && valid_head && g == 0 && partial) {
      const int64_t pi = ((int64_t)b * p.splits + split) * p.n_h + head;
      p.part_m[pi] = -INFINITY;
      p.part_l[pi] = 0.f;
    }
    return;
  }

  TiledCtx c;
  c.pool = reinterpret_cast<const char*>(p.pool);
  c.scales = p.scales;
  c.bt = block_table + (int64_t)b * p.max_blocks;  // read-only: block ids load as scalars
  c.bs = p.block_size;
  c.kv_len = p.lens[b] + (p.lens_plus_one ? 1 : 0);
  if constexpr (!F8) {
    // copy i of this wave moves 16 bytes P = 64 (first + i) + lane of the tile: chunk P % 72 of
    // row P / 72, from its swizzled source slot; the offsets (< 36864) are worked out once
#pragma unroll
    for (int k = 0; k < 5; ++k) c.dma_off[k] = 0;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int P = (kDmaPerWave * w + i) * 64 + lane;
      const int tr = P / kCPR;
      const uint32_t off = (uint32_t)(tr * kRow + ((P - tr * kCPR) ^ (tr & 7)) * 16);
      c.dma_off[i >> 1] |= off << (16 * (i & 1));
    }
  } else {
    // fp8 tiles: copy i of this wave (P = 5w + i) moves bytes 1024 P + 16 lane of the tile's codes
    // from their swizzled source slot, or (P = 18) the lane's 4 bytes of scales
#pragma unroll
    for (int k = 0; k < 3; ++k) c.dma_off[k] = 0;
#pragma unroll
    for (int i = 0; i < tiled8::kDmaPerWave; ++i) {
      const int P = tiled8::kDmaPerWave * w + i;
      const int byte = P * 1024 + lane * 16;
      const int tr = byte / tiled8::kRow, sl = (byte - tr * tiled8::kRow) >> 4;
      const uint32_t off =
          P < tiled8::kCodeCopies
              ? (uint32_t)(tr * tiled8::kRow + ((sl ^ (sl < 32 ? tiled8::swz_lat(tr) : tiled8::swz_rope(tr))) << 4))
              : (uint32_t)(lane * 4);
      c.dma_off[i >> 1] |= off << (16 * (i & 1));
    }
  }

  std::conditional_t<F8, QFp8, QBf16> q;
  {
    const bf16* qrow = reinterpret_cast<const bf16*>(p.q) + ((int64_t)b * p.n_h + (valid_head ? head : 0)) * kD;
    if constexpr (F8) {
      load_q_fp8(q, qrow, s_wave && valid_head, g);
    } else {
#pragma unroll
      for (int kc = 0; kc < 18; ++kc) {
        if (s_wave && valid_head) load8(q.v[kc], qrow + kc * 32 + 8 * g);
        else zero8(q.v[kc]);
      }
    }
  }
  SplitState st;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) st.o[db][hb] = floatx4{0, 0, 0, 0};
  st.m_ref = -INFINITY;
  st.l_part = 0.f;
  // the queries first: with them still in flight the compiler would wait for every copy of the
  // ring before the first tile
  MLA_WAVE_WAIT(waitcnt_vm(0));

  int t = t_begin;
  while (t <= t_end) {
    if (t == t_begin) {  // (re)start: tiles t_begin .. t_begin + 2 into buffers 0 .. 2, then S of the first
      if constexpr (F8) {
        issue_tile8<0>(c, t_begin, true, w, lane);
        issue_tile8<1>(c, t_begin + 1, t_begin + 1 < t_end, w, lane);
        issue_tile8<2>(c, t_begin + 2, t_begin + 2 < t_end, w, lane);
        if (w < 3) MLA_TILE_BARRIER(waitcnt_vm(2 * tiled8::kDmaPerWave));  // the first tile landed
        else if (w == 3) MLA_TILE_BARRIER(waitcnt_vm(2 * (tiled8::kDmaPerWave - 1)));
        else MLA_TILE_BARRIER(waitcnt_vm(0));
        if (s_wave) sp8_scores<0, 0>(q, st, t_begin, c.kv_len, p.scale_log2, w, lane);
      } else {
        issue_tile<0>(c, t_begin, true, w, lane);
        issue_tile<1>(c, t_begin + 1, t_begin + 1 < t_end, w, lane);
        issue_tile<2>(c, t_begin + 2, t_begin + 2 < t_end, w, lane);
        if (w < 4) MLA_TILE_BARRIER(waitcnt_vm(2 * kDmaPerWave));  // the first tile landed
        else MLA_TILE_BARRIER(waitcnt_vm(0));
        sp_scores_wave<0, 0>(q.v, st, t_begin, c.kv_len, p.scale_log2, s_wave, w, lane);
      }
      sp_barrier_next<F8>(w);
      t = t_begin + 1;
    }
    uint64_t fl = sp_phase<1, FULL, F8>(c, q, st, t, t_end, p.scale_log2, s_wave, nhb, w, lane);
    if (fl == 0 && t + 1 <= t_end) fl = sp_phase<2, FULL, F8>(c, q, st, t + 1, t_end, p.scale_log2, s_wave, nhb, w, lane);
    if (fl == 0 && t + 2 <= t_end) fl = sp_phase<3, FULL, F8>(c, q, st, t + 2, t_end, p.scale_log2, s_wave, nhb, w, lane);
    if (fl == 0 && t + 3 <= t_end) fl = sp_phase<0, FULL, F8>(c, q, st, t + 3, t_end, p.scale_log2, s_wave, nhb, w, lane);
    if (fl == 0) {
      t += kNBuf;
      continue;
    }
    // a reference was raised: start over from the first tile, keeping the raised references
    MLA_WAVE_WAIT(waitcnt_vm(0));
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int hb = 0; hb < 8; ++hb) st.o[db][hb] = floatx4{0, 0, 0, 0};
    st.l_part = 0.f;
    MLA_TILE_BARRIER(kWaitLgkm0);
    t = t_begin;
  }
  // the copies past the partition (reading nothing) must land before the LDS is released
  MLA_WAVE_WAIT(waitcnt_vm(0));
  // the four lane groups of a head hold partial sums over different tokens
  float l_run = wave_sum_xor(st.l_part, 16);
  l_run = wave_sum_xor(l_run, 32);
  const float m_run = st.m_ref;
  MLA_TILE_BARRIER(kWaitLgkm0);  // every wave is done with the last probabilities
  float* inv_l = reinterpret_cast<float*>(g_pex0);  // [head - h0]: 1 / l
  if (s_wave && g == 0) inv_l[16 * w + l16] = l_run > 0.f ? 1.f / l_run : 0.f;
  if (s_wave && valid_head && g == 0) {
    if (!partial) {
      if (p.lse) p.lse[(int64_t)b * p.n_h + head] = (m_run + log2f(l_run)) * 0.69314718055994531f;
    } else {
      const int64_t pi = ((int64_t)b * p.splits + split) * p.n_h + head;
      p.part_m[pi] = m_run;
      p.part_l[pi] = l_run;
    }
  }
  MLA_TILE_BARRIER(kWaitLgkm0);
  // the normalised rows O / l (with several partitions, the partition's own O_s / l_s: a convex
  // combination of latent values, stored in bf16 for half the partial traffic of fp32)
#pragma unroll
  for (int hb = 0; hb < 8; ++hb) {
    const int hh = h0 + 16 * hb + l16;
    if (hb < nhb && hh < p.n_h) {
      const float inv = inv_l[16 * hb + l16];
      bf16* out = !partial
                      ? reinterpret_cast<bf16*>(p.o_hat) + ((int64_t)b * p.n_h + hh) * kDC
                      : reinterpret_cast<bf16*>(p.part_o) + (((int64_t)b * p.splits + split) * p.n_h + hh) * kDC;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (bf16)(st.o[db][hb][r] * inv);
        *reinterpret_cast<bf16x4*>(out + 16 * (4 * w + db) + 4 * g) = v;
      }
    }
  }
}

// Log-sum-exp combination of the partitions: M = max_s m_s, w_s = 2^(m_s - M) l_s,
// o_hat = sum_s w_s o_s / sum_s w_s with o_s = O_s / l_s the partition's normalised output (PT:
// fp32 or bf16).  A 256-thread workgroup combines four (sequence, head) rows, one wave each;
// each lane owns DC/64 consecutive latent dims.  Empty partitions (max -inf) are skipped.
template <typename T, typename PT, int DC, bool COOP>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeAttnParams p) {
  constexpr int V = DC >= 64 ? DC / 64 : 1;  // dims per thread
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // b * n_h + head: one wave per row, or (COOP, many partitions) one workgroup per row, its four
  // waves taking every fourth group of partitions and adding up in LDS
  const int bh = COOP ? blockIdx.x : blockIdx.x * 4 + wv;
  if (bh >= p.B * p.n_h) return;
  const int lane = threadIdx.x & 63;
  const bool has_dims = V * lane < DC;
  const int b = bh / p.n_h, head = bh % p.n_h;
  const int64_t base = (int64_t)b * p.splits * p.n_h + head;  // partition s at base + s * n_h
  const int d = V * lane;
  // Two memory round trips: every partition's (max, normaliser), two per lane (partitions lane and
  // 64 + lane; beyond 128 read where needed; M by a wave reduction), then the output rows of the
  // non-empty partitions of two groups of kG at once.  With COOP the four waves take the groups in
  // turn (wave w: groups w, w + 4, ...); alone, a wave takes them all, in order.
  constexpr int kG = 8, NWv = COOP ? 4 : 1;
  const int w = COOP ? wv : 0;
  const int S = p.splits;
  float m2[2], l2[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sp = 64 * j + lane;
    m2[j] = sp < S ? p.part_m[base + (int64_t)sp * p.n_h] : -INFINITY;
    l2[j] = sp < S ? p.part_l[base + (int64_t)sp * p.n_h] : 0.f;
  }
  float M = fmaxf(m2[0], m2[1]);
  for (int c = 128; c < S; c += 64)
    if (c + lane < S) M = fmaxf(M, p.part_m[base + (int64_t)(c + lane) * p.n_h]);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  float L = 0.f;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  for (int s0 = kG * w; s0 < S; s0 += 2 * kG * NWv) {
    float ms[2][kG], ls[2][kG];
    PT v[2][kG][V];
    // a group lies wholly below partition 128 (values from the lanes that hold them) or wholly
    // above it (read here): one path per group, so that no row load waits on another
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int g0 = s0 + q * kG * NWv;  // the same in every lane
      if (g0 < 128) {
#pragma unroll
        for (int u = 0; u < kG; ++u) {
          ms[q][u] = lane_value(g0 < 64 ? m2[0] : m2[1], (g0 + u) & 63);
          ls[q][u] = lane_value(g0 < 64 ? l2[0] : l2[1], (g0 + u) & 63);
        }
      } else {
#pragma unroll
        for (int u = 0; u < kG; ++u) {
          ms[q][u] = g0 + u < S ? p.part_m[base + (int64_t)(g0 + u) * p.n_h] : -INFINITY;
          ls[q][u] = g0 + u < S ? p.part_l[base + (int64_t)(g0 + u) * p.n_h] : 0.f;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int u = 0; u < kG; ++u)
        if (ms[q][u] > -INFINITY) {  // (-inf past the last partition too)
          const PT* src =
              reinterpret_cast<const PT*>(p.part_o) + (base + (int64_t)(s0 + q * kG * NWv + u) * p.n_h) * DC + d;
#pragma unroll
          for (int i = 0; i < V; ++i) v[q][u][i] = has_dims ? src[i] : PT(0.f);
        }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int u = 0; u < kG; ++u)
        if (ms[q][u] > -INFINITY) {
          const float ws = exp2f(ms[q][u] - M) * ls[q][u];
          L += ws;
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] += ws * to_f32(v[q][u][i]);
        }
  }
  if constexpr (COOP) {
    __shared__ float red[4][V + 1][64];
#pragma unroll
    for (int i = 0; i < V; ++i) red[wv][i][lane] = acc[i];
    red[wv][V][lane] = L;
    __syncthreads();
    if (wv != 0) return;
    L = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (int w2 = 0; w2 < 4; ++w2) {
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += red[w2][i][lane];
      L += red[w2][V][lane];
    }
  }
  if (!has_dims) return;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  T* out = reinterpret_cast<T*>(p.o_hat) + (int64_t)bh * DC + d;
#pragma unroll
  for (int i = 0; i < V; ++i) out[i] = from_f32<T>(acc[i] * inv);
  if (p.lse && d == 0) p.lse[bh] = (M + log2f(L)) * 0.69314718055994531f;
}

// ----------------------------------------------------------------------------- host side
bool decode_tiled(DType t, int d_c, int d_hr, int block_size) {
  return t == DType::BF16 && d_c == 512 && d_hr == 64 && block_size % tiled::kT == 0;
}



static int v1_heads_per_block(int n_h) { return n_h >= 128 ? 128 : (n_h >= 64 ? 64 : 16); }

bool decode_supported(int d_c, int d_hr) { return (d_c == 512 && d_hr == 64) || (d_c == 32 && d_hr == 8); }

namespace {
template <typename T, int DC, int DR>
hipError_t launch(const DecodeAttnParams& p, hipStream_t s) {
  const int hpb = v1_heads_per_block(p.n_h);
  const int HG = (p.n_h + hpb - 1) / hpb;
  const int units = p.B * p.splits;
  const int blocks = (units + 7) / 8 * 8 * HG;
  if (units == 0) return hipSuccess;
  switch (hpb) {
    case 128: hipLaunchKernelGGL((decode_attn_kernel<T, DC, DR, 8>), dim3(blocks), dim3(512), 0, s, p, HG); break;
    case 64: hipLaunchKernelGGL((decode_attn_kernel<T, DC, DR, 4>), dim3(blocks), dim3(256), 0, s, p, HG); break;
    default: hipLaunchKernelGGL((decode_attn_kernel<T, DC, DR, 1>), dim3(blocks), dim3(64), 0, s, p, HG); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  if (p.splits >= 16)
    hipLaunchKernelGGL((decode_combine_kernel<T, float, DC, true>), dim3(p.B * p.n_h), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((decode_combine_kernel<T, float, DC, false>), dim3((p.B * p.n_h + 3) / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}
}  // namespace

bool decode_bf16_partials(DType t, const DecodeAttnParams& p) {
  return p.fp8 || decode_tiled(t, p.d_c, p.d_hr, p.block_size);
}

hipError_t decode_attention(DType t, const DecodeAttnParams& p, hipStream_t s) {
  if (p.leave_partials && !decode_bf16_partials(t, p)) return hipErrorInvalidValue;
  if (p.fp8 && !(t == DType::BF16 && p.d_c == 512 && p.d_hr == 64 && p.block_size % tiled8::kT == 0 && p.scales))
    return hipErrorInvalidValue;
  if (p.fp8 || decode_tiled(t, p.d_c, p.d_hr, p.block_size)) {
    const int HG = (p.n_h + 16 * tiled::kWaves - 1) / (16 * tiled::kWaves);
    if (p.B == 0) return hipSuccess;
    if (p.units && p.B > 64) return hipErrorInvalidValue;  // the table builder takes B <= 64
    if (p.units && !p.units_ready) hipLaunchKernelGGL(decode_units_kernel, dim3(1), dim3(256), 0, s, p);
    const int units = p.B * p.splits + (p.units ? p.B : 0);  // with a table: + B idle entries
    const int blocks = (units + 7) / 8 * 8 * HG;
    const bool full = p.n_h % (16 * tiled::kWaves) == 0;  // every head group full: the P.V loop needs no guards
    const dim3 grid(blocks), block(64 * tiled::kWaves);
    if (p.fp8) {
      if (full) hipLaunchKernelGGL((decode_attn_tiled_kernel<true, true>), grid, block, 0, s, p, HG, p.block_table);
      else hipLaunchKernelGGL((decode_attn_tiled_kernel<false, true>), grid, block, 0, s, p, HG, p.block_table);
    } else {
      if (full) hipLaunchKernelGGL((decode_attn_tiled_kernel<true, false>), grid, block, 0, s, p, HG, p.block_table);
      else hipLaunchKernelGGL((decode_attn_tiled_kernel<false, false>), grid, block, 0, s, p, HG, p.block_table);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1 || p.leave_partials) return e;
    if (p.splits >= 16)
      hipLaunchKernelGGL((decode_combine_kernel<bf16, bf16, 512, true>), dim3(p.B * p.n_h), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((decode_combine_kernel<bf16, bf16, 512, false>), dim3((p.B * p.n_h + 3) / 4), dim3(256), 0,
                         s, p);
    return hipGetLastError();
  }
  if (p.d_c == 512 && p.d_hr == 64)
    return t == DType::BF16 ? launch<bf16, 512, 64>(p, s) : launch<float, 512, 64>(p, s);
  if (p.d_c == 32 && p.d_hr == 8)
    return t == DType::BF16 ? launch<bf16, 32, 8>(p, s) : launch<float, 32, 8>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
