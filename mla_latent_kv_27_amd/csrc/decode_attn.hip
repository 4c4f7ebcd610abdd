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

#include "common.h"
#include "internal.h"

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
// Work units of the tiled kernels for small batches, where contexts of different lengths would
// leave most fixed-length partitions of the short sequences empty.  Each sequence has p.splits
// partition slots; sequence b takes n_b = ceil(tiles_b / tps) of them.  tps starts at the
// shortest length that fits the longest sequence in its slots and is raised while that lowers
// the finish time, counted in rounds of p.cus units (one per compute unit) times tps.  The table
// lists the partitions in sequence order, then the slots no partition uses (p >= n_b: they get
// an empty partial, max -inf and no output rows), then B idle units: (b, p, first tile, end
// tile), b = -1 when idle.  One workgroup builds it from the lengths in device memory (B <= 64),
// so the host needs only B and splits.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

__global__ void __launch_bounds__(256) decode_units_kernel(DecodeAttnParams p) {
  const int lane = threadIdx.x & 63;
  const int plus = p.lens_plus_one ? 1 : 0, S = p.splits, T = kTile;
  const int C = max(1, p.cus);
  // one lane per sequence (B <= 64)
  const int my_tiles = lane < p.B ? (p.lens[lane] + plus + T - 1) / T : 0;
  const int tot = wave_sum_int(my_tiles);
  int mx = my_tiles;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = max(mx, __shfl_xor(mx, d, 64));
  // partition length: the shortest one that fits every sequence in its S slots, or a longer one
  // when that finishes sooner; the finish time counts rounds of C units (one per compute unit)
  const int tmin = max(1, (mx + S - 1) / S);
  int tps = tmin;
  long best = -1;
  for (int k = 0; k <= 9; ++k) {
    const int cand = k < 9 ? tmin + tmin * k / 8 : max(tmin, (tot + C - 1) / C);
    const int used = wave_sum_int((my_tiles + cand - 1) / cand);
    const long cost = (long)((used + C - 1) / C) * cand;
    if (best < 0 || cost < best) {
      best = cost;
      tps = cand;
    }
  }
  // per-sequence partition counts and their prefix sums (B <= 64 here), then every thread fills
  // table entries
  __shared__ int s_tiles[64], s_pend[64], s_fend[64];  // tiles, partitions / free slots up to b
  if (threadIdx.x < 64) {
    const int tiles = my_tiles;
    const int n = lane < p.B ? (tiles + tps - 1) / tps : 0;
    s_tiles[lane] = tiles;
    s_pend[lane] = wave_incl_scan(n, lane);
    s_fend[lane] = wave_incl_scan(lane < p.B ? S - n : 0, lane);
  }
  __syncthreads();
  const int np = s_pend[p.B - 1];
  for (int j = threadIdx.x; j < p.B * S + p.B; j += blockDim.x) {
    int4 e = make_int4(-1, 0, 0, 0);
    if (j < np) {
      int i = 0;
      while (s_pend[i] <= j) ++i;
      const int k = j - (i ? s_pend[i - 1] : 0);
      e = make_int4(i, k, k * tps, min(s_tiles[i], (k + 1) * tps));
    } else if (j < p.B * S) {
      const int f = j - np;
      int i = 0;
      while (s_fend[i] <= f) ++i;
      const int n_i = s_pend[i] - (i ? s_pend[i - 1] : 0);
      e = make_int4(i, n_i + f - (i ? s_fend[i - 1] : 0), 0, 0);
    }
    p.units[j] = e;
  }
}

// ----------------------------------------------------------------------------- tiled kernel
// The DeepSeek-V2-sized bf16 case (d_c = 512, d_hr = 64).  A workgroup is eight waves of 16 heads
// (two waves per SIMD hide each other's LDS and copy latency); with more than 128 heads the other
// head groups' workgroups read the same tiles and get block ids on the same XCD, so their repeat
// reads come from its L2.
//   * Tiles of 32 tokens arrive by direct global->LDS copies into a ring of four buffers, three
//     tiles ahead of the one being multiplied.
//   * LDS row of a token = its 1152-byte cache entry as 72 16-byte chunks; chunk c of token t is
//     stored at chunk slot t*72 + (c ^ (t & 7)) so that the 16 tokens of an MFMA operand read
//     fall on different banks.
//   * S^T = K Q^T with 16x16x32 MFMA: A = 16 tokens x 32 latent dims (ds_read_b128),
//     B = Q^T held in registers for the whole kernel (18 k-chunks x 8 values).
//   * O^T = V^T P^T: the A operand (16 latent dims x 32 tokens) is read straight from the
//     token-major tile with the gfx950 LDS transpose read (ds_read_b64_tr_b16): within each
//     16-lane group, source lane s supplies 4 consecutive dims of token 4j + s/4 and lane i
//     receives dim i of those four tokens.
//   * Softmax scaling is lazy: all lanes of a head share a reference max that is only raised (and
//     O rescaled) when some score exceeds it by more than 2^8, so the common tile needs no
//     cross-lane exchange; every lane keeps a partial sum that is combined once at the end.
namespace tiled {
constexpr int kT = 32;                    // tokens per tile
constexpr int kNBuf = 4;                  // ring buffers (two tile pairs)
constexpr int kD = 576, kDC = 512;        // entry width, latent width
constexpr int kCPR = kD * 2 / 16;         // 72 chunks per entry
constexpr int kRow = kCPR * 16;           // 1152 bytes per entry
constexpr int kBytes = kT * kRow;         // 36864 per buffer
constexpr int kWaves = 8;
constexpr int kDmaTotal = kT * kCPR / 64;  // 36 one-KiB copies per tile: waves 0-3 issue 5, 4-7 issue 4
__device__ __forceinline__ int dma_count(int w) { return w < 4 ? 5 : 4; }
__device__ __forceinline__ int dma_first(int w) { return w < 4 ? 5 * w : 20 + 4 * (w - 4); }
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
  const int32_t* bt;
  int bs, kv_len;
};

// This wave's share (5 or 4) of the 36 direct-to-LDS copies of tile `tile` into buffer BUF.  block_size is a multiple
// of the tile size, so a tile lies inside one block: one uniform block-table lookup, and every row copied
// is a row of an allocated block (rows past the context are zeroed once the copies land).
template <int BUF>
__device__ __forceinline__ void issue_tile(const TiledCtx& c, int tile, int w, int lane) {
  using namespace tiled;
  char* dst = kv_buf<BUF>();
  const int tok0 = tile * kT;
  const int blk = tok0 / c.bs;
  const char* base = c.pool + ((int64_t)c.bt[blk] * c.bs + (tok0 - blk * c.bs)) * kRow;
  int ln = lane;
  asm volatile("" : "+v"(ln));  // recompute the lane offsets here instead of keeping them live
  const int first = dma_first(w), cnt = dma_count(w);
  const __amdgpu_buffer_rsrc_t span = dma_span(base, kBytes);  // the tile: 32 consecutive rows
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    if (i < cnt) {
      const int P = (first + i) * 64 + ln;
      const int t = P / kCPR;
      const int ch = (P - t * kCPR) ^ (t & 7);
      dma16(span, t * kRow + ch * 16, (lds_void_t*)(dst + (first + i) * 1024));
    }
  }
}

struct TiledState {
  floatx4 o[32];   // O^T: 32 blocks of 16 latent dims; lane: head l16, dims 16 d + 4 g + j
  float m_ref;     // shared reference max of this lane's head (log2 domain)
  float l_part;    // this lane's partial normaliser
};

// O^T += V^T P^T over the 32 tokens of the bf16 tile in buffer BUF (rows of 1152 bytes, chunk c of
// row r at slot c ^ (r & 7)); pf holds P for the lane's head, slot s = token 16 (s/4) + 4g + s%4.
template <int BUF>
__device__ __forceinline__ void tiled_pv(TiledState& st, const Frag8<bf16>& pf, int lane) {
  using namespace tiled;
  const char* buf = kv_buf<BUF>();
  const int g = lane >> 4, l16 = lane & 15;
  // O^T += V^T P^T : 32 blocks of 16 latent dims over the tile's 32 tokens
  // lane group g reads tokens 4g + s/4 (+16 for the second read); source lane s supplies dims
  // 16 d + 4 (s % 4) .. +3 = chunk 2d + (s%4)/2, byte (s % 2) * 8
  const int x = (4 * g + (l16 >> 2)) & 7;
  const int clo = (l16 & 3) >> 1;
  const char* vb[4];
#pragma unroll
  for (int par = 0; par < 4; ++par)
    vb[par] = buf + (4 * g + (l16 >> 2)) * kRow + (l16 & 1) * 8 + ((2 * par + clo) ^ x) * 16;
  shortx4 vlo[3], vhi[3];  // fragments two blocks ahead are in flight
#pragma unroll
  for (int d0 = 0; d0 < 2; ++d0) {
    vlo[d0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)vb[d0]);
    vhi[d0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(vb[d0] + 16 * kRow));
  }
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    if (d + 2 < 32) {
      const char* pv = vb[(d + 2) & 3] + 128 * ((d + 2) >> 2);
      vlo[(d + 2) % 3] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)pv);
      vhi[(d + 2) % 3] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(pv + 16 * kRow));
    }
    Frag8<bf16> a;
    a.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[d % 3], vhi[d % 3], 0, 1, 2, 3, 4, 5, 6, 7));
    st.o[d] = mma16(a, pf, st.o[d]);
  }
}

template <int BUF>
__device__ __forceinline__ void tiled_compute(const Frag8<bf16> (&q)[18], TiledState& st, int t, int kv_len,
                                              float scale_log2, int lane) {
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
    Frag8<bf16> a[3][2];  // [stage][tb]: fragments two k-chunks ahead are in flight
#pragma unroll
    for (int k0 = 0; k0 < 2; ++k0) {
      const char* pn = (k0 & 1 ? rb1 : rb0);
      a[k0][0].v = *reinterpret_cast<const bf16x8*>(pn);
      a[k0][1].v = *reinterpret_cast<const bf16x8*>(pn + 16 * kRow);
    }
#pragma unroll
    for (int kc = 0; kc < 18; ++kc) {
      if (kc + 2 < 18) {
        const char* pn = ((kc + 2) & 1 ? rb1 : rb0) + 128 * ((kc + 2) >> 1);
        a[(kc + 2) % 3][0].v = *reinterpret_cast<const bf16x8*>(pn);
        a[(kc + 2) % 3][1].v = *reinterpret_cast<const bf16x8*>(pn + 16 * kRow);
      }
      sc[0] = mma16(a[kc % 3][0], q[kc], sc[0]);
      sc[1] = mma16(a[kc % 3][1], q[kc], sc[1]);
    }
  }
  // ---- lazy online softmax
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
  if (__builtin_amdgcn_ballot_w64(lmax > st.m_ref + kLazy) != 0) {  // rare: raise the reference
    float hmax = wave_max_xor(lmax, 16);
    hmax = wave_max_xor(hmax, 32);
    const float m_new = fmaxf(st.m_ref, hmax);
    const float alpha = __builtin_amdgcn_exp2f(st.m_ref - m_new);  // -inf -> 0
    st.l_part *= alpha;
#pragma unroll
    for (int d = 0; d < 32; ++d) st.o[d] *= alpha;
    st.m_ref = m_new;
  }
  Frag8<bf16> pf;  // slot s = token 16 (s/4) + 4g + s%4
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16 e = (bf16)__builtin_amdgcn_exp2f(sc[tb][j] - st.m_ref);  // argument <= 8
      st.l_part += (float)e;
      pf.v[tb * 4 + j] = e;
    }
  tiled_pv<BUF>(st, pf, lane);
}

// Two tiles per barrier: tiles t and t+1 sit in ring buffers B0 and B0+1 (B0 = 0 or 2), and the
// only copies in flight are theirs.  Once they have landed and every wave is past the previous
// pair, the copies of tiles t+2 and t+3 go into the other two buffers, then both tiles are
// multiplied.  Half as many workgroup barriers as one per tile, and no pipeline drain between the
// two tiles of a pair.
template <int B0>
__device__ __forceinline__ void tiled_pair(const TiledCtx& c, const Frag8<bf16> (&q)[18], TiledState& st, int t,
                                           int t_end, float scale_log2, int w, int lane, int tid) {
  using namespace tiled;
  MLA_TILE_BARRIER(waitcnt_vm(0));
  if (t + 2 < t_end) issue_tile<(B0 + 2) % kNBuf>(c, t + 2, w, lane);
  if (t + 3 < t_end) issue_tile<(B0 + 3) % kNBuf>(c, t + 3, w, lane);
  const int last = min(t + 1, t_end - 1);  // only the sequence's last tile can be partial
  const int valid = c.kv_len - last * kT;
  if (valid < kT) {  // zero the rows past the end of the context (uniform branch)
    char* buf = last == t ? kv_buf<B0>() : kv_buf<B0 + 1>();
    for (int i = tid; i < (kT - valid) * kCPR; i += 64 * kWaves) st16(buf + (valid * kCPR + i) * 16, zero16());
    MLA_TILE_BARRIER(kWaitLgkm0);
  }
  tiled_compute<B0>(q, st, t, c.kv_len, scale_log2, lane);
  if (t + 1 < t_end) tiled_compute<B0 + 1>(q, st, t + 1, c.kv_len, scale_log2, lane);
}

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
  const int g = lane >> 4;
  const int head = hg * (16 * kWaves) + w * 16 + (lane & 15);
  const bool valid_head = head < p.n_h;

  TiledCtx c;
  c.pool = reinterpret_cast<const char*>(p.pool);
  c.bt = block_table + (int64_t)b * p.max_blocks;  // read-only: block ids load as scalars
  c.bs = p.block_size;
  c.kv_len = p.lens[b] + (p.lens_plus_one ? 1 : 0);

  Frag8<bf16> q[18];
  {
    const bf16* qrow = reinterpret_cast<const bf16*>(p.q) + ((int64_t)b * p.n_h + (valid_head ? head : 0)) * kD;
#pragma unroll
    for (int kc = 0; kc < 18; ++kc) {
      if (valid_head) load8(q[kc], qrow + kc * 32 + 8 * g);
      else zero8(q[kc]);
    }
  }
  TiledState st;
#pragma unroll
  for (int d = 0; d < 32; ++d) st.o[d] = floatx4{0, 0, 0, 0};
  st.m_ref = -INFINITY;
  st.l_part = 0.f;

  if (t_begin < t_end) issue_tile<0>(c, t_begin, w, lane);
  if (t_begin + 1 < t_end) issue_tile<1>(c, t_begin + 1, w, lane);
  for (int t = t_begin; t < t_end; t += kNBuf) {
    tiled_pair<0>(c, q, st, t, t_end, p.scale_log2, w, lane, tid);
    if (t + 2 < t_end) tiled_pair<2>(c, q, st, t + 2, t_end, p.scale_log2, w, lane, tid);
  }
  // the four lane groups of a head hold partial sums over different tokens
  float l_run = wave_sum_xor(st.l_part, 16);
  l_run = wave_sum_xor(l_run, 32);
  const float m_run = st.m_ref;

  if (!valid_head) return;
  if (p.splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    bf16* out = reinterpret_cast<bf16*>(p.o_hat) + ((int64_t)b * p.n_h + head) * kDC;
#pragma unroll
    for (int d = 0; d < 32; ++d) {
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (bf16)(st.o[d][r] * inv);
      *reinterpret_cast<bf16x4*>(out + d * 16 + 4 * g) = v;
    }
    if (p.lse && g == 0) p.lse[(int64_t)b * p.n_h + head] = (m_run + log2f(l_run)) * 0.69314718055994531f;
    return;
  }
  const int64_t pi = ((int64_t)b * p.splits + split) * p.n_h + head;
  if (g == 0) {
    p.part_m[pi] = m_run;
    p.part_l[pi] = l_run;
  }
  if (t_begin >= t_end) return;  // an empty partition: the combines skip it by its max (-inf)
  // the partition's normalised output O_s / l_s (a convex combination of latent values) in bf16:
  // half the partial traffic of fp32 for one more rounding of 2^-9 relative
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  bf16* po = reinterpret_cast<bf16*>(p.part_o) + pi * kDC;
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    bf16x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (bf16)(st.o[d][r] * inv);
    *reinterpret_cast<bf16x4*>(po + d * 16 + 4 * g) = v;
  }
}

// Log-sum-exp combination of the partitions: M = max_s m_s, w_s = 2^(m_s - M) l_s,
// o_hat = sum_s w_s o_s / sum_s w_s with o_s = O_s / l_s the partition's normalised output (PT:
// fp32 or bf16).  A 256-thread workgroup combines four (sequence, head) rows, one wave each;
// each lane owns DC/64 consecutive latent dims.  Empty partitions (max -inf) are skipped.
template <typename T, typename PT, int DC, bool COOP>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeAttnParams p) {
  constexpr int V = DC >= 64 ? DC / 64 : 1;  // dims per thread
  const int wv = threadIdx.x >> 6;
  // b * n_h + head: one wave per row, or (COOP, many partitions) one workgroup per row, its four
  // waves taking every fourth chunk of 64 partitions and adding up in LDS
  const int bh = COOP ? blockIdx.x : blockIdx.x * 4 + wv;
  if (bh >= p.B * p.n_h) return;
  const int lane = threadIdx.x & 63;
  const bool has_dims = V * lane < DC;
  const int b = bh / p.n_h, head = bh % p.n_h;
  const int64_t base = (int64_t)b * p.splits * p.n_h + head;  // partition s at base + s * n_h
  const int d = V * lane;
  // M: the partitions' maxima one per lane, then a wave reduction
  float M = -INFINITY;
  for (int c = 0; c < p.splits; c += 64)
    if (c + lane < p.splits) M = fmaxf(M, p.part_m[base + (int64_t)(c + lane) * p.n_h]);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  float L = 0.f;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  // 64 partitions' (max, normaliser) at a time sit one per lane; a group of kG is skipped when
  // all are empty, else the output rows of its non-empty partitions are loaded together
  constexpr int kG = 16;
  for (int c0 = COOP ? 64 * wv : 0; c0 < p.splits; c0 += COOP ? 256 : 64) {
    const int64_t pl = base + (int64_t)(c0 + lane) * p.n_h;
    const float m_l = c0 + lane < p.splits ? p.part_m[pl] : -INFINITY;
    const float l_l = c0 + lane < p.splits ? p.part_l[pl] : 0.f;
    const uint64_t used = __builtin_amdgcn_ballot_w64(m_l > -INFINITY);
    for (int s0 = c0; s0 < min(p.splits, c0 + 64); s0 += kG) {
      if (((used >> (s0 - c0)) & ((1ull << kG) - 1)) == 0) continue;
      float ms[kG], ls[kG];
      PT v[kG][V];
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        ms[u] = __shfl(m_l, s0 - c0 + u, 64);
        ls[u] = __shfl(l_l, s0 - c0 + u, 64);
        if (ms[u] > -INFINITY) {  // (-inf past the last partition too)
          const PT* src = reinterpret_cast<const PT*>(p.part_o) + (base + (int64_t)(s0 + u) * p.n_h) * DC + d;
#pragma unroll
          for (int i = 0; i < V; ++i) v[u][i] = has_dims ? src[i] : PT(0.f);
        }
      }
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        if (ms[u] > -INFINITY) {
          const float ws = exp2f(ms[u] - M) * ls[u];
          L += ws;
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] += ws * to_f32(v[u][i]);
        }
      }
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
// ----------------------------------------------------------------------------- fp8 cache
// The tiled kernel over the fp8 cache (per-token-scaled e4m3 codes, one scale per part of the
// entry).  A tile is 32 tokens x 576 code bytes plus their 32 (s_c, s_r) pairs: half the bytes.
//   * S^T = K Q^T runs on fp8 MFMAs straight from the codes: the query of each head is split
//     into two e4m3 parts sharing one scale, q / s_q = hi + lo (hi the nearest code, lo the code
//     of the remainder), which keeps about bf16 precision;
//     s_tj = scale s_q (s_c,j (q . code_c,j) + s_r,j (q^R . code_r,j)).  The latent part uses the
//     16x16x128 f8f6f4 MFMA (twice the rate of the 16x16x32 fp8 form), the rope part the
//     16x16x32 fp8 one.
//   * For O^T = V^T P^T each pair of tiles is first converted once, by the whole workgroup, into
//     bf16 tiles holding value(code_c) s_c (the layout of the bf16 kernel's tiles); the PV product
//     is then the bf16 kernel's.  Converting per wave instead would repeat it eight times.
namespace tiled8 {
constexpr int kT = 32;
constexpr int kNBuf = 4;
constexpr int kRow = 576;                  // code bytes per entry (36 chunks)
constexpr int kCodes = kT * kRow;          // 18432
constexpr int kScales = kT * 8;            // 256: (s_c, s_r) per token
constexpr int kBuf = kCodes + kScales;
constexpr int kWaves = 8;
constexpr int kCopies = kCodes / 1024;     // 18: waves 0-1 issue 3, waves 2-7 issue 2
constexpr float kLazy = 8.f;
// chunk c of token row t sits at slot c ^ swz(t): the 16 rows of a K fragment read fall in distinct
// banks
__device__ __forceinline__ int swz(int t) { return ((t >> 2) & 3) ^ (((t >> 4) & 1) << 1); }
}  // namespace tiled8

__shared__ __attribute__((aligned(1024))) char g_kv8_0[tiled8::kBuf];
__shared__ __attribute__((aligned(1024))) char g_kv8_1[tiled8::kBuf];
__shared__ __attribute__((aligned(1024))) char g_kv8_2[tiled8::kBuf];
__shared__ __attribute__((aligned(1024))) char g_kv8_3[tiled8::kBuf];
template <int BUF>
__device__ __forceinline__ char* kv8_buf() {
  return BUF == 0 ? g_kv8_0 : (BUF == 1 ? g_kv8_1 : (BUF == 2 ? g_kv8_2 : g_kv8_3));
}

struct Tiled8Ctx {
  const uint8_t* pool;
  const float* scales;
  const int32_t* bt;
  int bs, kv_len;
};

// This wave's share of tile `tile` into buffer BUF: code copies P = w, w + 8, w + 16 (< 18) and, for
// wave 7, the tile's 256 bytes of scales (4 bytes per lane).
template <int BUF>
__device__ __forceinline__ void issue_tile8(const Tiled8Ctx& c, int tile, int w, int lane) {
  using namespace tiled8;
  char* dst = kv8_buf<BUF>();
  const int tok0 = tile * kT;
  const int blk = tok0 / c.bs;
  const int64_t slot0 = (int64_t)c.bt[blk] * c.bs + (tok0 - blk * c.bs);
  const __amdgpu_buffer_rsrc_t codes = dma_span(c.pool + slot0 * kRow, kCodes);
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int P = i * kWaves + w;
    if (P < kCopies) {
      const int byte = P * 1024 + ln * 16;
      const int t = byte / kRow, sl = (byte - t * kRow) >> 4;
      dma16(codes, t * kRow + ((sl ^ swz(t)) << 4), (lds_void_t*)(dst + P * 1024));
    }
  }
  if (w == kWaves - 1) {
    const __amdgpu_buffer_rsrc_t sc = dma_span(c.scales + 2 * slot0, kScales);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(sc, (lds_void_t*)(dst + kCodes), 4, ln * 4, 0, 0, 0);
  }
}

// The latent codes of fp8 tile FB as bf16 values (exact: every e4m3 value is a bf16 value) into
// bf16 tile VB (rows of 1152 bytes, chunk c of row r at slot c ^ (r & 7)); the token's scale s_c
// goes into P instead.  32 rows x 64 chunks of 8 codes: thread tid takes chunk tid % 64 of rows
// tid / 64 + 8 i.
template <int FB, int VB>
__device__ __forceinline__ void convert_tile8(int tid) {
  using namespace tiled8;
  asm volatile("" : "+v"(tid));
  const char* src = kv8_buf<FB>();
  char* dst = kv_buf<VB>();
  const int t0 = tid >> 6, c = tid & 63;
  uint2 raw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 8 * i;
    raw[i] = *reinterpret_cast<const uint2*>(src + t * kRow + (((c >> 1) ^ swz(t)) << 4) + (c & 1) * 8);
  }
  char* out = dst + t0 * tiled::kRow + ((c ^ (t0 & 7)) << 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x8 v;
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i].x, 1.f, false);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i].x, 1.f, true);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i].y, 1.f, false);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i].y, 1.f, true);
    v[0] = p0[0];
    v[1] = p0[1];
    v[2] = p1[0];
    v[3] = p1[1];
    v[4] = p2[0];
    v[5] = p2[1];
    v[6] = p3[0];
    v[7] = p3[1];
    *reinterpret_cast<bf16x8*>(out + 8 * i * tiled::kRow) = v;
  }
}

struct QFp8 {
  intx8 c_hi[4], c_lo[4];  // latent part, chunk kc: codes of dims 128 kc + 32 g .. +31
  long r_hi[2], r_lo[2];   // rope part, chunk kr: codes of rope dims 32 kr + 8 g .. +7
  float s;                 // the head's query scale
};

template <int FB, int VB>
__device__ __forceinline__ void tiled8_compute(const QFp8& q, TiledState& st, int t, int kv_len, float scale_log2,
                                               int lane) {
  using namespace tiled8;
  const char* buf = kv8_buf<FB>();
  asm volatile("" : "+v"(lane));
  const int g = lane >> 4, l16 = lane & 15;
  // ---- S^T = K Q^T per part: lane holds head l16, tokens 16 tb + 4 g + j.  The k split of a
  // 16x16x128 MFMA only has to match between its operands: lane group g gives 32 consecutive
  // dims of the chunk for both K (two 16-byte slots of the row) and Q.
  floatx4 scc[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
  floatx4 scr[2] = {floatx4{0, 0, 0, 0}, floatx4{0, 0, 0, 0}};
  {
    const char* rows[2] = {buf + l16 * kRow, buf + (16 + l16) * kRow};
    const int sw[2] = {swz(l16), swz(16 + l16)};
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
    // rope part: 8 codes of dims 32 kr + 8 g: half (g & 1) of slot 32 + 2 kr + (g >> 1)
#pragma unroll
    for (int kr = 0; kr < 2; ++kr)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int ch = 32 + 2 * kr + (g >> 1);
        const long k8 = *reinterpret_cast<const long*>(rows[tb] + ((ch ^ sw[tb]) << 4) + (g & 1) * 8);
        scr[tb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(k8, q.r_hi[kr], scr[tb], 0, 0, 0);
        scr[tb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(k8, q.r_lo[kr], scr[tb], 0, 0, 0);
      }
  }
  // ---- per-token and per-head scales; lazy online softmax
  float lmax = -INFINITY;
  float sc[2][4], s_lat[2][4];
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
      sc[tb][j] = v;
      lmax = fmaxf(lmax, v);
    }
  }
  if (__builtin_amdgcn_ballot_w64(lmax > st.m_ref + kLazy) != 0) {  // rare: raise the reference
    float hmax = wave_max_xor(lmax, 16);
    hmax = wave_max_xor(hmax, 32);
    const float m_new = fmaxf(st.m_ref, hmax);
    const float alpha = __builtin_amdgcn_exp2f(st.m_ref - m_new);  // -inf -> 0
    st.l_part *= alpha;
#pragma unroll
    for (int d = 0; d < 32; ++d) st.o[d] *= alpha;
    st.m_ref = m_new;
  }
  Frag8<bf16> pf;  // slot s = token 16 (s/4) + 4g + s%4: the weight times the token's s_c
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = __builtin_amdgcn_exp2f(sc[tb][j] - st.m_ref);  // argument <= 8
      st.l_part += e;
      pf.v[tb * 4 + j] = (bf16)(e * s_lat[tb][j]);
    }
  tiled_pv<VB>(st, pf, lane);
}

// Two fp8 tiles per barrier (fp8 buffers B0, B0+1; bf16 tiles 0 and 1): wait for them, issue the
// next pair, convert the pair's latent parts to bf16 (all waves), then multiply both tiles.
template <int B0>
__device__ __forceinline__ void tiled8_pair(const Tiled8Ctx& c, const QFp8& q, TiledState& st, int t, int t_end,
                                            float scale_log2, int w, int lane, int tid) {
  using namespace tiled8;
  MLA_TILE_BARRIER(waitcnt_vm(0));  // the pair has landed; every wave is done with the last pair
  if (t + 2 < t_end) issue_tile8<(B0 + 2) % kNBuf>(c, t + 2, w, lane);
  if (t + 3 < t_end) issue_tile8<(B0 + 3) % kNBuf>(c, t + 3, w, lane);
  const int last = min(t + 1, t_end - 1);  // only the sequence's last tile can be partial
  const int valid = c.kv_len - last * kT;
  if (valid < kT) {  // rows past the end of the context: zero codes and scales (uniform branch)
    char* buf = last == t ? kv8_buf<B0>() : kv8_buf<B0 + 1>();
    for (int i = tid; i < (kT - valid) * (kRow / 16); i += 64 * kWaves) st16(buf + valid * kRow + i * 16, zero16());
    if (tid < (kT - valid) * 2) reinterpret_cast<float*>(buf + kCodes)[valid * 2 + tid] = 0.f;
    MLA_TILE_BARRIER(kWaitLgkm0);
  }
  convert_tile8<B0, 0>(tid);
  if (t + 1 < t_end) convert_tile8<B0 + 1, 1>(tid);
  MLA_TILE_BARRIER(kWaitLgkm0);
  tiled8_compute<B0, 0>(q, st, t, c.kv_len, scale_log2, lane);
  if (t + 1 < t_end) tiled8_compute<B0 + 1, 1>(q, st, t + 1, c.kv_len, scale_log2, lane);
}

__global__ void __launch_bounds__(512)
    decode_attn_fp8_kernel(DecodeAttnParams p, int HG, const int32_t* __restrict__ block_table) {
  using namespace tiled8;
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
  const int g = lane >> 4;
  const int head = hg * (16 * kWaves) + w * 16 + (lane & 15);
  const bool valid_head = head < p.n_h;

  Tiled8Ctx c;
  c.pool = reinterpret_cast<const uint8_t*>(p.pool);
  c.scales = p.scales;
  c.bt = block_table + (int64_t)b * p.max_blocks;
  c.bs = p.block_size;
  c.kv_len = p.lens[b] + (p.lens_plus_one ? 1 : 0);

  // the head's query as hi + lo e4m3 codes with one scale: s = amax / 448 over the head's 576
  // values (the head's four lane groups), hi = e4m3(q / s), lo = e4m3(q / s - hi)
  QFp8 q;
  {
    const bf16* qrow = reinterpret_cast<const bf16*>(p.q) + ((int64_t)b * p.n_h + (valid_head ? head : 0)) * 576;
    Frag8<bf16> qv[18];  // 0..15: latent dims 128 (i / 4) + 32 g + 8 (i % 4); 16, 17: rope dims 32 kr + 8 g
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 18; ++i) {
      const int off = i < 16 ? 128 * (i >> 2) + 32 * g + 8 * (i & 3) : 512 + 32 * (i - 16) + 8 * g;
      if (valid_head) load8(qv[i], qrow + off);
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
  TiledState st;
#pragma unroll
  for (int d = 0; d < 32; ++d) st.o[d] = floatx4{0, 0, 0, 0};
  st.m_ref = -INFINITY;
  st.l_part = 0.f;

  if (t_begin < t_end) issue_tile8<0>(c, t_begin, w, lane);
  if (t_begin + 1 < t_end) issue_tile8<1>(c, t_begin + 1, w, lane);
  for (int t = t_begin; t < t_end; t += kNBuf) {
    tiled8_pair<0>(c, q, st, t, t_end, p.scale_log2, w, lane, tid);
    if (t + 2 < t_end) tiled8_pair<2>(c, q, st, t + 2, t_end, p.scale_log2, w, lane, tid);
  }
  float l_run = wave_sum_xor(st.l_part, 16);
  l_run = wave_sum_xor(l_run, 32);
  const float m_run = st.m_ref;

  if (!valid_head) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  if (p.splits == 1) {
    bf16* out = reinterpret_cast<bf16*>(p.o_hat) + ((int64_t)b * p.n_h + head) * 512;
#pragma unroll
    for (int d = 0; d < 32; ++d) {
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (bf16)(st.o[d][r] * inv);
      *reinterpret_cast<bf16x4*>(out + d * 16 + 4 * g) = v;
    }
    if (p.lse && g == 0) p.lse[(int64_t)b * p.n_h + head] = (m_run + log2f(l_run)) * 0.69314718055994531f;
    return;
  }
  const int64_t pi = ((int64_t)b * p.splits + split) * p.n_h + head;
  if (g == 0) {
    p.part_m[pi] = m_run;
    p.part_l[pi] = l_run;
  }
  if (t_begin >= t_end) return;  // an empty partition: the combines skip it by its max (-inf)
  bf16* po = reinterpret_cast<bf16*>(p.part_o) + pi * 512;
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    bf16x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (bf16)(st.o[d][r] * inv);
    *reinterpret_cast<bf16x4*>(po + d * 16 + 4 * g) = v;
  }
}

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
  if (p.fp8) {
    if (t != DType::BF16 || p.d_c != 512 || p.d_hr != 64 || p.block_size % tiled8::kT != 0 || !p.scales)
      return hipErrorInvalidValue;
    const int HG = (p.n_h + 16 * tiled8::kWaves - 1) / (16 * tiled8::kWaves);
    if (p.B == 0) return hipSuccess;
    if (p.units && p.B > 64) return hipErrorInvalidValue;  // the table builder takes B <= 64
    if (p.units) hipLaunchKernelGGL(decode_units_kernel, dim3(1), dim3(256), 0, s, p);
    const int units = p.B * p.splits + (p.units ? p.B : 0);  // with a table: + B idle entries
    const int blocks = (units + 7) / 8 * 8 * HG;
    hipLaunchKernelGGL(decode_attn_fp8_kernel, dim3(blocks), dim3(64 * tiled8::kWaves), 0, s, p, HG, p.block_table);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1 || p.leave_partials) return e;
    if (p.splits >= 16)
      hipLaunchKernelGGL((decode_combine_kernel<bf16, bf16, 512, true>), dim3(p.B * p.n_h), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((decode_combine_kernel<bf16, bf16, 512, false>), dim3((p.B * p.n_h + 3) / 4), dim3(256), 0,
                         s, p);
    return hipGetLastError();
  }
  if (decode_tiled(t, p.d_c, p.d_hr, p.block_size)) {
    const int HG = (p.n_h + 16 * tiled::kWaves - 1) / (16 * tiled::kWaves);
    if (p.B == 0) return hipSuccess;
    if (p.units && p.B > 64) return hipErrorInvalidValue;  // the table builder takes B <= 64
    if (p.units) hipLaunchKernelGGL(decode_units_kernel, dim3(1), dim3(256), 0, s, p);
    const int units = p.B * p.splits + (p.units ? p.B : 0);  // with a table: + B idle entries
    const int blocks = (units + 7) / 8 * 8 * HG;
    hipLaunchKernelGGL(decode_attn_tiled_kernel, dim3(blocks), dim3(64 * tiled::kWaves), 0, s, p, HG,
                       p.block_table);
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
