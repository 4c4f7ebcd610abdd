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
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min(ntiles, t_begin + p.tiles_per_split);

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
  float* po = p.part_o + pi * DC;
#pragma unroll
  for (int d = 0; d < Sh::DB; ++d) *reinterpret_cast<floatx4*>(po + d * 16 + 4 * g) = o[d];
}

// Log-sum-exp combination of the partitions: M = max_s m_s, w_s = 2^(m_s - M),
// o_hat = sum_s w_s O_s / sum_s w_s l_s.
template <typename T, int DC>
__global__ void __launch_bounds__(128) decode_combine_kernel(DecodeAttnParams p) {
  const int bh = blockIdx.x;  // b * n_h + head
  const int b = bh / p.n_h, head = bh % p.n_h;
  float M = -INFINITY;
  for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.part_m[((int64_t)b * p.splits + s) * p.n_h + head]);
  float L = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    const int64_t pi = ((int64_t)b * p.splits + s) * p.n_h + head;
    const float ms = p.part_m[pi];
    if (ms > -INFINITY) L += exp2f(ms - M) * p.part_l[pi];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  T* out = reinterpret_cast<T*>(p.o_hat) + (int64_t)bh * DC;
  for (int d = threadIdx.x; d < DC; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < p.splits; ++s) {
      const int64_t pi = ((int64_t)b * p.splits + s) * p.n_h + head;
      const float ms = p.part_m[pi];
      if (ms > -INFINITY) acc += exp2f(ms - M) * p.part_o[pi * DC + d];
    }
    out[d] = from_f32<T>(acc * inv);
  }
  if (p.lse && threadIdx.x == 0) p.lse[bh] = (M + log2f(L)) * 0.69314718055994531f;
}

// ----------------------------------------------------------------------------- host side
int decode_tile_tokens() { return kTile; }

int decode_heads_per_block(int n_h) { return n_h >= 128 ? 128 : (n_h >= 64 ? 64 : 16); }

bool decode_supported(int d_c, int d_hr) { return (d_c == 512 && d_hr == 64) || (d_c == 32 && d_hr == 8); }

namespace {
template <typename T, int DC, int DR>
hipError_t launch(const DecodeAttnParams& p, hipStream_t s) {
  const int hpb = decode_heads_per_block(p.n_h);
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
  hipLaunchKernelGGL((decode_combine_kernel<T, DC>), dim3(p.B * p.n_h), dim3(128), 0, s, p);
  return hipGetLastError();
}
}  // namespace

hipError_t decode_attention(DType t, const DecodeAttnParams& p, hipStream_t s) {
  if (p.d_c == 512 && p.d_hr == 64)
    return t == DType::BF16 ? launch<bf16, 512, 64>(p, s) : launch<float, 512, 64>(p, s);
  if (p.d_c == 32 && p.d_hr == 8)
    return t == DType::BF16 ? launch<bf16, 32, 8>(p, s) : launch<float, 32, 8>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
