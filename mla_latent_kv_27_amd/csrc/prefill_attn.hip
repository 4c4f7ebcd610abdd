// Causal prefill attention of the MLA layer on gfx950 matrix cores (un-absorbed form).
//
// For prefill the per-head keys and values are rebuilt once from the latent
// (k^C_{j,i} = W_UK_i c^KV_j, v_{j,i} = W_UV_i c^KV_j; App. C "Full Formulas of MLA", DeepSeek-V2
// summary page), which costs far fewer flops than attending in the 576-wide latent space when
// every token is a query.  Each head then runs causal attention with
//   q = [q^C_i | RoPE(q^R_i)]  (d_h + d_hr),  k = [k^C_i | k^R] (k^R shared by all heads),
//   v = v_i (d_h),   o_{t,i} = sum_{j<=t} softmax_j(scale * q_t . k_j) v_j.
// A workgroup owns 128 queries of one head (four waves of 32) and walks 64-key tiles up to the
// diagonal with an online softmax.  The contraction S^T = K Q^T gives each lane one query and 16
// keys per 32-key block; those are exactly the B operand of O^T = V^T P^T, so probabilities stay
// in registers, and V arrives token-contiguous ([head][dim][token]) so V^T fragments are two
// 4-element runs per lane.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace mla {

constexpr int kBQ = 128;  // queries per workgroup
constexpr int kBKV = 64;  // keys per tile

template <typename T, int DH, int DR>
__global__ void __launch_bounds__(256) prefill_attn_kernel(PrefillAttnParams p) {
  constexpr int DQ = DH + DR;
  constexpr int DQP = (DQ + 15) / 16 * 16;
  constexpr int KS = DQP / 16;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int LDK = DQP + EPC;
  constexpr int LDV = kBKV + 8;
  constexpr int DHP = (DH + 31) / 32 * 32;  // value rows padded to whole 32-row blocks
  constexpr int DB = DHP / 32;
  __shared__ __attribute__((aligned(16))) T Ks[kBKV * LDK];
  __shared__ __attribute__((aligned(16))) T Vt[DHP * LDV];

  const int nqt = (p.T + kBQ - 1) / kBQ;
  const int x = blockIdx.x;
  const int qt = nqt - 1 - x / (p.n_h * p.S);  // longest rows first
  const int head = (x % (p.n_h * p.S)) % p.n_h;
  const int s = (x % (p.n_h * p.S)) / p.n_h;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 5, ql = lane & 31;
  const int qi = qt * kBQ + w * 32 + ql;  // query index within the sequence
  const int64_t MT = (int64_t)p.S * p.T;
  const int Tp = (p.T + kBKV - 1) / kBKV * kBKV;

  Frag8<T> q[KS];
  {
    const T* qrow = reinterpret_cast<const T*>(p.q) + (((int64_t)s * p.T + min(qi, p.T - 1)) * p.n_h + head) * DQ;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = ks * 16 + 8 * g;
      if (qi < p.T && k < DQ) load8(q[ks], qrow + k);
      else zero8(q[ks]);
    }
  }
  if (DQP > DQ) {
    for (int c = tid; c < kBKV * (DQP - DQ); c += 256) {
      const int r = c / (DQP - DQ), k = DQ + c % (DQP - DQ);
      Ks[r * LDK + k] = from_f32<T>(0.f);
    }
  }
  if (DHP > DH) {
    for (int c = tid; c < (DHP - DH) * LDV; c += 256) Vt[DH * LDV + c] = from_f32<T>(0.f);
  }

  floatx16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const T* kbase = reinterpret_cast<const T*>(p.k) + ((int64_t)head * MT + (int64_t)s * p.T) * DH;
  const T* krbase = reinterpret_cast<const T*>(p.kr) + (int64_t)s * p.T * p.ld_kr + p.kr_off;
  const T* vbase = reinterpret_cast<const T*>(p.vt) + ((int64_t)head * DH * p.S + s) * Tp;  // row d at + d*S*Tp
  const int64_t vrow = (int64_t)p.S * Tp;

  const int kt_end = min((p.T + kBKV - 1) / kBKV, ((qt + 1) * kBQ + kBKV - 1) / kBKV);
  for (int kt = 0; kt < kt_end; ++kt) {
    const int j0 = kt * kBKV;
    __syncthreads();
    for (int c = tid; c < kBKV * (DQ / EPC); c += 256) {
      const int r = c / (DQ / EPC), cc = (c % (DQ / EPC)) * EPC;
      const int j = j0 + r;
      Chunk16 v = zero16();
      if (j < p.T) v = cc < DH ? ld16(kbase + (int64_t)j * DH + cc) : ld16(krbase + (int64_t)j * p.ld_kr + (cc - DH));
      st16(&Ks[r * LDK + cc], v);
    }
    for (int c = tid; c < DH * (kBKV / EPC); c += 256) {
      const int d = c / (kBKV / EPC), cc = (c % (kBKV / EPC)) * EPC;
      Chunk16 v = ld16(vbase + d * vrow + j0 + cc);  // padded rows: always in bounds
      if (j0 + cc + EPC > p.T) {
        T* e = reinterpret_cast<T*>(&v);
        for (int xx = 0; xx < EPC; ++xx)
          if (j0 + cc + xx >= p.T) e[xx] = from_f32<T>(0.f);
      }
      st16(&Vt[d * LDV + cc], v);
    }
    __syncthreads();

    floatx16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frag8<T> a;
        load8(a, &Ks[(kb * 32 + ql) * LDK + ks * 16 + 8 * g]);
        sc[kb] = mma32(a, q[ks], sc[kb]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        const float v = (j <= qi && j < p.T) ? sc[kb][r] * p.scale_log2 : -INFINITY;
        sc[kb][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = wave_max_xor(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    // a wave whose queries all precede this tile sees only -inf; keep its state unchanged
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = to_f32(from_f32<T>(exp2f(sc[kb][r] - m_use)));  // as rounded for PV
        sc[kb][r] = e;
        sum += e;
      }
    sum = wave_sum_xor(sum, 32);
    l_run = l_run * alpha + sum;
    m_run = m_new;
#pragma unroll
    for (int d = 0; d < DB; ++d) o[d] *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        Frag8<T> pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) set8(pf, e, sc[kb][8 * half + e]);
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          Frag8<T> a;
          const T* vr = &Vt[(d * 32 + ql) * LDV + kb * 32 + half * 16 + 4 * g];
          load4x2(a, vr, vr + 8);
          o[d] = mma32(a, pf, o[d]);
        }
      }
  }

  if (qi >= p.T) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const int64_t orow = (((int64_t)s * p.T + qi) * p.n_h + head) * DH;
  T* out = reinterpret_cast<T*>(p.o) + orow;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dim = d * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (DHP > DH && dim >= DH) continue;
      const float v = o[d][r] * inv;
      out[dim] = from_f32<T>(v);
      if (p.o_f32) p.o_f32[orow + dim] = v;
    }
}

bool prefill_supported(int d_h, int d_hr) { return (d_h == 128 && d_hr == 64) || (d_h == 16 && d_hr == 8) || (d_h == 32 && d_hr == 8); }

namespace {
template <typename T, int DH, int DR>
hipError_t launch(const PrefillAttnParams& p, hipStream_t s) {
  const int nqt = (p.T + kBQ - 1) / kBQ;
  const int64_t blocks = (int64_t)nqt * p.n_h * p.S;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_attn_kernel<T, DH, DR>), dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}
}  // namespace

hipError_t prefill_attention(DType t, const PrefillAttnParams& p, hipStream_t s) {
  if (p.d_h == 128 && p.d_hr == 64)
    return t == DType::BF16 ? launch<bf16, 128, 64>(p, s) : launch<float, 128, 64>(p, s);
  if (p.d_h == 16 && p.d_hr == 8)
    return t == DType::BF16 ? launch<bf16, 16, 8>(p, s) : launch<float, 16, 8>(p, s);
  if (p.d_h == 32 && p.d_hr == 8)
    return t == DType::BF16 ? launch<bf16, 32, 8>(p, s) : launch<float, 32, 8>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
