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
  const int qi = qt * kBQ + w * 32 + ql;  // query index within the chunk
  const int off = p.q_off ? p.q_off[s] : 0;  // position of the chunk's first query
  const int qpos = off + qi;
  const int nk = off + p.T;                  // valid keys of this sequence
  const int Tk = p.Tk > 0 ? p.Tk : p.T;
  const int Tp = (Tk + kBKV - 1) / kBKV * kBKV;

  // [q^C | RoPE(q^R)] fragments: dims k .. k+7 of a chunk lie in one part (d_h and d_hr are
  // multiples of 8); the rope ones are four pairs, rotated in fp32 and then rounded to T
  Frag8<T> q[KS];
  {
    const int64_t row = (int64_t)s * p.T + min(qi, p.T - 1);
    const T* qrow = reinterpret_cast<const T*>(p.qc) + row * p.n_h * DH + (int64_t)head * DH;
    const float* rrow = p.qr + row * p.n_h * DR + (int64_t)head * DR;
    const float2* tab = p.rope + row * (DR / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = ks * 16 + 8 * g;
      if (qi >= p.T || k >= DQ) {
        zero8(q[ks]);
      } else if (k < DH) {
        load8(q[ks], qrow + k);
      } else {
        const int d0 = k - DH;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = rrow[d0 + 2 * i], x1 = rrow[d0 + 2 * i + 1];
          const float2 cs = tab[d0 / 2 + i];
          set8(q[ks], 2 * i, x0 * cs.x - x1 * cs.y);
          set8(q[ks], 2 * i + 1, x1 * cs.x + x0 * cs.y);
        }
      }
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

  const T* kbase = reinterpret_cast<const T*>(p.k) + (int64_t)s * Tk * p.k_ld + (int64_t)head * DH;
  const T* krbase = reinterpret_cast<const T*>(p.kr) + (int64_t)s * Tk * p.ld_kr + p.kr_off;
  const T* vbase = reinterpret_cast<const T*>(p.vt) + ((int64_t)head * DH * p.S + s) * Tp;  // row d at + d*S*Tp
  const int64_t vrow = (int64_t)p.S * Tp;

  const int kt_end = min((nk + kBKV - 1) / kBKV, (off + (qt + 1) * kBQ + kBKV - 1) / kBKV);
  for (int kt = 0; kt < kt_end; ++kt) {
    const int j0 = kt * kBKV;
    __syncthreads();
    for (int c = tid; c < kBKV * (DQ / EPC); c += 256) {
      const int r = c / (DQ / EPC), cc = (c % (DQ / EPC)) * EPC;
      const int j = j0 + r;
      Chunk16 v = zero16();
      if (j < nk) v = cc < DH ? ld16(kbase + (int64_t)j * p.k_ld + cc) : ld16(krbase + (int64_t)j * p.ld_kr + (cc - DH));
      st16(&Ks[r * LDK + cc], v);
    }
    for (int c = tid; c < DH * (kBKV / EPC); c += 256) {
      const int d = c / (kBKV / EPC), cc = (c % (kBKV / EPC)) * EPC;
      Chunk16 v = ld16(vbase + d * vrow + j0 + cc);  // padded rows: always in bounds
      if (j0 + cc + EPC > nk) {
        T* e = reinterpret_cast<T*>(&v);
        for (int xx = 0; xx < EPC; ++xx)
          if (j0 + cc + xx >= nk) e[xx] = from_f32<T>(0.f);
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
        const float v = (j <= qpos && j < nk) ? sc[kb][r] * p.scale_log2 : -INFINITY;
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

// ----------------------------------------------------------------------------- pipelined kernel
// The DeepSeek-V2 case (bf16, d_h = 128, d_hr = 64).  Same arithmetic as above, with the K and V^T
// tiles streamed by direct global->LDS copies into a ring of three 40 KiB stages (two tiles in
// flight while one is multiplied), one barrier per tile, and eight waves (256 queries of one head)
// sharing every tile.  LDS rows swizzle 16-byte chunks (slot = chunk ^ f(row)) so that the
// fragment reads of 32 rows spread over the banks.  Workgroups of the same head are placed on
// the same XCD so that their tiles come from its L2.
namespace pf2 {
constexpr int kWaves = 8;
constexpr int kQ = 32 * kWaves;      // queries per workgroup
constexpr int kKV = 64;              // keys per tile
constexpr int kDH = 128, kDR = 64, kDQ = kDH + kDR;
// a stage: key content rows (64 x 256 bytes), rope key rows (64 x 128 bytes), V^T rows (128 dims
// x 128 bytes = 64 keys); every copy instruction reads one of the three sources
constexpr int kKRow = kDH * 2, kRRow = kDR * 2;
constexpr int kKBytes = kKV * kKRow;    // 16 KiB
constexpr int kRBytes = kKV * kRRow;    // 8 KiB
constexpr int kVRow = kKV * 2;          // 128 bytes per value row (one dim, 64 keys)
constexpr int kVBytes = kDH * kVRow;    // 16 KiB
constexpr int kROff = kKBytes, kVOff = kKBytes + kRBytes;
constexpr int kStage = kKBytes + kRBytes + kVBytes;
constexpr int kNS = 3;
constexpr int kKCopies = kKBytes / 1024 / kWaves;  // 2 per wave (4 rows each)
constexpr int kRCopies = kRBytes / 1024 / kWaves;  // 1 per wave (8 rows)
constexpr int kVCopies = kVBytes / 1024 / kWaves;  // 2 per wave (8 rows)
constexpr int kCopies = kKCopies + kRCopies + kVCopies;
// 16-byte chunk c of a row r sits at slot c ^ swizzle: 16 consecutive rows then cover all banks
__device__ __forceinline__ int kslot(int r, int c) { return c ^ (r & 15); }         // 16-chunk rows
__device__ __forceinline__ int rslot(int r, int c) { return c ^ ((r >> 1) & 7); }   // 8-chunk rows
// V^T rows (128 bytes: 8 chunks of 8 keys).  The rows arrive with the 4-key pieces of every 16 keys
// in the order 0, 2, 1, 3 (the epilogue of the V^T product stores them so), which puts the 8 keys a
// lane group takes in one 16-key step (4g .. 4g+3 and 8 + 4g .. +3) in one chunk.  A fragment read
// is then one 16-byte read; LDS serves those 8 lanes (8 consecutive rows, one chunk) at a time, and
// rows 128 bytes apart share banks, so the chunk is XORed with row & 7.
__device__ __forceinline__ int vswz(int d) { return d & 7; }
// position of key k in a V^T row
__device__ __forceinline__ int vpos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }
}  // namespace pf2

__shared__ __attribute__((aligned(1024))) char g_pf_s0[pf2::kStage];
__shared__ __attribute__((aligned(1024))) char g_pf_s1[pf2::kStage];
__shared__ __attribute__((aligned(1024))) char g_pf_s2[pf2::kStage];

template <int ST>
__device__ __forceinline__ char* pf_stage() { return ST == 0 ? g_pf_s0 : (ST == 1 ? g_pf_s1 : g_pf_s2); }

struct Pf2Ctx {
  __amdgpu_buffer_rsrc_t k;   // key rows of this (sequence, head), krow bytes apart
  __amdgpu_buffer_rsrc_t kr;  // rope key rows of this sequence, ld_kr elements apart
  __amdgpu_buffer_rsrc_t vt;  // V^T rows of this (sequence, head): row d at d * vrow elements
  int ld_kr, vrow;
  int krow;  // bytes from one key row to the next (256 head-major, 2 n_h d_h token-major)
  int T;     // valid keys of this sequence
};

// Tile kt into stage ST: key rows (clamped to the last valid key, masked later) and V^T rows
// (padded to whole tiles, so always in bounds).
template <int ST>
__device__ __forceinline__ void pf2_issue(const Pf2Ctx& c, int kt, int w, int lane) {
  using namespace pf2;
  char* st = pf_stage<ST>();
  const int j0 = kt * kKV;
#pragma unroll
  for (int i = 0; i < kKCopies; ++i) {
    const int P = i * kWaves + w, r = 4 * P + (lane >> 4);
    const int j = min(j0 + r, c.T - 1);
    dma16(c.k, (uint32_t)(j * c.krow + kslot(r, lane & 15) * 16), (lds_void_t*)(st + P * 1024));
  }
#pragma unroll
  for (int i = 0; i < kRCopies; ++i) {
    const int P = i * kWaves + w, r = 8 * P + (lane >> 3);
    const int j = min(j0 + r, c.T - 1);
    dma16(c.kr, (uint32_t)(j * c.ld_kr * 2 + rslot(r, lane & 7) * 16), (lds_void_t*)(st + kROff + P * 1024));
  }
#pragma unroll
  for (int i = 0; i < kVCopies; ++i) {
    const int P = i * kWaves + w;
    const int C = P * 64 + lane;
    const int d = C / 8, sl = C % 8;
    const int ch = sl ^ vswz(d);
    dma16(c.vt, (uint32_t)((d * c.vrow + j0 + ch * 8) * 2), (lds_void_t*)(st + kVOff + P * 1024));
  }
}

struct Pf2State {
  floatx16 o[4];   // O^T: 4 blocks of 32 dims; lane: query l32, dims 32 d + 8 (r/4) + 4g + r%4
  float m_ref;     // the query's reference max, raw score units (shared by its two lanes)
  float l_part;    // this lane's partial normaliser (the two lanes of a query combine at the end)
};

// Lazy softmax: the reference max only moves (and O is rescaled) when a score exceeds it by more
// than kLazy / scale in log2 units, so the common tile needs no cross-lane exchange and no rescale.
constexpr float kPfLazy = 8.f;

template <int ST>
__device__ __forceinline__ void pf2_compute(const Frag8<bf16> (&q)[12], Pf2State& s, int kt, int qpos, int nk,
                                            bool masked, float scale_log2, int lane) {
  using namespace pf2;
  const char* st = pf_stage<ST>();
  const int g = lane >> 5, l32 = lane & 31, x = vswz(l32);
  const int j0 = kt * kKV;
  floatx16 sc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
    const int r = kb * 32 + l32;
    const char* krow = st + r * kKRow;
    const char* rrow = st + kROff + r * kRRow;
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) {
      Frag8<bf16> a;
      if (ks < 8) a.v = *reinterpret_cast<const bf16x8*>(krow + kslot(r, 2 * ks + g) * 16);
      else a.v = *reinterpret_cast<const bf16x8*>(rrow + rslot(r, 2 * (ks - 8) + g) * 16);
      sc[kb] = mma32(a, q[ks], sc[kb]);
    }
  }
  // raw scores; keys past the query or past the sequence only on the diagonal / last tile
  float mx = -INFINITY;
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (!(j <= qpos && j < nk)) sc[kb][r] = -INFINITY;
      }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
  if (__builtin_amdgcn_ballot_w64((mx - s.m_ref) * scale_log2 > kPfLazy) != 0) {  // rare: raise the reference
    const float qmax = wave_max_xor(mx, 32);
    const float m_new = fmaxf(s.m_ref, qmax);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f((s.m_ref - m_new) * scale_log2);  // first key: 0
    s.l_part *= alpha;
#pragma unroll
    for (int d = 0; d < 4; ++d) s.o[d] *= alpha;
    s.m_ref = m_new;
  }
  // p = 2^((s - m) scale) (argument <= kPfLazy); a query with no visible key yet keeps m = -inf
  const float mb = s.m_ref == -INFINITY ? 0.f : -s.m_ref * scale_log2;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = __builtin_amdgcn_exp2f(fmaf(sc[kb][r], scale_log2, mb));
      s.l_part += e;
      sc[kb][r] = e;
    }
  // O^T += V^T P^T: lane (dim 32 d + l32, group g) takes keys 16 (2kb + half) + 4g + 0..3 and
  // + 8 + 0..3: chunk 4kb + 2half + g of its row
  const char* vrow = st + kVOff + l32 * kVRow;
  const int gx = g ^ x;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      Frag8<bf16> pfr;
#pragma unroll
      for (int e = 0; e < 8; ++e) pfr.v[e] = (bf16)sc[kb][8 * half + e];
      const int cx = (4 * kb + 2 * half) ^ gx;  // (4kb + 2half + g) ^ x
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        Frag8<bf16> a;
        a.v = *reinterpret_cast<const bf16x8*>(vrow + d * 32 * kVRow + cx * 16);
        s.o[d] = mma32(a, pfr, s.o[d]);
      }
    }
}

// Tile kt of the ring (stage ST = kt % 3): wait for it (tile kt+1 may be in flight), refill the
// stage of tile kt-1 with tile kt+2, zero the value columns past the end of the sequence, and
// multiply unless every query of this wave precedes the tile.
template <int ST>
__device__ __forceinline__ void pf2_step(const Pf2Ctx& c, const Frag8<bf16> (&q)[12], Pf2State& s, int kt,
                                         int kt_end, int qpos_first, int qpos_last, int qpos, float scale_log2,
                                         int w, int lane, int tid) {
  using namespace pf2;
  if (kt + 1 < kt_end) MLA_TILE_BARRIER(waitcnt_vm(kCopies));
  else MLA_TILE_BARRIER(waitcnt_vm(0));
  if (kt + 2 < kt_end) pf2_issue<(ST + 2) % kNS>(c, kt + 2, w, lane);
  const int valid = c.T - kt * kKV;
  if (valid < kKV) {  // uniform: V^T columns of keys >= T (padding, uninitialised) -> 0
    char* v = pf_stage<ST>() + kVOff;
    for (int i = tid; i < kDH * (kKV - valid); i += 64 * kWaves) {
      const int d = i / (kKV - valid), pos = vpos(valid + i % (kKV - valid));
      const int slot = (pos >> 3) ^ vswz(d);
      *reinterpret_cast<bf16*>(v + d * kVRow + slot * 16 + (pos & 7) * 2) = (bf16)0.f;
    }
    MLA_TILE_BARRIER(kWaitLgkm0);
  }
  // the mask is needed only where the tile reaches past the wave's first query or the sequence
  const bool masked = kt * kKV + kKV - 1 > qpos_first || (kt + 1) * kKV > c.T;
  if (kt * kKV <= qpos_last) pf2_compute<ST>(q, s, kt, qpos, c.T, masked, scale_log2, lane);
}

__global__ void __launch_bounds__(512)
    prefill_attn_pipelined_kernel(PrefillAttnParams p, int nqt, int units) {
  using namespace pf2;
  // block id -> (unit = sequence * n_h + head, query tile): the query tiles of a unit share an
  // XCD (ids are dealt to the 8 XCDs round robin), longest rows first
  const int xcd = blockIdx.x % 8, r = blockIdx.x / 8;
  const int unit = (r / nqt) * 8 + xcd;
  if (unit >= units) return;
  const int qt = nqt - 1 - r % nqt;
  const int sq = unit / p.n_h, head = unit % p.n_h;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, ql = lane & 31;
  const int qi = qt * kQ + w * 32 + ql;
  const int off = p.q_off ? p.q_off[sq] : 0;  // position of the chunk's first query
  const int nk = off + p.T;                   // valid keys of this sequence
  const int qpos_last = off + min(qt * kQ + w * 32 + 31, p.T - 1);  // this wave's last query
  const int qpos_first = off + qt * kQ + w * 32;                     // and its first
  const int Tk = p.Tk > 0 ? p.Tk : p.T;
  const int Tp = (Tk + kKV - 1) / kKV * kKV;

  Pf2Ctx c;
  // spans below 2 GiB (checked by the launcher): offsets within them are 32-bit; key row j of
  // head h at j * k_ld + h * d_h
  c.k = dma_span(reinterpret_cast<const bf16*>(p.k) + (int64_t)sq * Tk * p.k_ld + (int64_t)head * kDH,
                 (uint32_t)(((int64_t)(nk - 1) * p.k_ld + kDH) * 2));
  c.krow = (int)(p.k_ld * 2);
  c.kr = dma_span(reinterpret_cast<const bf16*>(p.kr) + (int64_t)sq * Tk * p.ld_kr + p.kr_off,
                  (uint32_t)(((int64_t)(nk - 1) * p.ld_kr + kDR) * 2));
  c.ld_kr = (int)p.ld_kr;
  c.vrow = p.S * Tp;
  c.vt = dma_span(reinterpret_cast<const bf16*>(p.vt) + ((int64_t)head * kDH * p.S + sq) * Tp,
                  (uint32_t)(((int64_t)(kDH - 1) * c.vrow + Tp) * 2));
  c.T = nk;

  Frag8<bf16> q[12];
  {  // q^C, and q^R rotated here: dims 16 (ks - 8) + 8g .. +7 are 4 pairs
    const int64_t row = (int64_t)sq * p.T + min(qi, p.T - 1);
    const bf16* qrow = reinterpret_cast<const bf16*>(p.qc) + row * p.n_h * kDH + (int64_t)head * kDH;
    const float* rrow = p.qr + row * p.n_h * kDR + (int64_t)head * kDR;
    const float2* tab = p.rope + row * (kDR / 2);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) load8(q[ks], qrow + ks * 16 + 8 * g);
#pragma unroll
    for (int ks = 8; ks < 12; ++ks) {
      const int d0 = (ks - 8) * 16 + 8 * g;
      const floatx4 x0 = *reinterpret_cast<const floatx4*>(rrow + d0);
      const floatx4 x1 = *reinterpret_cast<const floatx4*>(rrow + d0 + 4);
      const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 cs = tab[d0 / 2 + i];
        q[ks].v[2 * i] = (bf16)(x[2 * i] * cs.x - x[2 * i + 1] * cs.y);
        q[ks].v[2 * i + 1] = (bf16)(x[2 * i + 1] * cs.x + x[2 * i] * cs.y);
      }
    }
    if (qi >= p.T)
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) zero8(q[ks]);
  }
  Pf2State s;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) s.o[d][rr] = 0.f;
  s.m_ref = -INFINITY;
  s.l_part = 0.f;

  const int kt_end = min((nk + kKV - 1) / kKV, (off + (qt + 1) * kQ + kKV - 1) / kKV);
  const int qpos = off + qi;
  if (kt_end > 0) pf2_issue<0>(c, 0, w, lane);
  if (kt_end > 1) pf2_issue<1>(c, 1, w, lane);
  for (int kt = 0; kt < kt_end; kt += kNS) {
    pf2_step<0>(c, q, s, kt, kt_end, qpos_first, qpos_last, qpos, p.scale_log2, w, lane, tid);
    if (kt + 1 < kt_end)
      pf2_step<1>(c, q, s, kt + 1, kt_end, qpos_first, qpos_last, qpos, p.scale_log2, w, lane, tid);
    if (kt + 2 < kt_end)
      pf2_step<2>(c, q, s, kt + 2, kt_end, qpos_first, qpos_last, qpos, p.scale_log2, w, lane, tid);
  }
  MLA_WAVE_WAIT(waitcnt_vm(0));

  const float l_run = wave_sum_xor(s.l_part, 32);  // the query's two lanes
  if (qi >= p.T) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const int64_t orow = (((int64_t)sq * p.T + qi) * p.n_h + head) * kDH;
  bf16* out = reinterpret_cast<bf16*>(p.o) + orow;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int rr = 0; rr < 16; rr += 4) {
      const int dim = d * 32 + 8 * (rr >> 2) + 4 * g;
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = s.o[d][rr + i] * inv;
        v[i] = (bf16)f;
        if (p.o_f32) p.o_f32[orow + dim + i] = f;
      }
      *reinterpret_cast<bf16x4*>(out + dim) = v;
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

// the pipelined kernel addresses each source span with 32-bit byte offsets
static bool pf2_spans_fit(int64_t S, int64_t Tk, int64_t ld_kr, int64_t k_ld) {
  const int64_t Tp = (Tk + pf2::kKV - 1) / pf2::kKV * pf2::kKV;
  return ((Tk - 1) * k_ld + pf2::kDH) * 2 < (1LL << 31) && ((Tk - 1) * ld_kr + pf2::kDR) * 2 < (1LL << 31) &&
         ((int64_t)(pf2::kDH - 1) * S * Tp + Tp) * 2 < (1LL << 31);
}

bool prefill_pipelined(DType t, int d_h, int d_hr, int64_t S, int64_t Tk, int64_t ld_kr, int64_t k_ld) {
  return t == DType::BF16 && d_h == 128 && d_hr == 64 && pf2_spans_fit(S, Tk, ld_kr, k_ld);
}

hipError_t prefill_attention(DType t, const PrefillAttnParams& p, hipStream_t s) {
  const int64_t Tk = p.Tk > 0 ? p.Tk : p.T;
  if (!p.qc || !p.qr || !p.rope || !p.k || p.k_ld < (int64_t)p.n_h * p.d_h) return hipErrorInvalidValue;
  // the DeepSeek-V2 head sizes in bf16 take the pipelined kernel (unless a source span needs
  // 64-bit offsets); every other supported size the synchronous one
  const bool pipelined = prefill_pipelined(t, p.d_h, p.d_hr, p.S, Tk, p.ld_kr, p.k_ld);
  if (pipelined) {
    const int nqt = (p.T + pf2::kQ - 1) / pf2::kQ;
    const int units = p.S * p.n_h;
    const int64_t blocks = (int64_t)(units + 7) / 8 * 8 * nqt;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_attn_pipelined_kernel, dim3((unsigned)blocks), dim3(64 * pf2::kWaves), 0, s, p, nqt,
                       units);
    return hipGetLastError();
  }
  if (p.d_h == 128 && p.d_hr == 64)
    return t == DType::BF16 ? launch<bf16, 128, 64>(p, s) : launch<float, 128, 64>(p, s);
  if (p.d_h == 16 && p.d_hr == 8)
    return t == DType::BF16 ? launch<bf16, 16, 8>(p, s) : launch<float, 16, 8>(p, s);
  if (p.d_h == 32 && p.d_hr == 8)
    return t == DType::BF16 ? launch<bf16, 32, 8>(p, s) : launch<float, 32, 8>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
