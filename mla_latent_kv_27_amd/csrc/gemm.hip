// Projection GEMMs of the MLA layer on gfx950 matrix cores.
//
// Every projection on the DeepSeek-V2 summary page's App. C ("Full Formulas of MLA") is a
// product y = W x with W row-major [out][in]; batched over heads it also covers the per-head
// up-projections W_UK_i / W_UV_i and the query absorption q_hat_i = W_UK_i^T q^C_i (an "NN"
// product against W_UK's row block).  One kernel template serves every shape: a workgroup
// computes a BM x BN tile with 32x32x16 bf16 MFMA (or the fp32 32x32x2 form), stages 32-wide
// k slices of both operands through LDS, and either stores through the epilogue (type
// conversion, RoPE on the rope columns, paged-cache row scatter, head-strided columns) or,
// when K is split across workgroups for small M, writes fp32 partials that a second kernel
// sums before running the same epilogue.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace mla {

constexpr int kBK = 32;  // k elements staged per iteration

__device__ __forceinline__ void rope_pair(const Epilogue& e, int row, int col, float& v, float partner) {
  if (col >= e.rope_col0) {
    const int k = ((col - e.rope_col0) % e.d_hr) >> 1;
    const float2 cs = e.rope_tab[(int64_t)row * (e.d_hr >> 1) + k];
    v = (col & 1) ? (partner * cs.y + v * cs.x) : (v * cs.x - partner * cs.y);
  }
}

template <typename T>
__device__ __forceinline__ void epi_store(const Epilogue& e, int z, int row, int col, float v) {
  int64_t rbase;
  if (e.block_table) {
    const int sq = e.row_seq[row], ps = e.row_pos[row];
    const int64_t slot =
        (int64_t)e.block_table[(int64_t)sq * e.max_blocks + ps / e.block_size] * e.block_size +
        ps % e.block_size;
    rbase = slot * e.ldc;
  } else {
    rbase = (int64_t)row * e.ldc;
  }
  const int64_t idx = (int64_t)z * e.batch_stride + rbase + (int64_t)(col / e.group) * e.group_stride +
                      e.group_off + col % e.group;
  if (e.c_f32)
    reinterpret_cast<float*>(e.C)[idx] = v;
  else
    reinterpret_cast<T*>(e.C)[idx] = from_f32<T>(v);
  if (e.C2) e.C2[idx] = v;
}

template <typename T, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
    gemm_kernel(GemmParams p, int splits, int k_per_split, float* __restrict__ partial) {
  constexpr int NT = 64 * WM * WN;
  constexpr int FM = BM / WM / 32, FN = BN / WN / 32;
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
  constexpr int LDK = kBK + 16 / sizeof(T);    // padded LDS row (elements)
  __shared__ __attribute__((aligned(16))) T As[BM * LDK];
  __shared__ __attribute__((aligned(16))) T Bs[BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tile = blockIdx.x;
  const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;
  const int z = blockIdx.y / splits, sp = blockIdx.y % splits;
  const int kb = sp * k_per_split, ke = min(p.K, kb + k_per_split);

  const T* A = reinterpret_cast<const T*>(p.A) + (int64_t)z * p.strideA;
  const T* B0 = reinterpret_cast<const T*>(p.B0) + (int64_t)z * p.strideB;
  const T* B1 = p.B1 ? reinterpret_cast<const T*>(p.B1) + (int64_t)z * p.strideB : nullptr;

  floatx16 acc[FM][FN];
  for (int i = 0; i < FM; ++i)
    for (int j = 0; j < FN; ++j)
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int k0 = kb; k0 < ke; k0 += kBK) {
    __syncthreads();
    // A slice: BM rows x kBK, 16-byte chunks
    for (int c = tid; c < BM * (kBK / EPC); c += NT) {
      const int r = c / (kBK / EPC), kc = (c % (kBK / EPC)) * EPC;
      const int gr = m0 + r, gk = k0 + kc;
      Chunk16 v = zero16();
      if (gr < p.M && gk < ke) v = ld16(A + (int64_t)gr * p.lda + gk);
      st16(&As[r * LDK + kc], v);
    }
    if (!p.nn) {
      for (int c = tid; c < BN * (kBK / EPC); c += NT) {
        const int r = c / (kBK / EPC), kc = (c % (kBK / EPC)) * EPC;
        const int gn = n0 + r, gk = k0 + kc;
        Chunk16 v = zero16();
        if (gn < p.N && gk < ke) {
          const T* src = gn < p.N0 ? B0 + (int64_t)gn * p.ldb : B1 + (int64_t)(gn - p.N0) * p.ldb;
          v = ld16(src + gk);
        }
        st16(&Bs[r * LDK + kc], v);
      }
    } else {
      // B stored [K][N]: read N-contiguous chunks, write transposed into Bs[n][k]
      for (int c = tid; c < kBK * (BN / EPC); c += NT) {
        const int kk = c / (BN / EPC), nc = (c % (BN / EPC)) * EPC;
        const int gk = k0 + kk, gn = n0 + nc;
        Chunk16 v = zero16();
        if (gk < ke && gn < p.N) v = ld16(B0 + (int64_t)gk * p.ldb + gn);
        const T* e = reinterpret_cast<const T*>(&v);
        for (int i = 0; i < EPC; ++i) Bs[(nc + i) * LDK + kk] = e[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      Frag8<T> a[FM], b[FN];
      const int kofs = ks * 16 + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i) load8(a[i], &As[(wm * FM * 32 + i * 32 + (lane & 31)) * LDK + kofs]);
#pragma unroll
      for (int j = 0; j < FN; ++j) load8(b[j], &Bs[(wn * FN * 32 + j * 32 + (lane & 31)) * LDK + kofs]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mma32(a[i], b[j], acc[i][j]);
    }
  }

  if (splits > 1) {
    float* P = partial + ((int64_t)(sp * p.batch + z) * p.M) * p.N;
    for (int i = 0; i < FM; ++i)
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * FN * 32 + j * 32 + (lane & 31);
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * FM * 32 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < p.M && col < p.N) P[(int64_t)row * p.N + col] = acc[i][j][r];
        }
      }
    return;
  }
  const bool tile_rope = n0 + BN > p.epi.rope_col0;  // uniform across the workgroup
  for (int i = 0; i < FM; ++i)
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * FN * 32 + j * 32 + (lane & 31);
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * FM * 32 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        float v = acc[i][j][r];
        if (tile_rope) {
          const float partner = __shfl_xor(v, 1, 64);
          if (row < p.M && col < p.N) rope_pair(p.epi, row, col, v, partner);
        }
        if (row < p.M && col < p.N) epi_store<T>(p.epi, z, row, col, v);
      }
    }
}

// Sums the split-K partials [splits][batch][M][N] and runs the epilogue; one thread per
// column pair so that RoPE pairs stay together.
template <typename T>
__global__ void __launch_bounds__(256)
    splitk_reduce_kernel(GemmParams p, int splits, const float* __restrict__ partial) {
  const int64_t pairs = (int64_t)p.batch * p.M * (p.N / 2);
  const int64_t stride = (int64_t)p.M * p.N * p.batch;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < pairs;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int cp = (int)(t % (p.N / 2));
    const int64_t zr = t / (p.N / 2);
    const int row = (int)(zr % p.M), z = (int)(zr / p.M);
    const int col = 2 * cp;
    const float* src = partial + ((int64_t)z * p.M + row) * p.N + col;
    float v0 = 0.f, v1 = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float2 v = *reinterpret_cast<const float2*>(src + s * stride);
      v0 += v.x;
      v1 += v.y;
    }
    const float e0 = v0, e1 = v1;
    rope_pair(p.epi, row, col, v0, e1);
    rope_pair(p.epi, row, col + 1, v1, e0);
    epi_store<T>(p.epi, z, row, col, v0);
    epi_store<T>(p.epi, z, row, col + 1, v1);
  }
}

// ----------------------------------------------------------------------------- host side
namespace {
struct Cfg {
  int bm, bn, wm, wn;
};
constexpr Cfg kCfgs[] = {{32, 128, 1, 4}, {64, 64, 2, 2}, {128, 128, 2, 2}};

template <typename T, int C>
hipError_t launch_cfg(const GemmParams& p, const GemmPlan& plan, float* partial, hipStream_t s) {
  constexpr Cfg c = kCfgs[C];
  const int tiles = ((p.M + c.bm - 1) / c.bm) * ((p.N + c.bn - 1) / c.bn);
  dim3 grid(tiles, p.batch * plan.splits);
  hipLaunchKernelGGL((gemm_kernel<T, c.bm, c.bn, c.wm, c.wn>), grid, dim3(64 * c.wm * c.wn), 0, s, p,
                     plan.splits, plan.k_per_split, partial);
  return hipGetLastError();
}

template <typename T>
hipError_t run_t(const GemmParams& p, const GemmPlan& plan, float* partial, hipStream_t s) {
  hipError_t err;
  switch (plan.cfg) {
    case 0: err = launch_cfg<T, 0>(p, plan, partial, s); break;
    case 1: err = launch_cfg<T, 1>(p, plan, partial, s); break;
    default: err = launch_cfg<T, 2>(p, plan, partial, s); break;
  }
  if (err != hipSuccess || plan.splits == 1) return err;
  const int64_t pairs = (int64_t)p.batch * p.M * (p.N / 2);
  const int blocks = (int)std::min<int64_t>((pairs + 255) / 256, 8192);
  hipLaunchKernelGGL(splitk_reduce_kernel<T>, dim3(blocks), dim3(256), 0, s, p, plan.splits, partial);
  return hipGetLastError();
}
}  // namespace

GemmPlan gemm_plan(int M, int N, int K, int batch, int cus) {
  GemmPlan pl;
  pl.cfg = M <= 32 ? 0 : (M <= 64 ? 1 : 2);
  pl.bm = kCfgs[pl.cfg].bm;
  pl.bn = kCfgs[pl.cfg].bn;
  const int64_t tiles = (int64_t)((M + pl.bm - 1) / pl.bm) * ((N + pl.bn - 1) / pl.bn) * batch;
  const int64_t want = 2LL * cus;
  int splits = 1;
  if (tiles < want && (N % 2) == 0) {
    splits = (int)((want + tiles - 1) / tiles);
    splits = std::min(splits, std::max(1, K / 256));
    splits = std::min(splits, 32);
  }
  int kps = ((K + splits - 1) / splits + kBK - 1) / kBK * kBK;
  splits = (K + kps - 1) / kps;
  pl.splits = std::max(1, splits);
  pl.k_per_split = pl.splits == 1 ? ((K + kBK - 1) / kBK) * kBK : kps;
  pl.partial_bytes = pl.splits > 1 ? (size_t)pl.splits * batch * M * N * sizeof(float) : 0;
  return pl;
}

size_t gemm_partial_bound(int M, int N, int K, int batch, int cus) {
  // every tile height is a multiple of 32, so within a 32-row bucket the split count is fixed
  // and the partial size grows with M: the bucket tops (and M itself) are the only candidates
  size_t best = 0;
  for (int m = 32; m < M + 32; m += 32) {
    const int mm = std::min(m, M);
    best = std::max(best, gemm_plan(mm, N, K, batch, cus).partial_bytes);
  }
  return best;
}

hipError_t gemm_run(DType t, const GemmParams& p, const GemmPlan& plan, float* partial, hipStream_t s) {
  if (p.M == 0 || p.N == 0 || p.batch == 0) return hipSuccess;
  return t == DType::BF16 ? run_t<bf16>(p, plan, partial, s) : run_t<float>(p, plan, partial, s);
}

}  // namespace mla
