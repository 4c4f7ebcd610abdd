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

// ----------------------------------------------------------------------------- skinny kernel
// Decode-sized products (M <= 64 rows, bf16, y = W x with W [N][K]) stream the weights once and
// are bound by HBM.  Each wave owns 32 output columns for all M rows:
//   * its weight rows come straight from global memory into registers, 64 contiguous bytes per
//     lane and k-step of 64 (two lanes per row cover the row's 128-byte line), three k-steps ahead;
//   * the activation slice of a k-step (M x 64) is copied once per workgroup into LDS by direct
//     global->LDS copies (four-stage ring, 16-byte chunks XOR-swizzled by row);
//   * the 32x32x16 MFMA k-slots are permuted so that lane group g owns k = 32g + 8j .. +7 in
//     sub-step j, which makes both operands' per-lane data contiguous.
namespace skinny {
constexpr int kKS = 64;      // k per step
constexpr int kWaves = 4;
constexpr int kBN = 32 * kWaves;
constexpr int kAStages = 4;
constexpr int kBStages = 4;  // register ring: steps s+1..s+3 in flight while s is multiplied
}  // namespace skinny

typedef __attribute__((address_space(3))) void lds_void_g;

template <int MB>
__device__ __forceinline__ void skinny_issue_a(const bf16* A, int64_t lda, int M, int k0, char* stage, int w,
                                               int lane) {
  // stage layout: row m (64 k = 128 bytes = 8 chunks), chunk c at slot c ^ (m & 7)
  constexpr int kInst = MB * 32 * 8 / 64;  // 1 KiB copies per workgroup (4 or 8)
#pragma unroll
  for (int i = 0; i < kInst / skinny::kWaves; ++i) {
    const int inst = w * (kInst / skinny::kWaves) + i;
    const int P = inst * 64 + lane;
    const int m = P >> 3, slot = P & 7;
    const int c = slot ^ (m & 7);
    const int mr = min(m, M - 1);  // rows past M copy a valid row; their results are dropped
    __builtin_amdgcn_global_load_lds((const void*)(A + (int64_t)mr * lda + k0 + c * 8),
                                     (lds_void_g*)(stage + inst * 1024), 16, 0, 0);
  }
}

template <int MB>
__global__ void __launch_bounds__(256)
    gemm_skinny_kernel(GemmParams p, int splits, int k_per_split, float* __restrict__ partial) {
  using namespace skinny;
  constexpr int kAStageBytes = MB * 32 * 128;
  constexpr int kAInstPerWave = MB * 32 * 8 / 64 / kWaves;  // 1 or 2
  __shared__ __attribute__((aligned(1024))) char As[kAStages][kAStageBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int n0 = blockIdx.x * kBN;
  const int z = blockIdx.y / splits, sp = blockIdx.y % splits;
  const int kb = sp * k_per_split, ke = min(p.K, kb + k_per_split);
  const int nsteps = (ke - kb) / kKS;

  const bf16* A = reinterpret_cast<const bf16*>(p.A) + (int64_t)z * p.strideA;
  // this lane's weight row (rows past N read row N-1; their columns are dropped)
  const int n = min(n0 + w * 32 + l32, p.N - 1);
  const bf16* brow = n < p.N0 ? reinterpret_cast<const bf16*>(p.B0) + (int64_t)z * p.strideB + (int64_t)n * p.ldb
                              : reinterpret_cast<const bf16*>(p.B1) + (int64_t)z * p.strideB + (int64_t)(n - p.N0) * p.ldb;
  brow += 32 * g;

  floatx16 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  bf16x8 bq[kBStages][4];
  // prologue: steps 0..2, each issued as [A copies, B loads] like every later step, so that the
  // wait for step t always leaves exactly the copies and loads of steps t+1 and t+2 in flight
#pragma unroll
  for (int s0 = 0; s0 < kBStages - 1; ++s0)
    if (s0 < nsteps) {
      skinny_issue_a<MB>(A, p.lda, p.M, kb + s0 * kKS, As[s0], w, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) bq[s0][j] = *reinterpret_cast<const bf16x8*>(brow + kb + s0 * kKS + 8 * j);
    }

  for (int s = 0; s < nsteps; s += kBStages) {
#pragma unroll
    for (int u = 0; u < kBStages; ++u) {
      const int st = s + u;
      if (st < nsteps) {
        // every step is issued as [A copies, B loads]; waiting until only the later steps'
        // (st+1, st+2, if they exist) copies and loads are outstanding completes step st
        const int later = min(nsteps - 1 - st, kBStages - 2);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (later >= 2) __builtin_amdgcn_s_waitcnt(((2 * (kAInstPerWave + 4)) & 0xF) | (((2 * (kAInstPerWave + 4)) >> 4) << 14) | (0xF << 8) | (0x7 << 4));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(((kAInstPerWave + 4) & 0xF) | (((kAInstPerWave + 4) >> 4) << 14) | (0xF << 8) | (0x7 << 4));
        else __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4));
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        // refill: the A stage of step st-1 (everyone is past it) and B slot of step st-1
        if (st + 3 < nsteps) {
          skinny_issue_a<MB>(A, p.lda, p.M, kb + (st + 3) * kKS, As[(u + 3) % kAStages], w, lane);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            bq[(u + 3) % kBStages][j] = *reinterpret_cast<const bf16x8*>(brow + kb + (st + 3) * kKS + 8 * j);
        }
        const char* as = As[u % kAStages];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          Frag8<bf16> bf;
          bf.v = bq[u][j];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const int m = mb * 32 + l32;
            Frag8<bf16> af;
            af.v = *reinterpret_cast<const bf16x8*>(as + m * 128 + (((4 * g + j) ^ (m & 7)) * 16));
            acc[mb] = mma32(af, bf, acc[mb]);
          }
        }
      }
    }
  }

  // C layout: lane col = n0 + w*32 + l32; value r at row mb*32 + 8*(r/4) + 4*g + r%4
  const int col = n0 + w * 32 + l32;
  if (splits > 1) {
    float* P = partial + ((int64_t)(sp * p.batch + z) * p.M) * p.N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row < p.M && col < p.N) P[(int64_t)row * p.N + col] = acc[mb][r];
      }
    return;
  }
  const bool tile_rope = n0 + kBN > p.epi.rope_col0;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = mb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      float v = acc[mb][r];
      if (tile_rope) {
        const float partner = __shfl_xor(v, 1, 64);
        if (row < p.M && col < p.N) rope_pair(p.epi, row, col, v, partner);
      }
      if (row < p.M && col < p.N) epi_store<bf16>(p.epi, z, row, col, v);
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
    case 3:
    case 4: {
      dim3 grid((p.N + skinny::kBN - 1) / skinny::kBN, p.batch * plan.splits);
      if (plan.cfg == 3)
        hipLaunchKernelGGL(gemm_skinny_kernel<1>, grid, dim3(256), 0, s, p, plan.splits, plan.k_per_split, partial);
      else
        hipLaunchKernelGGL(gemm_skinny_kernel<2>, grid, dim3(256), 0, s, p, plan.splits, plan.k_per_split, partial);
      err = hipGetLastError();
      break;
    }
    default: err = launch_cfg<T, 2>(p, plan, partial, s); break;
  }
  if (err != hipSuccess || plan.splits == 1) return err;
  const int64_t pairs = (int64_t)p.batch * p.M * (p.N / 2);
  const int blocks = (int)std::min<int64_t>((pairs + 255) / 256, 8192);
  hipLaunchKernelGGL(splitk_reduce_kernel<T>, dim3(blocks), dim3(256), 0, s, p, plan.splits, partial);
  return hipGetLastError();
}
}  // namespace

bool gemm_skinny_ok(DType t, const GemmParams& p) {
  return t == DType::BF16 && !p.nn && p.M <= 64 && p.K % skinny::kKS == 0 && p.N % 2 == 0 && p.lda % 8 == 0 &&
         p.ldb % 8 == 0 && p.strideA % 8 == 0 && p.strideB % 8 == 0;
}

GemmPlan gemm_plan_skinny(int M, int N, int K, int batch, int cus) {
  GemmPlan pl;
  pl.cfg = M <= 32 ? 3 : 4;
  pl.bm = M <= 32 ? 32 : 64;
  pl.bn = skinny::kBN;
  const int64_t tiles = (int64_t)((N + pl.bn - 1) / pl.bn) * batch;
  const int ksteps = K / skinny::kKS;
  // about two workgroups per CU, each streaming at least 8 k-steps
  int splits = (int)std::max<int64_t>(1, (2LL * cus + tiles - 1) / tiles);
  splits = std::min(splits, std::max(1, ksteps / 8));
  const int per = (ksteps + splits - 1) / splits;
  pl.splits = (ksteps + per - 1) / per;
  pl.k_per_split = per * skinny::kKS;
  pl.partial_bytes = pl.splits > 1 ? (size_t)pl.splits * batch * M * N * sizeof(float) : 0;
  return pl;
}

GemmPlan gemm_plan(int M, int N, int K, int batch, int cus, bool skinny_ok) {
  if (skinny_ok && M <= 64 && K % skinny::kKS == 0 && N % 2 == 0) return gemm_plan_skinny(M, N, K, batch, cus);
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

size_t gemm_partial_bound(int M, int N, int K, int batch, int cus, bool skinny_ok) {
  // every tile height is a multiple of 32, so within a 32-row bucket the split count is fixed
  // and the partial size grows with M: the bucket tops (and M itself) are the only candidates
  size_t best = 0;
  for (int m = 32; m < M + 32; m += 32) {
    const int mm = std::min(m, M);
    best = std::max(best, gemm_plan(mm, N, K, batch, cus, skinny_ok).partial_bytes);
  }
  return best;
}

hipError_t gemm_run(DType t, const GemmParams& p, const GemmPlan& plan, float* partial, hipStream_t s) {
  if (p.M == 0 || p.N == 0 || p.batch == 0) return hipSuccess;
  if ((plan.cfg == 3 || plan.cfg == 4) && (t != DType::BF16 || !gemm_skinny_ok(t, p))) return hipErrorInvalidValue;
  return t == DType::BF16 ? run_t<bf16>(p, plan, partial, s) : run_t<float>(p, plan, partial, s);
}

}  // namespace mla
