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
#include <numeric>

#include "common.h"
#include "internal.h"
#include "quant.h"
#include "units.h"

namespace mla {

constexpr int kBK = 32;  // k elements staged per iteration

// Rotation of one element of a RoPE pair by (cos, sin) = cs; partner is the pair's other element.
__device__ __forceinline__ float rope_rot(float v, float partner, float2 cs, bool odd) {
  return odd ? (partner * cs.y + v * cs.x) : (v * cs.x - partner * cs.y);
}
// (cos, sin) of RoPE column col (col >= e.rope_col0) in row `row`.
__device__ __forceinline__ float2 rope_cs(const Epilogue& e, int row, int col) {
  const int k = ((col - e.rope_col0) % e.d_hr) >> 1;
  return e.rope_tab[(int64_t)row * (e.d_hr >> 1) + k];
}
__device__ __forceinline__ void rope_pair(const Epilogue& e, int row, int col, float& v, float partner) {
  if (col >= e.rope_col0) v = rope_rot(v, partner, rope_cs(e, row, col), col & 1);
}

// Offset of column c within its output row: groups of e.group columns, group_stride apart.
__device__ __forceinline__ int64_t epi_col(const Epilogue& e, int c) {
  int j = c % e.group;
  if (e.perm16) j = (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);  // pieces 1 and 2 of 16 swap
  return (int64_t)(c / e.group) * e.group_stride + e.group_off + j;
}

template <typename T>
__device__ __forceinline__ void epi_store(const Epilogue& e, int z, int row, int col, float v) {
  int64_t rbase;
  if (e.block_table) {
    const int sq = e.row_seq ? e.row_seq[row] : row, ps = e.row_pos[row];
    const int64_t slot =
        (int64_t)e.block_table[(int64_t)sq * e.max_blocks + ps / e.block_size] * e.block_size +
        ps % e.block_size;
    rbase = slot * e.ldc;
  } else {
    rbase = (int64_t)row * e.ldc;
  }
  const int64_t idx = (int64_t)z * e.batch_stride + rbase + epi_col(e, col);
  if (e.c_f32)
    reinterpret_cast<float*>(e.C)[idx] = v;
  else
    reinterpret_cast<T*>(e.C)[idx] = from_f32<T>(v);
  if (e.C2) e.C2[idx] = v;
}

// The element (row, col) of the product through whichever epilogue owns the column; partner is
// the value of column col ^ 1 (RoPE pairs).
template <typename T>
__device__ __forceinline__ void out_elem(const GemmParams& p, int z, int row, int col, float v, float partner) {
  if (col >= p.E0) {
    rope_pair(p.epi2, row, col - p.E0, v, partner);
    epi_store<T>(p.epi2, z, row, col - p.E0, v);
  } else {
    rope_pair(p.epi, row, col, v, partner);
    epi_store<T>(p.epi, z, row, col, v);
  }
}

// Four consecutive columns col .. col+3 (col % 4 == 0) of one row through the epilogue; the
// values are already rotated.  One 8- or 16-byte store when the four land next to each other
// (no column group boundary inside), else element by element.  A paged epilogue's row position
// and sequence may be passed in (pos >= 0), read by the caller ahead of its other loads.
template <typename T>
__device__ __forceinline__ void out_quad(const GemmParams& p, int z, int row, int col, const float (&v)[4],
                                         int pos = -1, int seq = 0) {
  const bool hi = col >= p.E0;
  const Epilogue& e = hi ? p.epi2 : p.epi;
  const int c = hi ? col - p.E0 : col;
  if (c % e.group + 3 < e.group && (!e.perm16 || c % e.group % 4 == 0) && !e.c_f32 && !e.C2 && sizeof(T) == 2 &&
      (reinterpret_cast<uintptr_t>(e.C) & 7) == 0) {
    int64_t rbase;
    if (e.block_table) {
      const int sq = pos >= 0 ? seq : (e.row_seq ? e.row_seq[row] : row), ps = pos >= 0 ? pos : e.row_pos[row];
      rbase = ((int64_t)e.block_table[(int64_t)sq * e.max_blocks + ps / e.block_size] * e.block_size +
               ps % e.block_size) * e.ldc;
    } else {
      rbase = (int64_t)row * e.ldc;
    }
    const int64_t idx = (int64_t)z * e.batch_stride + rbase + epi_col(e, c);
    bf16x4 q = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(e.C) + idx) = q;
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) epi_store<T>(e, z, row, c + i, v[i]);
}

// Whether any column of [c0, c1) is rotated (so that partners must be exchanged).
__device__ __forceinline__ bool cols_have_rope(const GemmParams& p, int c0, int c1) {
  const int64_t lo_end = std::min<int64_t>(c1, p.E0);
  if (lo_end > std::max<int64_t>(c0, p.epi.rope_col0)) return true;
  return (int64_t)c1 > (int64_t)p.E0 + p.epi2.rope_col0;
}

// Row n of the stacked B operand ("NT" form).
template <typename T>
__device__ __forceinline__ const T* b_row(const GemmParams& p, int z, int n) {
  const void* base = n < p.N0 ? p.B0 : (n < p.N1 ? p.B1 : p.B2);
  const int r = n < p.N0 ? n : (n < p.N1 ? n - p.N0 : n - p.N1);
  return reinterpret_cast<const T*>(base) + (int64_t)z * p.strideB + (int64_t)r * p.ldb;
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
          v = ld16(b_row<T>(p, z, gn) + gk);
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
  const bool tile_rope = cols_have_rope(p, n0, n0 + BN);  // uniform across the workgroup
  for (int i = 0; i < FM; ++i)
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn * FN * 32 + j * 32 + (lane & 31);
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * FM * 32 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const float v = acc[i][j][r];
        const float partner = tile_rope ? __shfl_xor(v, 1, 64) : 0.f;
        if (row < p.M && col < p.N) out_elem<T>(p, z, row, col, v, partner);
      }
    }
}

// Sums the split-K partials [splits][batch][M][N] and runs the epilogue; a thread owns an even
// number of consecutive columns so that RoPE pairs stay together.
template <typename T, int V, int NF>
__global__ void __launch_bounds__(128)
    splitk_reduce_kernel(GemmParams p, int splits, const float* __restrict__ partial) {
  // one thread per V consecutive columns of one row; the splits are summed in order.  All the
  // partial loads of up to NF splits are issued before the first add: with a loop over a run-time
  // split count each load would wait for the previous add, one memory round trip per split (a
  // 14-way split then takes seven times the latency of one).  NF is the smallest of 2, 4, 8, 16
  // that covers the split count, so the registers, and with them the occupancy, follow it.
  constexpr int kInFlight = NF;
  typedef float vec_t __attribute__((ext_vector_type(V)));
  const int64_t groups = (int64_t)p.batch * p.M * (p.N / V);
  const int64_t stride = (int64_t)p.M * p.N * p.batch;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < groups;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int cg = (int)(t % (p.N / V));
    const int64_t zr = t / (p.N / V);
    const int row = (int)(zr % p.M), z = (int)(zr / p.M);
    const int col = V * cg;
    const float* src = partial + ((int64_t)z * p.M + row) * p.N + col;
    // the RoPE factors of the quad's two pairs are loaded ahead of the partials, so that their
    // round trip overlaps the partials' instead of following it
    float2 cs[2] = {};
    bool rot[2] = {false, false};
    int pos = -1, seq = 0;  // a paged epilogue's row position and sequence, read with them too
    if constexpr (V == 4) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bool hi = col + 2 * i >= p.E0;
        const Epilogue& e = hi ? p.epi2 : p.epi;
        const int c = hi ? col + 2 * i - p.E0 : col + 2 * i;
        rot[i] = c >= e.rope_col0;
        if (rot[i]) cs[i] = rope_cs(e, row, c);
      }
      const Epilogue& e = col >= p.E0 ? p.epi2 : p.epi;
      if (e.block_table) {
        pos = e.row_pos[row];
        seq = e.row_seq ? e.row_seq[row] : row;
      }
    }
    vec_t acc = {};
    for (int s = 0; s < splits; s += kInFlight) {
      vec_t v[kInFlight];
#pragma unroll
      for (int i = 0; i < kInFlight; ++i)
        if (s + i < splits) v[i] = *reinterpret_cast<const vec_t*>(src + (s + i) * stride);
#pragma unroll
      for (int i = 0; i < kInFlight; ++i)
        if (s + i < splits) acc += v[i];
    }
    if constexpr (V == 4) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        v[i] = rot[i / 2] ? rope_rot(acc[i], acc[i + 1], cs[i / 2], false) : acc[i];
        v[i + 1] = rot[i / 2] ? rope_rot(acc[i + 1], acc[i], cs[i / 2], true) : acc[i + 1];
      }
      out_quad<T>(p, z, row, col, v, pos, seq);
    } else {
#pragma unroll
      for (int i = 0; i < V; i += 2) {
        out_elem<T>(p, z, row, col + i, acc[i], acc[i + 1]);
        out_elem<T>(p, z, row, col + i + 1, acc[i + 1], acc[i]);
      }
    }
  }
}

// ----------------------------------------------------------------------------- skinny kernel
// Decode-sized products (M <= 64 rows, bf16, y = W x with W [N][K]) read every weight byte once
// and are bound by HBM.  A workgroup of four waves owns 128 output columns and one k range;
// each wave owns 32 of the columns.
//   Weights: each wave copies its own 32 rows straight into a private LDS ring of kNS 64-k
//     stages (kNS steps in flight), with a coalesced pattern: one copy instruction covers
//     eight whole 128-byte row segments.  Only the issuing wave reads a stage, so no barrier
//     is needed for them.  Reading weights with MFMA-fragment-shaped per-lane loads instead
//     touches four times as many cache lines per instruction and needs several times more
//     waves in flight to reach the same bandwidth.
//   Activations: shared by the four waves, copied in chunks of kChunk steps into a double
//     buffer, with one barrier per chunk.
// The LDS footprint (80 KiB) lets two workgroups share a compute unit.
// Both LDS images swizzle 16-byte chunks (slot = chunk ^ (row & 7)) so that fragment reads,
// 32 rows at one chunk, spread over all banks.  In sub-step j (16 k) of a step, lane group g
// supplies k-chunk 2j + g of the step to the 32x32x16 MFMA for both operands.
// The copies of steps and chunks past the end re-read the last one (in bounds, never used),
// so every wait below counts the same number of copies in flight.
namespace skinny {
constexpr int kKS = 64;                    // k per step: 128 bytes of a weight row
constexpr int kWaves = 4;
constexpr int kBN = 32 * kWaves;           // columns per workgroup
constexpr int kNS = 3;                     // weight stages per wave
constexpr int kChunk = 2;                  // steps per activation chunk
constexpr int kStage = 32 * 128;           // bytes of one wave's weight stage
constexpr int kBI = kStage / 1024;         // weight copy instructions per step (4)
constexpr int kAChunkRow = kChunk * kKS * 2;  // bytes of one activation row in a chunk
constexpr int kARowsPerCopy = 1024 / kAChunkRow;
constexpr int kPeriod = kNS * 2 * kChunk / std::gcd(kNS, 2 * kChunk);  // steps unrolled
// the step waits below assume the ring never holds steps of more than two chunks
static_assert(kNS - 1 <= kChunk, "ring deeper than a chunk");
static_assert(kPeriod % kNS == 0 && kPeriod % (2 * kChunk) == 0, "unroll period");
// activation copies per wave per chunk for MB row blocks
template <int MB>
constexpr int a_copies() { return MB * 32 * kAChunkRow / (1024 * kWaves); }
// activation chunks issued after weight step s (position q in its chunk) was issued and before
// step s waits for it: multiples of kChunk in (s - kNS + 1, s]
constexpr int a_after_b(int q) {
  return (q >= 0 ? q / kChunk : -((-q + kChunk - 1) / kChunk)) -
         ((q - kNS + 1) >= 0 ? (q - kNS + 1) / kChunk : -((-(q - kNS + 1) + kChunk - 1) / kChunk));
}
}  // namespace skinny

__shared__ __attribute__((aligned(1024))) char g_sk_a0[64 * skinny::kAChunkRow];
__shared__ __attribute__((aligned(1024))) char g_sk_a1[64 * skinny::kAChunkRow];
__shared__ __attribute__((aligned(1024))) char g_sk_b[skinny::kNS][skinny::kWaves * skinny::kStage];

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
template <int AB>
__device__ __forceinline__ char* sk_abuf() { return AB == 0 ? g_sk_a0 : g_sk_a1; }
template <int ST>
__device__ __forceinline__ char* sk_bbuf() { return g_sk_b[ST]; }

struct SkinnyCtx {
  const bf16* a;        // activation row 0 of this batch at k = kb
  int64_t lda;
  int M, nsteps, nchunks;
  const bf16* brow[skinny::kBI];  // this lane's weight row of copy i, at k = kb + its chunk
  int w, lane;
};

// Activation chunk c (clamped to the last one) into buffer AB: MB*32 rows x kAChunkRow bytes;
// copy instruction p of the workgroup covers kARowsPerCopy whole row segments.
template <int MB, int AB>
__device__ __forceinline__ void sk_issue_a(const SkinnyCtx& x, int c) {
  using namespace skinny;
  constexpr int CPR = kAChunkRow / 16;  // 16-byte chunks per row segment
  c = min(c, x.nchunks - 1);
  char* dst = sk_abuf<AB>();
  const int slot = x.lane % CPR;
#pragma unroll
  for (int i = 0; i < a_copies<MB>(); ++i) {
    const int p = i * kWaves + x.w;
    const int row = p * kARowsPerCopy + x.lane / CPR;
    const int ch = slot ^ (row & 7);                  // 16-byte chunk of the row segment
    // the last chunk may hold fewer steps: clamp its k inside the k range
    const int kk = min(c * (kChunk * kKS) + ch * 8, (x.nsteps - 1) * kKS + (ch & 7) * 8);
    const bf16* src = x.a + (int64_t)min(row, x.M - 1) * x.lda + kk;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(dst + p * 1024), 16, 0, 0);
  }
}

// Weight step s (clamped to the last one) into this wave's part of stage ST.
template <int ST>
__device__ __forceinline__ void sk_issue_b(const SkinnyCtx& x, int s) {
  using namespace skinny;
  s = min(s, x.nsteps - 1);
  char* dst = sk_bbuf<ST>() + x.w * kStage;
#pragma unroll
  for (int i = 0; i < kBI; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(x.brow[i] + s * kKS), (lds_void_t*)(dst + i * 1024), 16, 0, 0);
}

// One step (s = position U of the unrolled period): the copies that refill the ring, waits,
// and 4 x MB MFMAs.
//   At a chunk's first step, activation chunk c must have landed for every wave: after it this
//   wave issued kNS - 1 weight steps (prologue, c = 0) or the kChunk weight steps of chunk c-1.
//   Step s's weight copy is followed by the kNS - 1 later weight steps and a_after_b(q)
//   activation chunks.
template <int MB, int U>
__device__ __forceinline__ void sk_step(const SkinnyCtx& x, int s, floatx16 (&acc)[MB]) {
  using namespace skinny;
  constexpr int ST = U % kNS, AB = (U / kChunk) % 2, Q = U % kChunk;
  if (Q == 0) {
    if (s == 0) MLA_TILE_BARRIER(waitcnt_vm((kNS - 1) * kBI));
    else MLA_TILE_BARRIER(waitcnt_vm(kChunk * kBI));
    sk_issue_a<MB, 1 - AB>(x, s / kChunk + 1);
  }
  // stage (ST + kNS - 1) % kNS was last read in step s - 1, whose reads have completed
  sk_issue_b<(ST + kNS - 1) % kNS>(x, s + kNS - 1);
  MLA_WAVE_WAIT(waitcnt_vm((kNS - 1) * kBI + a_after_b(Q) * a_copies<MB>()));

  // Fragment reads.  The compiler would make every LDS read that follows a direct-to-LDS copy
  // wait for all copies in flight, which serialises the ring; the reads and their wait are one
  // asm block instead, ordered after the waits above (outputs early-clobber: every read is in
  // flight before the first result lands).
  int lane = x.lane;
  asm volatile("" : "+v"(lane));
  const int g = lane >> 5, l32 = lane & 31, x7 = l32 & 7;
  const uint32_t bb = lds_addr(sk_bbuf<ST>()) + x.w * kStage + l32 * 128;
  const uint32_t ab = lds_addr(sk_abuf<AB>()) + l32 * kAChunkRow + Q * 128;
  uint32_t sw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sw[j] = ((2 * j + g) ^ x7) * 16;
  bf16x8 bq[4], aq[MB][4];
  if constexpr (MB == 1) {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(bq[0]), "=&v"(bq[1]), "=&v"(bq[2]), "=&v"(bq[3]), "=&v"(aq[0][0]), "=&v"(aq[0][1]), "=&v"(aq[0][2]),
          "=&v"(aq[0][3])
        : "v"(bb + sw[0]), "v"(bb + sw[1]), "v"(bb + sw[2]), "v"(bb + sw[3]), "v"(ab + sw[0]), "v"(ab + sw[1]),
          "v"(ab + sw[2]), "v"(ab + sw[3]));
  } else {
    // rows 32 + l32 of the activation chunk share (row & 7) with l32: same swizzle, 32 rows on
    asm volatile(
        "ds_read_b128 %0, %12\n\tds_read_b128 %1, %13\n\tds_read_b128 %2, %14\n\tds_read_b128 %3, %15\n\t"
        "ds_read_b128 %4, %16\n\tds_read_b128 %5, %17\n\tds_read_b128 %6, %18\n\tds_read_b128 %7, %19\n\t"
        "ds_read_b128 %8, %16 offset:%20\n\tds_read_b128 %9, %17 offset:%20\n\t"
        "ds_read_b128 %10, %18 offset:%20\n\tds_read_b128 %11, %19 offset:%20\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(bq[0]), "=&v"(bq[1]), "=&v"(bq[2]), "=&v"(bq[3]), "=&v"(aq[0][0]), "=&v"(aq[0][1]), "=&v"(aq[0][2]),
          "=&v"(aq[0][3]), "=&v"(aq[1][0]), "=&v"(aq[1][1]), "=&v"(aq[1][2]), "=&v"(aq[1][3])
        : "v"(bb + sw[0]), "v"(bb + sw[1]), "v"(bb + sw[2]), "v"(bb + sw[3]), "v"(ab + sw[0]), "v"(ab + sw[1]),
          "v"(ab + sw[2]), "v"(ab + sw[3]), "n"(32 * kAChunkRow));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    Frag8<bf16> bf;
    bf.v = bq[j];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      Frag8<bf16> af;
      af.v = aq[mb][j];
      acc[mb] = mma32(af, bf, acc[mb]);
    }
  }
}

// The first kNS - 1 weight stages.
template <int ST>
__device__ __forceinline__ void sk_prologue_b(const SkinnyCtx& x) {
  if constexpr (ST < skinny::kNS - 1) {
    sk_issue_b<ST>(x, ST);
    sk_prologue_b<ST + 1>(x);
  }
}

// Steps s .. s + kPeriod - 1 with compile-time ring, buffer and chunk positions.
template <int MB, int U>
__device__ __forceinline__ void sk_period(const SkinnyCtx& x, int s, floatx16 (&acc)[MB]) {
  if constexpr (U < skinny::kPeriod) {
    if (s + U < x.nsteps) {
      sk_step<MB, U>(x, s + U, acc);
      sk_period<MB, U + 1>(x, s, acc);
    }
  }
}

template <int MB>
__global__ void __launch_bounds__(256)
    gemm_skinny_kernel(GemmParams p, int splits, int k_per_split, float* __restrict__ partial) {
  using namespace skinny;
  const int tid = threadIdx.x, lane = tid & 63;
  if (p.side_rope.tab && blockIdx.x == gridDim.x - 1) {  // the extra column: the RoPE table
    const RopeJob& r = p.side_rope;
    for (int64_t i = blockIdx.y * (int64_t)blockDim.x + tid; i < (int64_t)r.n * r.half;
         i += (int64_t)gridDim.y * blockDim.x)
      r.tab[i] = rope_table_entry(r.pos, r.half, r.f, i);
    return;
  }
  const int w = tid >> 6;
  const int n0 = blockIdx.x * kBN;
  const int z = blockIdx.y / splits, sp = blockIdx.y % splits;
  const int kb = sp * k_per_split, ke = min(p.K, kb + k_per_split);

  SkinnyCtx x;
  x.a = reinterpret_cast<const bf16*>(p.A) + (int64_t)z * p.strideA + kb;
  x.lda = p.lda;
  x.M = p.M;
  x.nsteps = (ke - kb) / kKS;
  x.nchunks = (x.nsteps + kChunk - 1) / kChunk;
  x.w = w;
  x.lane = lane;
  {
    const int r8 = lane >> 3;                      // row within the copy's 8 rows
    const int ch = (lane & 7) ^ r8;                // 16-byte chunk this lane copies
#pragma unroll
    for (int i = 0; i < kBI; ++i) {
      // rows past N copy row N - 1; their columns are dropped
      const int n = min(n0 + w * 32 + 8 * i + r8, p.N - 1);
      x.brow[i] = b_row<bf16>(p, z, n) + kb + ch * 8;
    }
  }

  floatx16 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  if (x.nsteps > 0) {
    sk_issue_a<MB, 0>(x, 0);
    sk_prologue_b<0>(x);
    for (int s = 0; s < x.nsteps; s += kPeriod) sk_period<MB, 0>(x, s, acc);
    // the ring's last copies (re-reads past the end) must land before the LDS is released
    MLA_WAVE_WAIT(waitcnt_vm(0));
  }

  // C layout: lane col = n0 + w*32 + l32; value r at row mb*32 + 8*(r/4) + 4*g + r%4
  const int g = lane >> 5;
  const int col = n0 + w * 32 + (lane & 31);
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
  const bool tile_rope = cols_have_rope(p, n0, n0 + kBN);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = mb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      const float v = acc[mb][r];
      const float partner = tile_rope ? __shfl_xor(v, 1, 64) : 0.f;
      if (row < p.M && col < p.N) out_elem<bf16>(p, z, row, col, v, partner);
    }
}

// ----------------------------------------------------------------------------- large-M kernel
// Prefill-sized bf16 "NT" products (M in the thousands).  A workgroup of eight waves computes a
// 256 x 256 tile, each wave 128 x 64 (4 x 2 blocks of 32x32x16 MFMA).  Both operands arrive by
// direct global->LDS copies into two 64-k stages (the next stage's copies in flight while the
// current one is multiplied), one barrier per stage; inside a stage the fragment reads of its
// second half run while its first half is multiplied.  LDS rows are 128 bytes (eight 16-byte
// chunks); chunk c of row r sits in slot c ^ ((r >> 1) & 7), which keeps the 16-byte fragment
// reads free of bank conflicts.
namespace big {
constexpr int kTileM = 256, kTileN = 256, kStepK = 64;
constexpr int kWaves = 8;                     // 2 (rows) x 4 (columns)
constexpr int kFM = 4, kFN = 2;               // 32-blocks per wave
constexpr int kRowB = kStepK * 2;             // bytes per LDS row
constexpr int kOp = kTileM * kRowB;           // 32 KiB per operand per stage
constexpr int kCopies = kOp / 1024 / kWaves;  // 4 copy instructions per operand per wave
constexpr int kGroupM = 4;                    // tile rows per group of the tile order
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
}  // namespace big

__shared__ __attribute__((aligned(1024))) char g_big_s0[2 * big::kOp];
__shared__ __attribute__((aligned(1024))) char g_big_s1[2 * big::kOp];
template <int ST>
__device__ __forceinline__ char* big_stage() { return ST == 0 ? g_big_s0 : g_big_s1; }

struct BigCtx {
  const bf16* a[big::kCopies];  // this lane's source of A copy i at k = 0
  const bf16* b[big::kCopies];
  int w, lane;
};

// The copy as one asm statement (M0 = the LDS destination), which the compiler does not track: the
// fragment reads of the other stage then need no wait for these copies (the barrier's own wait on
// the vector memory counter covers them).
__device__ __forceinline__ void big_copy(const void* src, const void* lds_dst) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_dst;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(m0)
               : "memory", "m0");
}

template <int ST>
__device__ __forceinline__ void big_issue(const BigCtx& x, int step) {
  using namespace big;
  char* st = big_stage<ST>();
  const int k = step * kStepK;
#pragma unroll
  for (int i = 0; i < kCopies; ++i) {
    const int P = i * kWaves + x.w;
    big_copy(x.a[i] + k, st + P * 1024);
    big_copy(x.b[i] + k, st + kOp + P * 1024);
  }
}

// Fragments of two 16-k sub-steps (2h, 2h + 1) of stage ST, as plain LDS reads (the copies are
// untracked asm, so the compiler's waits concern these reads only).
struct BigHalf {
  bf16x8 a[2][big::kFM], b[2][big::kFN];
};
template <int ST>
__device__ __forceinline__ void big_read(const BigCtx& x, int h, BigHalf& f) {
  using namespace big;
  int lane = x.lane;
  asm volatile("" : "+v"(lane));
  const int g = lane >> 5, l32 = lane & 31, sw = swz(l32);
  const int wm = x.w >> 2, wn = x.w & 3;
  const char* st = big_stage<ST>();
  const int s0 = ((4 * h + g) ^ sw) * 16, s1 = ((4 * h + 2 + g) ^ sw) * 16;
  const char* pa = st + (wm * 128 + l32) * kRowB;
  const char* pb = st + kOp + (wn * 64 + l32) * kRowB;
#pragma unroll
  for (int fm = 0; fm < kFM; ++fm) {
    f.a[0][fm] = *reinterpret_cast<const bf16x8*>(pa + fm * 4096 + s0);
    f.a[1][fm] = *reinterpret_cast<const bf16x8*>(pa + fm * 4096 + s1);
  }
#pragma unroll
  for (int fn = 0; fn < kFN; ++fn) {
    f.b[0][fn] = *reinterpret_cast<const bf16x8*>(pb + fn * 4096 + s0);
    f.b[1][fn] = *reinterpret_cast<const bf16x8*>(pb + fn * 4096 + s1);
  }
}
__device__ __forceinline__ void big_mfma(const BigHalf& f, floatx16 (&acc)[big::kFM][big::kFN]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int fm = 0; fm < big::kFM; ++fm)
#pragma unroll
      for (int fn = 0; fn < big::kFN; ++fn) {
        Frag8<bf16> a, b;
        a.v = f.a[t][fm];
        b.v = f.b[t][fn];
        acc[fm][fn] = mma32(a, b, acc[fm][fn]);
      }
}

// One 64-k stage: the second half's fragments are read while the first half is multiplied.
template <int ST>
__device__ __forceinline__ void big_step(const BigCtx& x, int s, int nsteps, floatx16 (&acc)[big::kFM][big::kFN]) {
  MLA_TILE_BARRIER(waitcnt_vm_lgkm0(0));  // this stage's copies have landed, the other stage is free
  if (s + 1 < nsteps) big_issue<1 - ST>(x, s + 1);
  BigHalf f0, f1;
  big_read<ST>(x, 0, f0);
  big_read<ST>(x, 1, f1);
  big_mfma(f0, acc);
  big_mfma(f1, acc);
}

// Row base (element offset of the row's start) of an epilogue.
__device__ __forceinline__ int64_t epi_row_base(const Epilogue& e, int row) {
  if (e.block_table) {
    const int sq = e.row_seq ? e.row_seq[row] : row, ps = e.row_pos[row];
    return ((int64_t)e.block_table[(int64_t)sq * e.max_blocks + ps / e.block_size] * e.block_size +
            ps % e.block_size) * e.ldc;
  }
  return (int64_t)row * e.ldc;
}

// With splits > 1, workgroup z-index `split` multiplies k in [split kps, (split + 1) kps) and stores
// its raw fp32 sums into partial[split][batch][M][N] for the split-K reduce pass, which runs the
// epilogue.
__global__ void __launch_bounds__(512) gemm_big_kernel(GemmParams p, int splits, int kps, float* __restrict__ partial) {
  using namespace big;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles_m = (p.M + kTileM - 1) / kTileM, tiles_n = (p.N + kTileN - 1) / kTileN;
  // Tile order: workgroups are dealt to the 8 XCDs in turn, so block b runs on XCD b % 8.  Give
  // each XCD a contiguous range of the tile order, and walk that order in groups of kGroupM tile
  // rows (column by column inside a group): the workgroups resident on one XCD then share a few
  // A and B panels in that XCD's L2.
  int t;
  {
    const int T = tiles_m * tiles_n, b = blockIdx.x, xcd = b & 7, local = b >> 3;
    const int per = T >> 3, extra = T & 7;
    t = xcd * per + min(xcd, extra) + local;
  }
  int m_t, n_t;
  {
    const int span = kGroupM * tiles_n, grp = t / span, in = t % span;
    const int gm = min(kGroupM, tiles_m - grp * kGroupM);
    m_t = grp * kGroupM + in % gm;
    n_t = in / gm;
  }
  const int m0 = m_t * kTileM, n0 = n_t * kTileN;
  const int z = blockIdx.y, split = blockIdx.z;
  const int k0 = split * kps, k1 = min(p.K, k0 + kps);  // a multiple of kStepK each
  BigCtx x;
  x.w = w;
  x.lane = lane;
  {
    const bf16* A = reinterpret_cast<const bf16*>(p.A) + (int64_t)z * p.strideA;
#pragma unroll
    for (int i = 0; i < kCopies; ++i) {
      const int row = (i * kWaves + w) * 8 + (lane >> 3);  // tile row of this lane's copy
      const int ch = (lane & 7) ^ swz(row);                 // source chunk landing in slot lane & 7
      x.a[i] = A + (int64_t)min(m0 + row, p.M - 1) * p.lda + k0 + ch * 8;
      x.b[i] = b_row<bf16>(p, z, min(n0 + row, p.N - 1)) + k0 + ch * 8;
    }
  }
  floatx16 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int nsteps = (k1 - k0) / kStepK;
  big_issue<0>(x, 0);
  for (int s = 0; s < nsteps; s += 2) {
    big_step<0>(x, s, nsteps, acc);
    if (s + 1 < nsteps) big_step<1>(x, s + 1, nsteps, acc);
  }

  if (splits > 1) {  // the raw sums (uniform: the whole workgroup returns here)
    const int g = lane >> 5, l32 = lane & 31;
    const int wm = w >> 2, wn = w & 3;
    float* out = partial + ((int64_t)split * p.batch + z) * p.M * p.N;
#pragma unroll
    for (int fm = 0; fm < kFM; ++fm)
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn) {
        const int col = n0 + wn * 64 + fn * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 128 + fm * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (row < p.M && col < p.N) out[(int64_t)row * p.N + col] = acc[fm][fn][r];
        }
      }
    return;
  }
  // Epilogue through LDS, half a wave block (64 x 64) at a time, in the wave's own 16 KiB: the
  // accumulators are only ever indexed by constants (a loop over them that is too long to unroll
  // would move them to scratch memory).  On the way out each lane owns one column, so the column's
  // part of the address is worked out once and the row's part is shared by the wave.
  __syncthreads();  // every wave is done with the operand stages
  const int g = lane >> 5, l32 = lane & 31;
  const int wm = w >> 2, wn = w & 3;
  float* ep = reinterpret_cast<float*>((w < 4 ? g_big_s0 : g_big_s1) + (w & 3) * 16384);
  const int col = n0 + wn * 64 + lane;
  const bool hi = col >= p.E0;
  const int c = hi ? col - p.E0 : col;
  // this lane's epilogue fields, picked once (the two epilogues are kernel arguments)
  const int64_t col_off = (int64_t)z * (hi ? p.epi2.batch_stride : p.epi.batch_stride) + epi_col(hi ? p.epi2 : p.epi, c);
  const int e_rope0 = hi ? p.epi2.rope_col0 : p.epi.rope_col0, e_dhr = hi ? p.epi2.d_hr : p.epi.d_hr;
  const float2* e_tab = hi ? p.epi2.rope_tab : p.epi.rope_tab;
  const bool rot = c >= e_rope0;
  const int rk = rot ? ((c - e_rope0) % e_dhr) >> 1 : 0;
  void* e_C = hi ? p.epi2.C : p.epi.C;
  float* e_C2 = hi ? p.epi2.C2 : p.epi.C2;
  const bool e_f32 = hi ? p.epi2.c_f32 : p.epi.c_f32;
  const bool col_ok = col < p.N;
  // The vector path: every group of four columns lies in one epilogue's range and one of its
  // column groups, its RoPE pairs start at even columns, and rows of 4 elements are aligned.
  const bool vec4 = p.N % 4 == 0 && (p.E0 >= p.N || p.E0 % 4 == 0) && p.epi.group % 4 == 0 &&
                    p.epi2.group % 4 == 0 && p.epi.ldc % 4 == 0 && p.epi2.ldc % 4 == 0 &&
                    p.epi.group_stride % 4 == 0 && p.epi2.group_stride % 4 == 0 &&
                    p.epi.group_off % 4 == 0 && p.epi2.group_off % 4 == 0 && p.epi.batch_stride % 4 == 0 &&
                    p.epi2.batch_stride % 4 == 0 && (p.epi.rope_tab == nullptr || p.epi.rope_col0 % 4 == 0) &&
                    (p.epi2.rope_tab == nullptr || p.epi2.rope_col0 % 4 == 0) &&
                    p.epi.d_hr % 4 == 0 && p.epi2.d_hr % 4 == 0;
  // this lane's fields for the vector path: columns v_col .. v_col + 3
  const int v_col = n0 + wn * 64 + 4 * (lane & 15);
  const bool v_hi = v_col >= p.E0;
  const int v_c = v_hi ? v_col - p.E0 : v_col;
  const Epilogue& ve = v_hi ? p.epi2 : p.epi;
  const int64_t v_off = (int64_t)z * ve.batch_stride + epi_col(ve, v_c);  // 4 columns stay together
  const bool v_rot = ve.rope_tab != nullptr && v_c >= ve.rope_col0;
  const int v_dhr = ve.d_hr;
  const int v_rk = v_rot ? ((v_c - ve.rope_col0) % v_dhr) >> 1 : 0;
  const float2* v_tab = ve.rope_tab;
  void* v_C = ve.C;
  float* v_C2 = ve.C2;
  const bool v_f32 = ve.c_f32;
  const bool v_ok = v_col < p.N;
  // Eight columns per lane (one 16-byte store, 8 rows per instruction) where the layout allows it:
  // bf16 outputs without an fp32 copy or the Vt key order, every group of 8 columns in one range.
  const bool vec8 = vec4 && p.N % 8 == 0 && (p.E0 >= p.N || p.E0 % 8 == 0) && p.epi.group % 8 == 0 &&
                    p.epi2.group % 8 == 0 && p.epi.ldc % 8 == 0 && p.epi2.ldc % 8 == 0 &&
                    p.epi.group_stride % 8 == 0 && p.epi2.group_stride % 8 == 0 && p.epi.group_off % 8 == 0 &&
                    p.epi2.group_off % 8 == 0 && p.epi.batch_stride % 8 == 0 && p.epi2.batch_stride % 8 == 0 &&
                    (p.epi.rope_tab == nullptr || p.epi.rope_col0 % 8 == 0) &&
                    (p.epi2.rope_tab == nullptr || p.epi2.rope_col0 % 8 == 0) && p.epi.d_hr % 8 == 0 &&
                    p.epi2.d_hr % 8 == 0 && !p.epi.perm16 && !p.epi2.perm16 && !p.epi.c_f32 && !p.epi2.c_f32 &&
                    !p.epi.C2 && !p.epi2.C2 && (reinterpret_cast<uintptr_t>(p.epi.C) & 15) == 0 &&
                    (p.E0 >= p.N || (reinterpret_cast<uintptr_t>(p.epi2.C) & 15) == 0);
  const int w_col = n0 + wn * 64 + 8 * (lane & 7);
  const bool w_hi = w_col >= p.E0;
  const int w_c = w_hi ? w_col - p.E0 : w_col;
  const Epilogue& we = w_hi ? p.epi2 : p.epi;
  const int64_t w_off = (int64_t)z * we.batch_stride + epi_col(we, w_c);
  const bool w_rot = we.rope_tab != nullptr && w_c >= we.rope_col0;
  const int w_rk = w_rot ? ((w_c - we.rope_col0) % we.d_hr) >> 1 : 0;
  const bool w_ok = w_col < p.N;
  // element (lr, lc) at lr*64 + (lc ^ 32*((lr >> 2) & 1)): the two row groups one write covers
  // land in different banks
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int fn = 0; fn < kFN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = f * 32 + 8 * (r >> 2) + 4 * g + (r & 3), lc = fn * 32 + l32;
          ep[lr * 64 + (lc ^ (((lr >> 2) & 1) << 5))] = acc[2 * h + f][fn][r];
        }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_wave_barrier();
    const int row0 = m0 + wm * 128 + h * 64;
    const int nrows = min(64, p.M - row0);
    if (vec8) {
      const int rq = lane >> 3, cq = 8 * (lane & 7);
      for (int lr = rq; lr < nrows; lr += 8) {
        const int sw = ((lr >> 2) & 1) << 5;
        floatx4 a = *reinterpret_cast<const floatx4*>(&ep[lr * 64 + (cq ^ sw)]);
        floatx4 b = *reinterpret_cast<const floatx4*>(&ep[lr * 64 + ((cq + 4) ^ sw)]);
        const int row = row0 + lr;
        if (w_rot) {
          const float2* tb = we.rope_tab + (int64_t)row * (we.d_hr >> 1) + w_rk;
          const float4 c0 = *reinterpret_cast<const float4*>(tb), c1 = *reinterpret_cast<const float4*>(tb + 2);
          a = floatx4{a[0] * c0.x - a[1] * c0.y, a[1] * c0.x + a[0] * c0.y, a[2] * c0.z - a[3] * c0.w,
                      a[3] * c0.z + a[2] * c0.w};
          b = floatx4{b[0] * c1.x - b[1] * c1.y, b[1] * c1.x + b[0] * c1.y, b[2] * c1.z - b[3] * c1.w,
                      b[3] * c1.z + b[2] * c1.w};
        }
        if (w_ok) {
          const int64_t idx = epi_row_base(we, row) + w_off;
          bf16x8 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o[i] = from_f32<bf16>(a[i]);
            o[4 + i] = from_f32<bf16>(b[i]);
          }
          *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(we.C) + idx) = o;
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();
      continue;
    }
    if (vec4) {
      // four consecutive columns and one of four rows per lane: 8- (or 16-) byte stores, RoPE
      // pairs inside the lane
      const int rq = lane >> 4, cq = 4 * (lane & 15);
      for (int lr = rq; lr < nrows; lr += 4) {
        const int sw = ((lr >> 2) & 1) << 5;
        floatx4 v = *reinterpret_cast<const floatx4*>(&ep[lr * 64 + (cq ^ sw)]);
        const int row = row0 + lr;
        if (v_rot) {
          const float4 cs = *reinterpret_cast<const float4*>(&v_tab[(int64_t)row * (v_dhr >> 1) + v_rk]);
          const float a0 = v[0] * cs.x - v[1] * cs.y, a1 = v[1] * cs.x + v[0] * cs.y;
          const float b0 = v[2] * cs.z - v[3] * cs.w, b1 = v[3] * cs.z + v[2] * cs.w;
          v = floatx4{a0, a1, b0, b1};
        }
        if (v_ok) {
          const int64_t idx = epi_row_base(v_hi ? p.epi2 : p.epi, row) + v_off;
          if (v_f32) {
            *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(v_C) + idx) = v;
          } else {
            bf16x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = from_f32<bf16>(v[i]);
            *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(v_C) + idx) = o;
          }
          if (v_C2) *reinterpret_cast<floatx4*>(v_C2 + idx) = v;
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_wave_barrier();
      continue;
    }
    const int my_row = min(row0 + lane, p.M - 1);
    const int64_t rb_lo = epi_row_base(p.epi, my_row);
    const int64_t rb_hi = p.E0 < p.N ? epi_row_base(p.epi2, my_row) : 0;
    for (int lr = 0; lr < nrows; ++lr) {
      const int sw = ((lr >> 2) & 1) << 5;
      float v = ep[lr * 64 + (lane ^ sw)];
      const int64_t lo = (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)rb_lo, lr) |
                         ((int64_t)__builtin_amdgcn_readlane((int)(rb_lo >> 32), lr) << 32);
      const int64_t hib = (int64_t)(uint32_t)__builtin_amdgcn_readlane((int)rb_hi, lr) |
                          ((int64_t)__builtin_amdgcn_readlane((int)(rb_hi >> 32), lr) << 32);
      if (rot) {
        const float partner = ep[lr * 64 + ((lane ^ 1) ^ sw)];
        const float2 cs = e_tab[(int64_t)(row0 + lr) * (e_dhr >> 1) + rk];
        v = (c & 1) ? (partner * cs.y + v * cs.x) : (v * cs.x - partner * cs.y);
      }
      if (col_ok) {
        const int64_t idx = (hi ? hib : lo) + col_off;
        if (e_f32)
          reinterpret_cast<float*>(e_C)[idx] = v;
        else
          reinterpret_cast<bf16*>(e_C)[idx] = from_f32<bf16>(v);
        if (e_C2) e_C2[idx] = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_wave_barrier();
  }
}

// ----------------------------------------------------------------------------- W_UK absorption
// q_hat[b][h][c] = sum_k q^C[b][h][k] W_UK[h*d_h + k][c] (App. C, W_UK folded into the query):
// per head a product whose weight operand has its output dimension contiguous, so the
// k-contiguous fragments the MFMA takes come from an LDS copy of the weight slice read with
// ds_read_b64_tr_b16 (16 lanes read a 4 (k) x 16 (c) block and each lane receives one column).
// Workgroup = (128-column slice of d_c, head): its d_h x 128 weight slice is copied to LDS once
// and serves every batch row; 4 waves of 32 columns each; the head's queries are copied to LDS
// in blocks of 64 batch rows.
namespace absorb {
constexpr int kCols = 128;  // columns of d_c per workgroup
constexpr int kDh = 128;    // d_h (both operands' LDS rows are 256 bytes = 16 chunks)
constexpr int kRowB = 256;
constexpr int kMB = 64;     // batch rows per block
constexpr int kWaves = 4;
// weight row r, chunk c at slot c ^ (2 (r & 3)): the four rows one transposed read covers fall
// in distinct banks; query row m, chunk c at slot c ^ (m & 15): the 16 rows one fragment read
// covers fall in distinct banks
__device__ __forceinline__ int wslot(int r, int c) { return c ^ ((r & 3) << 1); }
__device__ __forceinline__ int qslot(int m, int c) { return c ^ (m & 15); }
}  // namespace absorb

// With a units job (u_rows == 1) grid row 0 builds the decode attention's balanced work-unit table
// (workgroup x = 0; the others of the row return).  The next q_rows rows are the quantiser's: wave
// wv of workgroup (x, y) quantises new entry (y' gridDim.x + x) kWaves + wv of the job, y' = y -
// u_rows.  Both kinds of rows come first, so that their few workgroups start with the launch
// instead of trailing it.
__global__ void __launch_bounds__(256) absorb_kernel(const bf16* __restrict__ qc, const bf16* __restrict__ w,
                                                     bf16* __restrict__ out, int B, int n_h, int d_c,
                                                     int64_t out_ld, int64_t out_hs, QuantJob qj, int q_rows,
                                                     DecodeAttnParams uj, int u_rows) {
  using namespace absorb;
  __shared__ __attribute__((aligned(1024))) char lw[kDh * kRowB];
  __shared__ __attribute__((aligned(1024))) char lq[kMB * kRowB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  if ((int)blockIdx.y < u_rows) {  // the whole workgroup (one synchronisation inside)
    if (blockIdx.x == 0) build_decode_units(uj);
    return;
  }
  if ((int)blockIdx.y < u_rows + q_rows) {  // the whole workgroup: no barrier below is reached
    const int row = (((int)blockIdx.y - u_rows) * (int)gridDim.x + (int)blockIdx.x) * kWaves + wv;
    if (row < qj.n)
      quant::quantize_entry(reinterpret_cast<bf16*>(qj.src) + (int64_t)row * qj.src_ld, row, qj.dst,
                            reinterpret_cast<const bf16*>(qj.gain), qj.eps, qj.writeback, lane);
    return;
  }
  const int c0 = blockIdx.x * kCols, h = blockIdx.y - q_rows - u_rows;
  const int sub = lane >> 4, sl = lane & 15;  // copy lane: row 4P + sub, slot sl (1 KiB = 4 rows)
  // the weight slice: 32 copies, 8 per wave
#pragma unroll
  for (int i = 0; i < kDh / 4 / kWaves; ++i) {
    const int P = i * kWaves + wv, r = 4 * P + sub;
    const bf16* src = w + ((int64_t)h * kDh + r) * d_c + c0 + 8 * wslot(r, sl);
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(lw + P * 1024), 16, 0, 0);
  }
  // one block of the head's queries: 16 copies, 4 per wave (rows past B repeat row B-1)
  auto copy_q = [&](int m0) {
#pragma unroll
    for (int i = 0; i < kMB / 4 / kWaves; ++i) {
      const int P = i * kWaves + wv, r = 4 * P + sub;
      const int m = min(m0 + r, B - 1);
      const bf16* src = qc + ((int64_t)m * n_h + h) * kDh + 8 * qslot(r, sl);
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(lq + P * 1024), 16, 0, 0);
    }
  };
  copy_q(0);
  const int G = lane >> 4, i16 = lane & 15;
  MLA_TILE_BARRIER(waitcnt_vm(0));
  // B fragments of this wave's two 16-column blocks for every 32-k step: lane (G, i) holds column
  // i, k = 32 kk + 8G .. +7; source lane s of the two reads supplies row 32 kk + 8G + s/4 (+4),
  // columns 4 (s % 4) .. +3
  Frag8<bf16> bf[kDh / 32][2];
  {
    const int rsub = i16 >> 2, cq = i16 & 3;
#pragma unroll
    for (int kk = 0; kk < kDh / 32; ++kk)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = wv * 32 + nb * 16 + 4 * cq;  // within the slice
        const int chunk = col >> 3, byte = (col & 7) * 2;
        const int r_lo = 32 * kk + 8 * G + rsub, r_hi = r_lo + 4;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_shortx4_t*)(lw + r_lo * kRowB + wslot(r_lo, chunk) * 16 + byte));
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_shortx4_t*)(lw + r_hi * kRowB + wslot(r_hi, chunk) * 16 + byte));
        bf[kk][nb].v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
  }
  for (int m0 = 0; m0 < B; m0 += kMB) {
    if (m0 > 0) {
      __syncthreads();  // every wave is done with the previous block
      copy_q(m0);
      MLA_TILE_BARRIER(waitcnt_vm(0));
    }
    floatx4 acc[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = floatx4{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < kDh / 32; ++kk)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        // A fragment: batch row m0 + 16 mb + i, k = 32 kk + 8G .. +7 (chunk 4 kk + G)
        const int r = mb * 16 + i16;
        Frag8<bf16> a;
        a.v = *reinterpret_cast<const bf16x8*>(lq + r * kRowB + qslot(r, 4 * kk + G) * 16);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mma16(a, bf[kk][nb], acc[mb][nb]);
      }
    // C lane: column i, rows 4G + j
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + mb * 16 + 4 * G + j;
        if (m < B) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            out[(int64_t)m * out_ld + (int64_t)h * out_hs + c0 + wv * 32 + nb * 16 + i16] = (bf16)acc[mb][nb][j];
        }
      }
  }
}

bool absorb_ok(DType t, int d_h, int d_c) {
  return t == DType::BF16 && d_h == absorb::kDh && d_c % absorb::kCols == 0;
}

hipError_t absorb_run(const void* qc, const void* w_uk, void* qhat, int B, int n_h, int d_h, int d_c,
                      int64_t out_ld, int64_t out_hs, hipStream_t s, const QuantJob* qj,
                      const DecodeAttnParams* units) {
  const QuantJob job = qj ? *qj : QuantJob{};
  if (units && (!units->units || units->B > 64 || units->B < 1)) return hipErrorInvalidValue;
  if (B == 0 && job.n <= 0 && !units) return hipSuccess;
  // the units table's row, then the quantiser's rows, then the heads
  const int u_rows = units ? 1 : 0;
  const int per_row = d_c / absorb::kCols * absorb::kWaves;  // entries per grid row
  const int q_rows = job.n > 0 ? (job.n + per_row - 1) / per_row : 0;
  dim3 grid(d_c / absorb::kCols, (B > 0 ? n_h : 0) + q_rows + u_rows);
  (void)d_h;  // == absorb::kDh (absorb_ok)
  hipLaunchKernelGGL(absorb_kernel, grid, dim3(64 * absorb::kWaves), 0, s, reinterpret_cast<const bf16*>(qc),
                     reinterpret_cast<const bf16*>(w_uk), reinterpret_cast<bf16*>(qhat), B, n_h, d_c, out_ld, out_hs,
                     job, q_rows, units ? *units : DecodeAttnParams{}, u_rows);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- W_UV per head
// o[b][h][d] = sum_c W_UV[h*d_h + d][c] o_hat[b][h][c] (App. C, W_UV applied after the softmax):
// per head a skinny product over d_c = 512 with both operands c-contiguous.  Workgroup = (16 NW
// columns d of one head): the head's o_hat rows (64 at a time, 1 KiB each) are staged in LDS and
// shared by NW waves of 16 columns, each wave holding its 16 weight rows in registers.  One pass
// over k, no split.
//
// With the KV partitions' outputs given (split-KV decode), the rows are not read from o_hat but
// combined on the way into LDS: o_hat = sum_s w_s o_s / sum_s w_s with w_s = 2^(m_s - M) l_s and
// M = max_s m_s (the log-sum-exp rule), o_s = O_s / l_s in bf16.  Then one workgroup takes a
// whole head (NW = d_h / 16) so that every partition row is read once.
namespace uvk {
constexpr int kDc = 512;    // d_c: an LDS row of o_hat is 1 KiB (64 chunks)
constexpr int kRowB = 2 * kDc;
constexpr int kMB = 64;     // batch rows per block
constexpr int kWaves = 4;   // plain o_hat input
constexpr int kWavesParts = 8;  // partition input: d_h = 128
constexpr int kCols = 16 * kWaves;
constexpr int kMBParts = 32;  // rows per workgroup with partition input
constexpr int kRowsInFlight = kMBParts / kWavesParts;  // rows a wave combines at once (loads in flight)
// chunk c of o_hat row m at slot c ^ (m & 15): the 16 rows one fragment read covers fall in
// distinct banks
__device__ __forceinline__ int slot(int m, int c) { return c ^ (m & 15); }
}  // namespace uvk

template <int NW, bool PARTS>
__global__ void __launch_bounds__(64 * NW) uv_kernel(const bf16* __restrict__ ohat, UvPartials parts,
                                                     const bf16* __restrict__ w, bf16* __restrict__ o,
                                                     float* __restrict__ o32, int B, int n_h, int d_h) {
  using namespace uvk;
  constexpr int MB = PARTS ? kMBParts : kMB;  // rows per LDS block
  __shared__ __attribute__((aligned(1024))) char la[MB * kRowB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  int h, c0, m_begin, m_stop;
  if constexpr (PARTS) {  // block id -> (head, chunk of MB rows); a head's chunks 8 ids apart
    const int RB = (B + MB - 1) / MB, r = blockIdx.x / 8;
    h = (r / RB) * 8 + blockIdx.x % 8;
    if (h >= n_h) return;
    c0 = 0;
    m_begin = (r % RB) * MB;
    m_stop = m_begin + 1;
  } else {
    h = blockIdx.y;
    c0 = blockIdx.x * 16 * NW;
    m_begin = 0;
    m_stop = B;
  }
  const int d0 = c0 + wv * 16;
  const int G = lane >> 4, i16 = lane & 15;
  // one copy instruction per o_hat row (rows past B repeat row B-1)
  auto copy_a = [&](int m0) {
#pragma unroll
    for (int i = 0; i < MB / NW; ++i) {
      const int r = i * NW + wv;
      const int m = min(m0 + r, B - 1);
      const bf16* src = ohat + ((int64_t)m * n_h + h) * kDc + 8 * slot(r, lane);
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void_t*)(la + r * kRowB), 16, 0, 0);
    }
  };
  // rows r = i NW + wv of the block, kRowsInFlight at a time: lane holds dims 8 lane .. +7.  Lane u
  // reads partition u's max and normaliser (fewer than 16 partitions here; M by a wave reduction);
  // the output rows go four partitions at a time.  The maxima, the normalisers and the first four
  // partitions' rows are all issued before any of them is used, one memory round trip instead of
  // one per dependent load.  A row is read whether or not its partition is empty (an empty one
  // writes only its max, -inf, and its row is then never added: the loads stay inside the
  // partials, and skipping them would cost another round trip).
  auto combine_a = [&](int m0) {
    const int S = parts.splits;
    for (int i0 = 0; i0 < MB / NW; i0 += kRowsInFlight) {
      float M[kRowsInFlight], L[kRowsInFlight], acc[kRowsInFlight][8], m_l[kRowsInFlight], l_l[kRowsInFlight];
      int64_t base[kRowsInFlight];
      bool live[kRowsInFlight];  // rows past B are not read (their products are never stored)
#pragma unroll
      for (int k = 0; k < kRowsInFlight; ++k) {
        const int m = m0 + (i0 + k) * NW + wv;
        live[k] = m < B;
        base[k] = (int64_t)min(m, B - 1) * S * n_h + h;  // partition s at base + s n_h
        const bool in = live[k] && lane < S;
        m_l[k] = in ? parts.m[base[k] + (int64_t)lane * n_h] : -INFINITY;
        l_l[k] = in ? parts.l[base[k] + (int64_t)lane * n_h] : 0.f;
        L[k] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
      }
      auto load_group = [&](int s0, bf16x8 (&v)[kRowsInFlight][4]) {
#pragma unroll
        for (int k = 0; k < kRowsInFlight; ++k)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (live[k] && s0 + u < S)
              v[k][u] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(parts.o) +
                                                        (base[k] + (int64_t)(s0 + u) * n_h) * kDc + 8 * lane);
      };
      auto add_group = [&](int s0, const bf16x8 (&v)[kRowsInFlight][4]) {
#pragma unroll
        for (int k = 0; k < kRowsInFlight; ++k)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float ms = lane_value(m_l[k], s0 + u), ls = lane_value(l_l[k], s0 + u);
            if (s0 + u < S && ms > -INFINITY) {
              const float ws = exp2f(ms - M[k]) * ls;
              L[k] += ws;
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[k][e] += ws * (float)v[k][u][e];
            }
          }
      };
      bf16x8 v[kRowsInFlight][4];
      load_group(0, v);
#pragma unroll
      for (int k = 0; k < kRowsInFlight; ++k) {
        M[k] = wave_max_xor(wave_max_xor(wave_max_xor(m_l[k], 1), 2), 4);
        M[k] = wave_max_xor(wave_max_xor(wave_max_xor(M[k], 8), 16), 32);
      }
      add_group(0, v);
      for (int s0 = 4; s0 < S; s0 += 4) {
        load_group(s0, v);
        add_group(s0, v);
      }
#pragma unroll
      for (int k = 0; k < kRowsInFlight; ++k) {
        const int r = (i0 + k) * NW + wv;
        const float inv = L[k] > 0.f ? 1.f / L[k] : 0.f;
        bf16x8 out;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = (bf16)(acc[k][e] * inv);
        *reinterpret_cast<bf16x8*>(la + r * kRowB + slot(r, lane) * 16) = out;
      }
    }
  };
  // With many partitions (16 or more: long contexts, small batches) every wave takes part in
  // every row: wave w walks the row's groups w, w + NW, ... of eight partitions, and the waves'
  // partial sums meet in LDS, where the row's owner normalises them into the A block.  Every
  // partition's (max, normaliser) is read first, two per lane (partitions lane and 64 + lane;
  // beyond 128 read where needed), so that each group then takes one round trip for its non-empty
  // partitions' rows (the weights held in registers leave room for one group in flight).
  auto combine_coop = [&](int m0, float* red) {
    constexpr int kCoopG = 8;  // partitions per wave and group
    const int S = parts.splits;
    for (int r = 0; r < MB && m0 + r < B; ++r) {
      const int64_t base = (int64_t)(m0 + r) * S * n_h + h;
      float m2[2], l2[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int sp = 64 * j + lane;
        m2[j] = sp < S ? parts.m[base + (int64_t)sp * n_h] : -INFINITY;
        l2[j] = sp < S ? parts.l[base + (int64_t)sp * n_h] : 0.f;
      }
      float M = fmaxf(m2[0], m2[1]);
      for (int c = 128; c < S; c += 64)
        if (c + lane < S) M = fmaxf(M, parts.m[base + (int64_t)(c + lane) * n_h]);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) M = fmaxf(M, __shfl_xor(M, d, 64));
      float L = 0.f, acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
      for (int s0 = kCoopG * wv; s0 < S; s0 += kCoopG * NW) {
        // a group lies wholly below partition 128 (values from the lanes that hold them) or wholly
        // above it (read here): one path per group, so that no row load waits on another
        float ms[kCoopG], ls[kCoopG];
        bf16x8 v[kCoopG];
        if (s0 < 128) {
#pragma unroll
          for (int u = 0; u < kCoopG; ++u) {
            ms[u] = lane_value(s0 < 64 ? m2[0] : m2[1], (s0 + u) & 63);
            ls[u] = lane_value(s0 < 64 ? l2[0] : l2[1], (s0 + u) & 63);
          }
        } else {
#pragma unroll
          for (int u = 0; u < kCoopG; ++u) {
            ms[u] = s0 + u < S ? parts.m[base + (int64_t)(s0 + u) * n_h] : -INFINITY;
            ls[u] = s0 + u < S ? parts.l[base + (int64_t)(s0 + u) * n_h] : 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < kCoopG; ++u)
          if (ms[u] > -INFINITY)  // (-inf past the last partition too)
            v[u] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(parts.o) +
                                                    (base + (int64_t)(s0 + u) * n_h) * kDc + 8 * lane);
#pragma unroll
        for (int u = 0; u < kCoopG; ++u)
          if (ms[u] > -INFINITY) {
            const float ws = exp2f(ms[u] - M) * ls[u];
            L += ws;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += ws * (float)v[u][e];
          }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) red[(wv * 9 + e) * 64 + lane] = acc[e];
      red[(wv * 9 + 8) * 64 + lane] = L;
      __syncthreads();
      if (wv == r % NW) {
        float Lt = 0.f, A[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) A[e] = 0.f;
        for (int w2 = 0; w2 < NW; ++w2) {
#pragma unroll
          for (int e = 0; e < 8; ++e) A[e] += red[(w2 * 9 + e) * 64 + lane];
          Lt += red[(w2 * 9 + 8) * 64 + lane];
        }
        const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
        bf16x8 out;
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = (bf16)(A[e] * inv);
        *reinterpret_cast<bf16x8*>(la + r * kRowB + slot(r, lane) * 16) = out;
      }
      __syncthreads();  // the partial sums are read before the next row overwrites them
    }
  };
  // B fragments: lane (G, i) holds weight row d0 + i, k = 32 kk + 8G .. +7
  Frag8<bf16> bw[kDc / 32];
  {
    const bf16* wr = w + ((int64_t)h * d_h + d0 + i16) * kDc + 8 * G;
#pragma unroll
    for (int kk = 0; kk < kDc / 32; ++kk) load8(bw[kk], wr + 32 * kk);
  }
  float* red = nullptr;  // the waves' partial sums of one row (cooperative combine)
  if constexpr (PARTS) {
    __shared__ float red_s[NW * 9 * 64];
    red = red_s;
  }
  auto combine = [&](int m0) {
    if (parts.splits >= 16) combine_coop(m0, red);
    else combine_a(m0);
  };
  if constexpr (PARTS) {
    combine(m_begin);
    MLA_TILE_BARRIER(kWaitLgkm0);
  } else {
    copy_a(0);
    MLA_TILE_BARRIER(waitcnt_vm(0));
  }
  for (int m0 = m_begin; m0 < m_stop; m0 += MB) {
    if (m0 > m_begin) {
      __syncthreads();  // every wave is done with the previous block
      if constexpr (PARTS) {
        combine(m0);
        MLA_TILE_BARRIER(kWaitLgkm0);
      } else {
        copy_a(m0);
        MLA_TILE_BARRIER(waitcnt_vm(0));
      }
    }
    floatx4 acc[MB / 16];
#pragma unroll
    for (int mb = 0; mb < MB / 16; ++mb) acc[mb] = floatx4{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < kDc / 32; ++kk)
#pragma unroll
      for (int mb = 0; mb < MB / 16; ++mb) {
        const int r = mb * 16 + i16;  // A fragment: row r, k = 32 kk + 8G .. +7 (chunk 4 kk + G)
        Frag8<bf16> a;
        a.v = *reinterpret_cast<const bf16x8*>(la + r * kRowB + slot(r, 4 * kk + G) * 16);
        acc[mb] = mma16(a, bw[kk], acc[mb]);
      }
    // C lane: column d0 + i, rows 4G + j
#pragma unroll
    for (int mb = 0; mb < MB / 16; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + mb * 16 + 4 * G + j;
        if (m < B) {
          const int64_t idx = ((int64_t)m * n_h + h) * d_h + d0 + i16;
          o[idx] = (bf16)acc[mb][j];
          if (o32) o32[idx] = acc[mb][j];
        }
      }
  }
}

bool uv_ok(DType t, int d_h, int d_c) { return t == DType::BF16 && d_c == uvk::kDc && d_h % uvk::kCols == 0; }
bool uv_parts_ok(DType t, int d_h, int d_c) { return uv_ok(t, d_h, d_c) && d_h == 16 * uvk::kWavesParts; }
int uv_parts_workgroups(int B, int n_h) { return (n_h + 7) / 8 * 8 * ((B + uvk::kMBParts - 1) / uvk::kMBParts); }

hipError_t uv_run(const void* ohat, const void* w_uv, void* o, float* o32, int B, int n_h, int d_h,
                  hipStream_t s, const UvPartials* parts) {
  if (B == 0) return hipSuccess;
  if (parts) {
    if (d_h != 16 * uvk::kWavesParts || parts->splits < 1) return hipErrorInvalidValue;
    const int blocks = uv_parts_workgroups(B, n_h);
    hipLaunchKernelGGL((uv_kernel<uvk::kWavesParts, true>), dim3(blocks), dim3(64 * uvk::kWavesParts), 0, s,
                       nullptr, *parts, reinterpret_cast<const bf16*>(w_uv), reinterpret_cast<bf16*>(o), o32, B,
                       n_h, d_h);
    return hipGetLastError();
  }
  dim3 grid(d_h / uvk::kCols, n_h);
  hipLaunchKernelGGL((uv_kernel<uvk::kWaves, false>), grid, dim3(64 * uvk::kWaves), 0, s,
                     reinterpret_cast<const bf16*>(ohat), UvPartials{}, reinterpret_cast<const bf16*>(w_uv),
                     reinterpret_cast<bf16*>(o), o32, B, n_h, d_h);
  return hipGetLastError();
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

template <typename T, int V>
void launch_reduce(const GemmParams& p, int splits, const float* partial, int blocks, hipStream_t s) {
  auto k = splits <= 2 ? splitk_reduce_kernel<T, V, 2>
           : splits <= 4 ? splitk_reduce_kernel<T, V, 4>
           : splits <= 8 ? splitk_reduce_kernel<T, V, 8> : splitk_reduce_kernel<T, V, 16>;
  hipLaunchKernelGGL(k, dim3(blocks), dim3(128), 0, s, p, splits, partial);
}

template <typename T>
hipError_t run_t(const GemmParams& p_in, const GemmPlan& plan, float* partial, hipStream_t s) {
  hipError_t err;
  // the RoPE table rides along in the skinny kernel when a reduce pass (which runs the epilogue)
  // follows it; otherwise it is filled by its own launch first
  const bool side = p_in.side_rope.tab && (plan.cfg == 3 || plan.cfg == 4) && plan.splits > 1;
  GemmParams p = p_in;
  if (p.side_rope.tab && !side) {
    const RopeJob& r = p.side_rope;
    err = rope_table(r.pos, r.n, 2 * r.half, r.f, r.tab, s);
    if (err != hipSuccess) return err;
    p.side_rope = RopeJob{};
  }
  switch (plan.cfg) {
    case 0: err = launch_cfg<T, 0>(p, plan, partial, s); break;
    case 1: err = launch_cfg<T, 1>(p, plan, partial, s); break;
    case 5: {
      dim3 grid(((p.M + big::kTileM - 1) / big::kTileM) * ((p.N + big::kTileN - 1) / big::kTileN), p.batch,
                plan.splits);
      hipLaunchKernelGGL(gemm_big_kernel, grid, dim3(64 * big::kWaves), 0, s, p, plan.splits, plan.k_per_split,
                         partial);
      err = hipGetLastError();
      break;
    }
    case 3:
    case 4: {
      dim3 grid((p.N + skinny::kBN - 1) / skinny::kBN + (side ? 1 : 0), p.batch * plan.splits);
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
  // 128-thread blocks so that small outputs still spread over the compute units
  if (p.N % 4 == 0 && p.E0 % 4 == 0) {
    const int64_t groups = (int64_t)p.batch * p.M * (p.N / 4);
    const int blocks = (int)std::min<int64_t>((groups + 127) / 128, 16384);
    launch_reduce<T, 4>(p, plan.splits, partial, blocks, s);
  } else {
    const int64_t groups = (int64_t)p.batch * p.M * (p.N / 2);
    const int blocks = (int)std::min<int64_t>((groups + 127) / 128, 16384);
    launch_reduce<T, 2>(p, plan.splits, partial, blocks, s);
  }
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
  // A compute unit streams at most ~20 GB/s, about 1/256 of the chip's HBM rate (measured), so
  // the grid should put one workgroup on as many compute units as possible without doubling up
  // on some: floor(cus / tiles) splits; when that is 1 (tiles in (cus/2, cus]) two splits still
  // beat leaving compute units idle (two workgroups fit per compute unit).  Each split streams at
  // least four steps.
  int splits = (int)std::max<int64_t>(1, cus / tiles);
  if (splits == 1 && 2 * tiles <= 2LL * cus && tiles * 2 > cus) splits = 2;
  splits = std::min(splits, std::max(1, ksteps / 4));
  const int per = (ksteps + splits - 1) / splits;
  pl.splits = (ksteps + per - 1) / per;
  pl.k_per_split = per * skinny::kKS;
  pl.partial_bytes = pl.splits > 1 ? (size_t)pl.splits * batch * M * N * sizeof(float) : 0;
  return pl;
}

GemmPlan gemm_plan(int M, int N, int K, int batch, int cus, bool skinny_ok) {
  if (skinny_ok && M <= 64 && K % skinny::kKS == 0 && N % 2 == 0) return gemm_plan_skinny(M, N, K, batch, cus);
  // large products: 256 x 256 tiles, one k range when there are enough tiles to fill the compute
  // units, else the k range split into at most ceil(cus / tiles) pieces of at least four 64-k steps
  // (measured on 512-row products: 0.19 PFLOP/s on the generic tiles, split 256 x 256 tiles and a
  // reduce pass instead).  Too few tiles even then (a short K): the generic tiles.
  if (skinny_ok && K % big::kStepK == 0 && N % 2 == 0) {
    const int64_t tiles =
        (int64_t)((M + big::kTileM - 1) / big::kTileM) * ((N + big::kTileN - 1) / big::kTileN) * batch;
    const int ksteps = K / big::kStepK;
    int splits = tiles >= cus ? 1 : (int)std::min<int64_t>((cus + tiles - 1) / tiles, std::max(1, ksteps / 4));
    const int per = (ksteps + splits - 1) / splits;
    splits = (ksteps + per - 1) / per;
    if (tiles * splits >= cus / 2) {
      GemmPlan pl;
      pl.cfg = 5;
      pl.bm = big::kTileM;
      pl.bn = big::kTileN;
      pl.splits = splits;
      pl.k_per_split = per * big::kStepK;
      pl.partial_bytes = splits > 1 ? (size_t)splits * batch * M * N * sizeof(float) : 0;
      return pl;
    }
  }
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
  if (plan.cfg == 5 && (t != DType::BF16 || p.nn || p.K % big::kStepK != 0 || p.lda % 8 != 0 || p.ldb % 8 != 0 ||
                        p.strideA % 8 != 0 || p.strideB % 8 != 0))
    return hipErrorInvalidValue;
  return t == DType::BF16 ? run_t<bf16>(p, plan, partial, s) : run_t<float>(p, plan, partial, s);
}

}  // namespace mla
