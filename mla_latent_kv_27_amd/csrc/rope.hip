// Small helper kernels: RoPE angle tables, the latent RMSNorm, prefill row bookkeeping, paged
// row scatter.
//
// RoPE follows the reading of the DeepSeek-V2 summary page's App. C ("RoPE(.)", the RoFormer
// rotation it cites): interleaved pairs (x_2k, x_2k+1) rotate by pos * theta_k, theta_k =
// base^(-2k/d_hr).  With YaRN (section 3.1.4; the YaRN paper's NTK-by-parts form, which the page
// cites) a pair that turns r_k = L theta_k / (2 pi) times over the original context L keeps
// theta_k above beta turns, is slowed to theta_k / s below alpha turns, and is blended linearly
// in r_k between.  The angle is formed and reduced modulo 2*pi in fp64 so that positions near
// 1.3e5 keep full fp32 accuracy in cos/sin.
#include <initializer_list>

#include "common.h"
#include "internal.h"

namespace mla {

__global__ void __launch_bounds__(256)
    rope_table_kernel(const int32_t* __restrict__ pos, int n, int half, RopeFreq f, float2* tab) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= (int64_t)n * half) return;
  tab[i] = rope_table_entry(pos, half, f, i);
}

hipError_t rope_table(const int32_t* pos, int n, int d_hr, const RopeFreq& f, float2* tab, hipStream_t s) {
  const int half = d_hr / 2;
  const int64_t total = (int64_t)n * half;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, pos, n,
                     half, f, tab);
  return hipGetLastError();
}

// RMSNorm after the compressed latents (section 3.1.2 of the DeepSeek-V2 summary page): one wave
// per row; the mean square is accumulated in fp32 from the stored values.
template <typename T>
__global__ void __launch_bounds__(256)
    rmsnorm_rows_kernel(T* __restrict__ x, int n, int W, int64_t ld, const T* __restrict__ g, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  T* r = x + row * ld;
  float ss = 0.f;
  for (int i = lane; i < W; i += 64) {
    const float v = to_f32(r[i]);
    ss += v * v;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) ss = wave_sum_xor(ss, m);
  const float inv = 1.0f / sqrtf(ss / (float)W + eps);
  for (int i = lane; i < W; i += 64) r[i] = from_f32<T>(to_f32(r[i]) * inv * to_f32(g[i]));
}

// The same on 16-byte chunks with every load of a row in flight at once: lane l holds chunks l,
// l + 64, ... (at most NC of them) in registers.  Rows of L elements; the first W are normalised
// (gain g, when set), the rest (an entry's rope part) pass unchanged.  The loops above issue one
// element per lane and iteration over a run-time width, so each load waits for the previous add
// (24 dependent round trips for a 1536-wide c^q row).
template <typename T, int NC>
struct RowChunks {
  static constexpr int kEV = 16 / sizeof(T);  // elements per chunk
  typedef T vec_t __attribute__((ext_vector_type(kEV)));
  vec_t v[NC];
  __device__ __forceinline__ bool has(int k, int lane, int L) const { return (lane + 64 * k) * kEV < L; }
  __device__ __forceinline__ void load(const T* x, int L, int lane) {
#pragma unroll
    for (int k = 0; k < NC; ++k)
      if (has(k, lane, L)) v[k] = *reinterpret_cast<const vec_t*>(x + (lane + 64 * k) * kEV);
  }
  __device__ __forceinline__ void store(T* x, int L, int lane) const {
#pragma unroll
    for (int k = 0; k < NC; ++k)
      if (has(k, lane, L)) *reinterpret_cast<vec_t*>(x + (lane + 64 * k) * kEV) = v[k];
  }
  // x[i] <- x[i] / rms(x[0..W)) * g[i] for i < W, with gv holding g's chunks
  __device__ __forceinline__ void normalise(const RowChunks& gv, int W, float eps, int lane) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NC; ++k)
      if (has(k, lane, W))
#pragma unroll
        for (int e = 0; e < kEV; ++e) {
          const float a = to_f32(v[k][e]);
          ss += a * a;
        }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) ss = wave_sum_xor(ss, m);
    const float inv = 1.0f / sqrtf(ss / (float)W + eps);
#pragma unroll
    for (int k = 0; k < NC; ++k)
      if (has(k, lane, W))
#pragma unroll
        for (int e = 0; e < kEV; ++e) v[k][e] = from_f32<T>(to_f32(v[k][e]) * inv * to_f32(gv.v[k][e]));
  }
};
constexpr int kRowChunks = 4;  // chunks per lane: rows up to 2048 bf16 or 1024 fp32 values

template <typename T>
__global__ void __launch_bounds__(256)
    rmsnorm_rows_vec_kernel(T* __restrict__ x, int n, int W, int64_t ld, const T* __restrict__ g, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  RowChunks<T, kRowChunks> v, gv;
  v.load(x + row * ld, W, lane);
  gv.load(g, W, lane);
  v.normalise(gv, W, eps, lane);
  v.store(x + row * ld, W, lane);
}

// Whether rows of these widths and pointers take the 16-byte chunks.
template <typename T>
bool chunked_rows_ok(std::initializer_list<int64_t> widths, std::initializer_list<const void*> ptrs) {
  constexpr int ev = 16 / sizeof(T);
  for (int64_t w : widths)
    if (w % ev != 0 || w > (int64_t)64 * kRowChunks * ev) return false;
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return false;
  return true;
}

template <typename T>
hipError_t rmsnorm_rows_t(void* x, int n, int W, int64_t ld, const void* gain, float eps, hipStream_t s) {
  const dim3 grid((n + 3) / 4), block(256);
  if (chunked_rows_ok<T>({W, ld}, {x, gain}))
    hipLaunchKernelGGL(rmsnorm_rows_vec_kernel<T>, grid, block, 0, s, reinterpret_cast<T*>(x), n, W, ld,
                       reinterpret_cast<const T*>(gain), eps);
  else
    hipLaunchKernelGGL(rmsnorm_rows_kernel<T>, grid, block, 0, s, reinterpret_cast<T*>(x), n, W, ld,
                       reinterpret_cast<const T*>(gain), eps);
  return hipGetLastError();
}

hipError_t rmsnorm_rows(DType t, void* x, int n, int W, int64_t ld, const void* gain, float eps, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  return t == DType::BF16 ? rmsnorm_rows_t<bf16>(x, n, W, ld, gain, eps, s)
                          : rmsnorm_rows_t<float>(x, n, W, ld, gain, eps, s);
}

// One wave per row: rows < n_e are new cache entries (normalise the latent part, store in place
// and into the page), the next n_q rows are c^q rows (normalise in place).
template <typename T>
__global__ void __launch_bounds__(256) latent_finish_kernel(LatentFinish f) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= f.n_e + f.n_q) return;
  const bool entry = row < f.n_e;
  T* x = entry ? reinterpret_cast<T*>(f.entries) + (int64_t)row * f.E
               : reinterpret_cast<T*>(f.cq) + (int64_t)(row - f.n_e) * f.d_cq;
  const int W = entry ? f.d_c : f.d_cq;
  const T* g = reinterpret_cast<const T*>(entry ? f.g_ckv : f.g_cq);
  if (g) {
    float ss = 0.f;
    for (int i = lane; i < W; i += 64) {
      const float v = to_f32(x[i]);
      ss += v * v;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) ss = wave_sum_xor(ss, m);
    const float inv = 1.0f / sqrtf(ss / (float)W + f.eps);
    for (int i = lane; i < W; i += 64) x[i] = from_f32<T>(to_f32(x[i]) * inv * to_f32(g[i]));
  }
  if (!entry) return;
  const int sq = f.seq ? f.seq[row] : row, ps = f.pos[row];
  const int64_t slot = (int64_t)f.block_table[(int64_t)sq * f.max_blocks + ps / f.block_size] * f.block_size +
                       ps % f.block_size;
  T* dst = reinterpret_cast<T*>(f.pool) + slot * f.E;
  for (int i = lane; i < f.E; i += 64) dst[i] = x[i];  // this lane's own writes above: no barrier needed
}

// The same on 16-byte chunks (RowChunks): an entry's page position is read first, with the row,
// so that its block-table read overlaps the row's; the row is read once, normalised in registers,
// stored in place and into its page.
template <typename T>
__global__ void __launch_bounds__(256) latent_finish_vec_kernel(LatentFinish f) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= f.n_e + f.n_q) return;
  const bool entry = row < f.n_e;
  T* x = entry ? reinterpret_cast<T*>(f.entries) + (int64_t)row * f.E
               : reinterpret_cast<T*>(f.cq) + (int64_t)(row - f.n_e) * f.d_cq;
  const int W = entry ? f.d_c : f.d_cq, L = entry ? f.E : f.d_cq;
  const T* g = reinterpret_cast<const T*>(entry ? f.g_ckv : f.g_cq);
  int sq = 0, ps = 0;
  if (entry) {
    sq = f.seq ? f.seq[row] : row;
    ps = f.pos[row];
  }
  RowChunks<T, kRowChunks> v, gv;
  v.load(x, L, lane);
  if (g) gv.load(g, W, lane);
  int64_t slot = 0;
  if (entry)
    slot = (int64_t)f.block_table[(int64_t)sq * f.max_blocks + ps / f.block_size] * f.block_size + ps % f.block_size;
  if (g) {
    v.normalise(gv, W, f.eps, lane);
    v.store(x, W, lane);
  }
  if (entry) v.store(reinterpret_cast<T*>(f.pool) + slot * f.E, L, lane);
}

template <typename T>
hipError_t latent_finish_t(const LatentFinish& f, hipStream_t s) {
  const dim3 grid((f.n_e + f.n_q + 3) / 4), block(256);
  const bool vec = chunked_rows_ok<T>({f.E, f.d_c, f.n_q > 0 ? f.d_cq : 0},
                                      {f.entries, f.g_ckv, f.pool, f.n_q > 0 ? f.cq : nullptr, f.g_cq});
  if (vec)
    hipLaunchKernelGGL(latent_finish_vec_kernel<T>, grid, block, 0, s, f);
  else
    hipLaunchKernelGGL(latent_finish_kernel<T>, grid, block, 0, s, f);
  return hipGetLastError();
}

hipError_t latent_finish(DType t, const LatentFinish& f, hipStream_t s) {
  const int rows = f.n_e + f.n_q;
  if (rows <= 0) return hipSuccess;
  return t == DType::BF16 ? latent_finish_t<bf16>(f, s) : latent_finish_t<float>(f, s);
}

__global__ void __launch_bounds__(256)
    prefill_rows_kernel(int n, int T, int32_t* seq, int32_t* pos, const int32_t* __restrict__ start) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < n) {
    seq[r] = r / T;
    pos[r] = r % T + (start ? start[r / T] : 0);
  }
}

hipError_t prefill_rows(int n, int T, int32_t* seq, int32_t* pos, hipStream_t s, const int32_t* start) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, s, n, T, seq, pos, start);
  return hipGetLastError();
}

// One thread per 16-byte chunk of an output row.  fp8: the chunk's 8 values come from 8 code
// bytes and the part's scale (the latent part's for columns < d_c, else the rope key's).
template <bool FP8>
__global__ void __launch_bounds__(256)
    gather_entries_kernel(const char* __restrict__ pool, const float* __restrict__ scales,
                          const int32_t* __restrict__ bt, int max_blocks, int block_size,
                          const int32_t* __restrict__ start, const char* __restrict__ fresh, int T, int S, int Tk,
                          int row_bytes, int d_c, char* __restrict__ out) {
  const int cpr = row_bytes / 16;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= (int64_t)S * Tk * cpr) return;
  const int64_t row = i / cpr;
  const int c = (int)(i % cpr);
  const int b = (int)(row / Tk), j = (int)(row % Tk);
  const int s0 = start[b];
  Chunk16 v = zero16();
  if (j >= s0 && j < s0 + T) {  // a row of the chunk itself, as computed
    v = ld16(fresh + ((int64_t)b * T + (j - s0)) * row_bytes + c * 16);
  } else if (j < s0) {  // the cached prefix
    const int64_t slot = (int64_t)bt[(int64_t)b * max_blocks + j / block_size] * block_size + j % block_size;
    if (FP8) {
      const int E = row_bytes / 2;  // bf16 values per entry = code bytes per entry
      const uint2 raw = *reinterpret_cast<const uint2*>(pool + slot * E + 8 * c);
      const float sc = scales[2 * slot + (8 * c < d_c ? 0 : 1)];
      const floatx2 f0 = __builtin_amdgcn_cvt_pk_f32_fp8(raw.x, false), f1 = __builtin_amdgcn_cvt_pk_f32_fp8(raw.x, true);
      const floatx2 f2 = __builtin_amdgcn_cvt_pk_f32_fp8(raw.y, false), f3 = __builtin_amdgcn_cvt_pk_f32_fp8(raw.y, true);
      bf16x8 o;
      o[0] = (bf16)(f0[0] * sc);
      o[1] = (bf16)(f0[1] * sc);
      o[2] = (bf16)(f1[0] * sc);
      o[3] = (bf16)(f1[1] * sc);
      o[4] = (bf16)(f2[0] * sc);
      o[5] = (bf16)(f2[1] * sc);
      o[6] = (bf16)(f3[0] * sc);
      o[7] = (bf16)(f3[1] * sc);
      v = __builtin_bit_cast(Chunk16, o);
    } else {
      v = ld16(pool + slot * row_bytes + c * 16);
    }
  }
  st16(out + row * row_bytes + c * 16, v);
}

hipError_t gather_entries(DType t, const void* pool, const float* scales, const int32_t* block_table, int max_blocks,
                          int block_size, const int32_t* start, const void* fresh, int T, int S, int Tk, int E, int d_c,
                          void* out, hipStream_t s) {
  const int es = scales ? 2 : (int)dsize(t);  // output element size (bf16 for the fp8 cache)
  const int row_bytes = E * es;
  const int64_t total = (int64_t)S * Tk * (row_bytes / 16);
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  if (scales)
    hipLaunchKernelGGL(gather_entries_kernel<true>, grid, block, 0, s, reinterpret_cast<const char*>(pool), scales,
                       block_table, max_blocks, block_size, start, reinterpret_cast<const char*>(fresh), T, S, Tk, row_bytes, d_c,
                       reinterpret_cast<char*>(out));
  else
    hipLaunchKernelGGL(gather_entries_kernel<false>, grid, block, 0, s, reinterpret_cast<const char*>(pool), scales,
                       block_table, max_blocks, block_size, start, reinterpret_cast<const char*>(fresh), T, S, Tk, row_bytes, d_c,
                       reinterpret_cast<char*>(out));
  return hipGetLastError();
}

// One thread per 16-byte chunk of a row.
__global__ void __launch_bounds__(256)
    scatter_rows_kernel(const char* __restrict__ src, int n, int row_bytes, char* __restrict__ pool,
                        const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos,
                        const int32_t* __restrict__ bt, int max_blocks, int block_size) {
  const int cpr = row_bytes / 16;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= (int64_t)n * cpr) return;
  const int r = (int)(i / cpr), c = (int)(i % cpr);
  const int sq = row_seq ? row_seq[r] : r, ps = row_pos[r];
  const int64_t slot = (int64_t)bt[(int64_t)sq * max_blocks + ps / block_size] * block_size + ps % block_size;
  st16(pool + slot * row_bytes + c * 16, ld16(src + (int64_t)r * row_bytes + c * 16));
}

hipError_t scatter_rows(DType t, const void* src, int n, int width, void* pool, const int32_t* row_seq,
                        const int32_t* row_pos, const int32_t* block_table, int max_blocks, int block_size,
                        hipStream_t s) {
  const int row_bytes = width * (int)dsize(t);
  const int64_t total = (int64_t)n * (row_bytes / 16);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const char*>(src), n, row_bytes, reinterpret_cast<char*>(pool), row_seq,
                     row_pos, block_table, max_blocks, block_size);
  return hipGetLastError();
}

}  // namespace mla
