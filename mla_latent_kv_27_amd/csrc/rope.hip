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
#include "common.h"
#include "internal.h"

namespace mla {

__global__ void __launch_bounds__(256)
    rope_table_kernel(const int32_t* __restrict__ pos, int n, int half, RopeFreq f, float2* tab) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= (int64_t)n * half) return;
  const int r = (int)(i / half), k = (int)(i % half);
  const double two_pi = 6.283185307179586476925286766559;
  double theta = exp(-(2.0 * k / (2.0 * half)) * log(f.base));
  if (f.scale > 1.0) {
    const double turns = f.orig_ctx * theta / two_pi;
    const double g = fmin(fmax((turns - f.alpha) / (f.beta - f.alpha), 0.0), 1.0);
    theta = g * theta + (1.0 - g) * (theta / f.scale);
  }
  double a = (double)pos[r] * theta;
  a = a - floor(a / two_pi) * two_pi;
  double sn, cs;
  sincos(a, &sn, &cs);
  tab[i] = make_float2((float)cs, (float)sn);
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

hipError_t rmsnorm_rows(DType t, void* x, int n, int W, int64_t ld, const void* gain, float eps, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 grid((n + 3) / 4), block(256);
  if (t == DType::BF16)
    hipLaunchKernelGGL(rmsnorm_rows_kernel<bf16>, grid, block, 0, s, reinterpret_cast<bf16*>(x), n, W, ld,
                       reinterpret_cast<const bf16*>(gain), eps);
  else
    hipLaunchKernelGGL(rmsnorm_rows_kernel<float>, grid, block, 0, s, reinterpret_cast<float*>(x), n, W, ld,
                       reinterpret_cast<const float*>(gain), eps);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) prefill_rows_kernel(int n, int T, int32_t* seq, int32_t* pos) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r < n) {
    seq[r] = r / T;
    pos[r] = r % T;
  }
}

hipError_t prefill_rows(int n, int T, int32_t* seq, int32_t* pos, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, s, n, T, seq, pos);
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
