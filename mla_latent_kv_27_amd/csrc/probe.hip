// HBM streaming ceiling of the device, measured the way the decode kernels stream: read-only
// passes over a buffer larger than the last-level cache.  Not part of the MLA computation; the
// benchmark reports the kernels' bandwidth against this measured ceiling next to the vendor
// peak.  Built into its own library (libmla_probe.so) so the MLA library carries none of it.
//
// Two forms:
//   * register loads: each lane keeps UNROLL independent 16-byte loads in flight per iteration,
//     grid-strided over the buffer; the words are folded into one value per workgroup so that
//     the loads cannot be removed;
//   * direct-to-LDS copies (buffer_load ... lds), the way the decode attention kernel fills its
//     tile ring: each wave streams its contiguous slab through a ring of NB 1-KiB slots per
//     wave, keeping NB - 1 copies in flight.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int UNROLL>
__global__ void __launch_bounds__(256) stream_read_regs(const u32x4* __restrict__ src, int64_t n16,
                                                        uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Each wave streams bytes [w0, w1) of the buffer (1-KiB copies: 64 lanes x 16 bytes) into its
// ring of NB slots; a copy is waited for NB - 1 copies later and its slot reused.
template <int NB>
__global__ void __launch_bounds__(256) stream_read_lds(const char* __restrict__ src, int64_t bytes,
                                                       uint32_t* __restrict__ sink) {
  __shared__ __attribute__((aligned(1024))) char ring[4][NB][1024];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int64_t per = (bytes / 1024 + waves - 1) / waves * 1024;
  const int64_t w0 = ((int64_t)blockIdx.x * 4 + w) * per;
  const int64_t w1 = w0 + per < bytes ? w0 + per : bytes;
  const int64_t n = w1 > w0 ? (w1 - w0) / 1024 : 0;
  for (int64_t c = 0; c < n; ++c) {
    const int slot = (int)(c % NB);
    __builtin_amdgcn_global_load_lds((const void*)(src + w0 + c * 1024 + lane * 16),
                                     (lds_void_t*)&ring[w][slot][0], 16, 0, 0);
    if (c >= NB - 1) {
      // the copy issued NB - 1 steps ago has landed (at most NB - 1 younger ones in flight)
      __builtin_amdgcn_s_waitcnt((((NB - 1) >> 4) << 14) | (0xF << 8) | (0x7 << 4) | ((NB - 1) & 0xF));
    }
  }
  __builtin_amdgcn_s_waitcnt((0 << 14) | (0xF << 8) | (0x7 << 4) | 0);
  __syncthreads();
  uint32_t x = *reinterpret_cast<const uint32_t*>(&ring[w][0][lane * 16]);
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

// MFMA-fragment-shaped reads of a row-major matrix of 2-byte elements, rows of `row_bytes`: a wave
// owns 16 consecutive rows and reads them 32 elements (64 bytes) of each row per instruction, lane l
// taking row l % 16 and 16 bytes at 16 (l / 16) of that 64-byte piece (the A-operand layout of a
// 16x16x32 MFMA), with UNROLL instructions in flight.  Rows are dealt to waves round robin.
template <int UNROLL>
__global__ void __launch_bounds__(256) stream_read_frag(const char* __restrict__ src, int64_t bytes, int row_bytes,
                                                        uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t nrows = bytes / row_bytes;
  const int64_t groups = nrows / 16;
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int per_row = row_bytes / 64;  // instructions per row group
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t grp = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); grp < groups; grp += waves) {
    const char* base = src + (grp * 16 + (lane & 15)) * row_bytes + 16 * (lane >> 4);
    int c = 0;
    for (; c + UNROLL <= per_row; c += UNROLL) {
      u32x4 v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (c + u) * 64));
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) acc ^= v[u];
    }
    for (; c < per_row; ++c) acc ^= *reinterpret_cast<const u32x4*>(base + c * 64);
  }
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int m = 32; m >= 1; m >>= 1) x ^= __shfl_xor(x, m, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

}  // namespace

extern "C" {

// One read pass over `bytes` bytes at `src` (device, 16-byte aligned, bytes a multiple of 1024).
// variant: 0..3 register loads with 2, 4, 8, 16 loads in flight per lane; 4..6 direct-to-LDS
// copies with rings of 4, 8, 16 slots per wave; 7, 8: MFMA-operand-shaped reads of 32-KiB rows
// with 8, 16 loads in flight per lane.  blocks: workgroups of 256 threads.  sink:
// device, >= blocks uint32.  Returns 0, or -1 on bad arguments, -4 on a launch failure.
int mla_probe_stream_read(const void* src, int64_t bytes, int variant, int blocks, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 1024 || blocks <= 0) return -1;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t n16 = bytes / 16;
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  const char* c = reinterpret_cast<const char*>(src);
  switch (variant) {
    case 0: hipLaunchKernelGGL(stream_read_regs<2>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
    case 1: hipLaunchKernelGGL(stream_read_regs<4>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_regs<8>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
    case 3: hipLaunchKernelGGL(stream_read_regs<16>, dim3(blocks), dim3(256), 0, s, p, n16, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_lds<4>, dim3(blocks), dim3(256), 0, s, c, bytes, sink); break;
    case 5: hipLaunchKernelGGL(stream_read_lds<8>, dim3(blocks), dim3(256), 0, s, c, bytes, sink); break;
    case 6: hipLaunchKernelGGL(stream_read_lds<16>, dim3(blocks), dim3(256), 0, s, c, bytes, sink); break;
    // weight-matrix shaped reads: rows of 32 KiB (16384 bf16, the longest DeepSeek-V2 weight row)
    case 7: hipLaunchKernelGGL(stream_read_frag<8>, dim3(blocks), dim3(256), 0, s, c, bytes, 32768, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_frag<16>, dim3(blocks), dim3(256), 0, s, c, bytes, 32768, sink); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
