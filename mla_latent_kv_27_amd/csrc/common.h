// Device-side building blocks shared by the MLA kernels (gfx950 / CDNA4, wave64).
//
// Matrix-core fragments.  Every contraction here is written against one lane layout,
// valid for both storage types:
//   16x16 tile, k-chunk 32: lane l holds row/col (l % 16) and the 8 consecutive k values
//                           8*(l/16) .. 8*(l/16)+7 of the chunk;
//                           accumulator j (0..3) of lane l is element (row 4*(l/16)+j, col l%16).
//   32x32 tile, k-chunk 16: lane l holds row/col (l % 32) and k values 8*(l/32) .. +7;
//                           accumulator j (0..15) is element (row 8*(j/4) + 4*(l/32) + j%4,
//                           col l%32).
// bf16 uses one v_mfma_f32_{16x16x32,32x32x16}_bf16 per chunk.  fp32 uses eight
// v_mfma_f32_{16x16x4,32x32x2}_f32 whose k-slot g of step i stands for k = 8g + i, which
// gives the same per-lane k ownership; a sum over k does not depend on its order.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

typedef __bf16 bf16;

// 8 consecutive k values owned by one lane.
template <typename T>
struct Frag8;
template <>
struct Frag8<bf16> {
  bf16x8 v;
};
template <>
struct Frag8<float> {
  floatx4 lo, hi;
};

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ void load8(Frag8<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void load8(Frag8<float>& f, const float* p) {
  f.lo = *reinterpret_cast<const floatx4*>(p);
  f.hi = *reinterpret_cast<const floatx4*>(p + 4);
}
// Two runs of 4 consecutive elements (8-byte aligned for bf16, 16-byte for fp32).
__device__ __forceinline__ void load4x2(Frag8<bf16>& f, const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void load4x2(Frag8<float>& f, const float* p0, const float* p1) {
  f.lo = *reinterpret_cast<const floatx4*>(p0);
  f.hi = *reinterpret_cast<const floatx4*>(p1);
}
__device__ __forceinline__ void zero8(Frag8<bf16>& f) {
  for (int i = 0; i < 8; ++i) f.v[i] = (bf16)0.0f;
}
__device__ __forceinline__ void zero8(Frag8<float>& f) {
  f.lo = floatx4{0, 0, 0, 0};
  f.hi = floatx4{0, 0, 0, 0};
}
__device__ __forceinline__ void set8(Frag8<bf16>& f, int i, float x) { f.v[i] = (bf16)x; }
__device__ __forceinline__ void set8(Frag8<float>& f, int i, float x) {
  if (i < 4) f.lo[i] = x; else f.hi[i - 4] = x;
}

__device__ __forceinline__ floatx4 mma16(const Frag8<bf16>& a, const Frag8<bf16>& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma16(const Frag8<float>& a, const Frag8<float>& b, floatx4 c) {
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[i], b.lo[i], c, 0, 0, 0);
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[i], b.hi[i], c, 0, 0, 0);
  return c;
}
__device__ __forceinline__ floatx16 mma32(const Frag8<bf16>& a, const Frag8<bf16>& b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mma32(const Frag8<float>& a, const Frag8<float>& b, floatx16 c) {
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[i], b.lo[i], c, 0, 0, 0);
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[i], b.hi[i], c, 0, 0, 0);
  return c;
}

// 16-byte global/LDS chunk copies.
struct alignas(16) Chunk16 {
  uint32_t w[4];
};
__device__ __forceinline__ Chunk16 ld16(const void* p) { return *reinterpret_cast<const Chunk16*>(p); }
__device__ __forceinline__ void st16(void* p, const Chunk16& c) { *reinterpret_cast<Chunk16*>(p) = c; }
__device__ __forceinline__ Chunk16 zero16() { return Chunk16{{0u, 0u, 0u, 0u}}; }

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float wave_sum_xor(float v, int mask) { return v + __shfl_xor(v, mask, 64); }

constexpr float kLog2e = 1.4426950408889634f;

// ---- direct-to-LDS copies and the waits that go with them
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4_t;

// Buffer-form copies (buffer_load_dwordx4 ... lds).  Same transfer as the global form: lane i's
// 16 bytes land at the LDS destination + 16 i.  The compiler counts the buffer form as a vector
// memory access only, whereas it treats a global-form copy as possibly in flight on the LDS
// counter as well and then makes every later wait for an LDS read drain all LDS reads in flight;
// with the buffer form, fragment reads of other LDS buffers keep their partial waits.
// The resource spans `bytes` from a wave-uniform base: offsets stay 32-bit, and a copy whose
// offset falls outside the span reads zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_span(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t span, uint32_t off, lds_void_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(span, dst, 16, off, 0, 0, 0);
}

// The value lane `src` (the same in every lane) holds, read with v_readlane: a scalar result, no
// LDS round trip as a shuffle would take.
__device__ __forceinline__ float lane_value(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), src));
}

// s_waitcnt immediates (gfx9 encoding): vmcnt in bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]; the unused counters are left at their maximum.
constexpr int waitcnt_vm(int n) { return ((n >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (n & 0xF); }
// vmcnt(n) and lgkmcnt(0): the wave's LDS writes have completed as well
constexpr int waitcnt_vm_lgkm0(int n) { return ((n >> 4) << 14) | (0x7 << 4) | (n & 0xF); }
constexpr int kWaitLgkm0 = (0x3 << 14) | (0x7 << 4) | 0xF;

// Workgroup barrier for the pipeline: waits only on what the caller asked for (unlike
// __syncthreads, whose release fence would also wait for the copies in flight), and
// compiler-only fences keep LDS accesses from being moved across it.
#define MLA_TILE_BARRIER(waitcnt_imm)            \
  do {                                           \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);     \
    __builtin_amdgcn_s_waitcnt(waitcnt_imm);     \
    __builtin_amdgcn_s_barrier();                \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);     \
  } while (0)

// The same wait without the barrier: for copies into LDS that only the issuing wave reads.
#define MLA_WAVE_WAIT(waitcnt_imm)               \
  do {                                           \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);     \
    __builtin_amdgcn_s_waitcnt(waitcnt_imm);     \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);     \
  } while (0)

}  // namespace mla
