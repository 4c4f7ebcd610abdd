// fp8 latent cache: the quantiser of one entry, as a device function for one wave.  Its own kernel
// (latent_fp8.hip) and the W_UK absorption launch of a decode step (which quantises the step's new
// entries in workgroups of its own) both call it.
//
// The serving section of the page "DeepSeek-V2 paper summary" (section 3.2.3) stores the KV
// cache at about 6 bits per element.  This library reads that as OCP e4m3 codes with one fp32
// scale per token for each part of the cached entry [c^KV | k^R] (App. C): s = amax(|part|) / 448,
// code = e4m3(x / s), rounded to nearest, ties to even, saturating at +-448; an all-zero part has
// s = 0 and zero codes.  The input is the bf16 entry the bf16 cache would hold, so the codes are a
// function of bf16 values, computed in fp32.
//
// d_c = 512, d_hr = 64: lane l holds latent values 8l .. 8l+7 and rope value l; two wave-wide
// maxima give the scales; each lane stores 8 + 1 codes.
#pragma once

#include "common.h"
#include "internal.h"

namespace mla {
namespace quant {

// e4m3 code of y (finite fp32), nearest value with ties to the even code, saturating at 448.
// Subnormals (exponent field 0) are m * 2^-9; a normal value is (1 + m/8) 2^(E-7).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a != a) return 0x7Fu;
  if (!(a < 448.f)) return sign | 0x7Eu;
  if (a < 0.015625f) {                      // below 2^-6: steps of 2^-9 (m = 8 is 2^-6 itself)
    return sign | (uint32_t)rintf(a * 512.f);
  }
  int e;
  const float f = frexpf(a, &e);            // a = f 2^e, f in [0.5, 1)
  float q = rintf(f * 16.f);                // 8 + m, in [8, 16]
  int E = e + 6;                            // biased exponent of 2^(e-1)
  if (q == 16.f) {
    q = 8.f;
    ++E;
  }
  const uint32_t code = ((uint32_t)E << 3) | ((uint32_t)q - 8u);
  return sign | min(code, 0x7Eu);
}

constexpr int kDc = 512, kDr = 64, kEntry = kDc + kDr;

// Entry `row` (bf16, at e) into its slot of dst.  gain != nullptr: the latent part is first
// RMS-normalised (x * g / sqrt(mean(x^2) + eps), the latent norm of section 3.1.2) and rounded to
// bf16, as the bf16 cache would store it; with writeback the normalised bf16 values also replace
// the source row.
__device__ __forceinline__ void quantize_entry(bf16* e, int row, const QuantDst& dst, const bf16* gain, float eps,
                                               bool writeback, int lane) {
  bf16x8 cv = *reinterpret_cast<const bf16x8*>(e + 8 * lane);
  const float rv = (float)e[kDc + lane];
  if (gain) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += (float)cv[i] * (float)cv[i];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) ss = wave_sum_xor(ss, m);
    const float inv = 1.0f / sqrtf(ss / (float)kDc + eps);
    const bf16x8 gv = *reinterpret_cast<const bf16x8*>(gain + 8 * lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) cv[i] = (bf16)((float)cv[i] * inv * (float)gv[i]);
    if (writeback) *reinterpret_cast<bf16x8*>(e + 8 * lane) = cv;
  }
  float c[8];
  float amax_c = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c[i] = (float)cv[i];
    amax_c = fmaxf(amax_c, fabsf(c[i]));
  }
  float amax_r = fabsf(rv);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    amax_c = wave_max_xor(amax_c, m);
    amax_r = wave_max_xor(amax_r, m);
  }
  const float s_c = amax_c / 448.f, s_r = amax_r / 448.f;  // IEEE fp32 division
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t code = s_c > 0.f ? e4m3_code(c[i] / s_c) : 0u;
    if (i < 4) lo |= code << (8 * i);
    else hi |= code << (8 * (i - 4));
  }
  const uint32_t rcode = s_r > 0.f ? e4m3_code(rv / s_r) : 0u;
  int64_t slot = row;
  if (dst.block_table) {
    const int sq = dst.row_seq ? dst.row_seq[row] : row, ps = dst.row_pos[row];
    slot = (int64_t)dst.block_table[(int64_t)sq * dst.max_blocks + ps / dst.block_size] * dst.block_size +
           ps % dst.block_size;
  }
  uint8_t* out = dst.codes + slot * kEntry;
  *reinterpret_cast<uint2*>(out + 8 * lane) = make_uint2(lo, hi);
  out[kDc + lane] = (uint8_t)rcode;
  if (lane == 0) *reinterpret_cast<float2*>(dst.scales + 2 * slot) = make_float2(s_c, s_r);
}

}  // namespace quant
}  // namespace mla
