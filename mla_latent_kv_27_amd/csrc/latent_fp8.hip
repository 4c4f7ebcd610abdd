// fp8 latent cache: the quantiser kernel (the per-entry quantiser itself, and the reading of the
// page it follows, are in quant.h).  One wave per entry.
#include <hip/hip_runtime.h>

#include "common.h"
#include "internal.h"
#include "quant.h"

namespace mla {

namespace {

__global__ void __launch_bounds__(256) quantize_entries_kernel(bf16* __restrict__ src, int64_t src_ld, int n,
                                                               QuantDst dst, const bf16* __restrict__ gain, float eps,
                                                               bool writeback) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  quant::quantize_entry(src + (int64_t)row * src_ld, row, dst, gain, eps, writeback, lane);
}

}  // namespace

bool fp8_cache_ok(int d_c, int d_hr) { return d_c == quant::kDc && d_hr == quant::kDr; }

hipError_t quantize_entries_run(const void* src, int64_t src_ld, int n, const QuantDst& dst, hipStream_t s,
                                const void* gain, float eps, bool writeback) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_entries_kernel, dim3((n + 3) / 4), dim3(256), 0, s,
                     reinterpret_cast<bf16*>(const_cast<void*>(src)), src_ld, n, dst,
                     reinterpret_cast<const bf16*>(gain), eps, writeback);
  return hipGetLastError();
}

}  // namespace mla
