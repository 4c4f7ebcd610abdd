// Plain weight products through hipBLASLt: D[M][N] = A[M][K] B[N][K]^T, row-major, bf16 in, bf16
// (or fp32) out with fp32 accumulation and nothing fused on the way out.  The library's tuned kernels beat
// the hand-written weight-streaming and large-tile kernels on these shapes (measured on MI355X,
// e.g. 1.46 ms against 2.44 ms for the 16384-token output projection), so in prefill the products
// whose epilogue is a plain store go here; the ones with paging stay on the kernels in gemm.hip,
// and so do the decode products (64 rows), where the weight-streaming kernel is faster.
//
// hipBLASLt is column-major: the row-major D^T = B A^T is its D (N x M, ld ldd) = op(B) A' with
// B read as a K x N matrix (ld ldb) transposed and A as a K x M matrix (ld lda).
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "internal.h"

namespace mla {
namespace {

struct BlasPlan {
  bool ok = false;
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  size_t ws = 0;
};

using PlanKey = std::tuple<int, int, int, int, int64_t, int64_t, int64_t, size_t, bool>;

struct BlasState {
  std::mutex mu;
  std::map<int, hipblasLtHandle_t> handles;  // one per device, kept until the process ends
  std::map<PlanKey, BlasPlan> plans;
};

BlasState& state() {
  static BlasState* s = new BlasState();  // never destroyed: handles outlive static teardown
  return *s;
}

bool make_plan(hipblasLtHandle_t h, int M, int N, int K, int64_t lda, int64_t ldb, int64_t ldd, size_t ws_cap,
               bool d_f32, BlasPlan& p) {
  if (hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return false;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  if (hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) != HIPBLAS_STATUS_SUCCESS)
    return false;
  if (hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, N, ldb) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, M, lda) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.ld, d_f32 ? HIP_R_32F : HIP_R_16BF, N, M, ldd) != HIPBLAS_STATUS_SUCCESS)
    return false;
  hipblasLtMatmulPreference_t pref;
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return false;
  uint64_t cap = ws_cap;
  hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap, sizeof(cap));
  hipblasLtMatmulHeuristicResult_t res[1];
  int n = 0;
  const hipblasStatus_t st = hipblasLtMatmulAlgoGetHeuristic(h, p.op, p.la, p.lb, p.ld, p.ld, pref, 1, res, &n);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (st != HIPBLAS_STATUS_SUCCESS || n < 1 || res[0].workspaceSize > ws_cap) return false;
  p.algo = res[0].algo;
  p.ws = res[0].workspaceSize;
  return true;
}

}  // namespace

hipError_t blas_gemm_nt(const void* A, int64_t lda, const void* B, int64_t ldb, void* D, int64_t ldd, int M, int N,
                        int K, void* ws, size_t ws_bytes, hipStream_t s, bool d_f32) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  BlasState& S = state();
  BlasPlan* plan;
  hipblasLtHandle_t h;
  {
    std::lock_guard<std::mutex> lock(S.mu);
    auto hit = S.handles.find(dev);
    if (hit == S.handles.end()) {
      hipblasLtHandle_t nh;
      if (hipblasLtCreate(&nh) != HIPBLAS_STATUS_SUCCESS) return hipErrorNotSupported;
      hit = S.handles.emplace(dev, nh).first;
    }
    h = hit->second;
    const PlanKey key{dev, M, N, K, lda, ldb, ldd, ws_bytes, d_f32};
    auto pit = S.plans.find(key);
    if (pit == S.plans.end()) {
      BlasPlan p;
      p.ok = make_plan(h, M, N, K, lda, ldb, ldd, ws_bytes, d_f32, p);
      pit = S.plans.emplace(key, p).first;
    }
    plan = &pit->second;
  }
  if (!plan->ok) return hipErrorNotSupported;
  const float alpha = 1.f, beta = 0.f;
  const hipblasStatus_t st = hipblasLtMatmul(h, plan->op, &alpha, B, plan->la, A, plan->lb, &beta, D, plan->ld, D,
                                             plan->ld, &plan->algo, ws, plan->ws, s);
  return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace mla
