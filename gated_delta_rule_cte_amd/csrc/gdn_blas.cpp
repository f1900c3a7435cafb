// The prefill layer's in_proj products are plain GEMMs (bf16 operands, fp32
// accumulation, bf16 out, all row-major): they go to the vendor library
// (hipBLASLt) with its heuristic's first algorithm and no workspace, so no
// split-K reduction pass runs and nothing is allocated per call.  The plan of
// each shape (descriptors and algorithm) is made once per device and kept.
// "GDN Block TKG Kernel API Reference" (summary: the in_proj projection) read
// for a whole sequence.
#include <hipblaslt/hipblaslt.h>

#include <list>
#include <mutex>

#include "gdn_launch.h"

namespace gdn {
namespace {

struct Plan {
  int M, N, K;
  hipblasLtMatmulDesc_t op;
  hipblasLtMatrixLayout_t la, lb, lc;
  hipblasLtMatmulAlgo_t algo;
};
struct DeviceBlas {
  bool tried = false;
  hipblasLtHandle_t h = nullptr;
  std::list<Plan> plans;  // stable addresses
};
constexpr int kMaxDevices = 64;
std::mutex g_blas_mu;
DeviceBlas g_blas[kMaxDevices];

// Row-major C[M, N] = A[M, K] B[K, N] seen column-major is C^T = B^T A^T with
// B^T an N x K matrix of leading dimension N and A^T a K x M matrix of leading
// dimension K: no transposes, the library's first operand is B.
Plan* plan_for(DeviceBlas& d, int M, int N, int K) {
  for (Plan& p : d.plans)
    if (p.M == M && p.N == N && p.K == K) return &p;
  Plan p{M, N, K, nullptr, nullptr, nullptr, nullptr, {}};
  bool good = hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  const hipblasOperation_t nt = HIPBLAS_OP_N;
  good = good && hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSA, &nt, sizeof(nt)) == HIPBLAS_STATUS_SUCCESS;
  good = good && hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSB, &nt, sizeof(nt)) == HIPBLAS_STATUS_SUCCESS;
  good = good && hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, N, K, N) == HIPBLAS_STATUS_SUCCESS;
  good = good && hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, M, K) == HIPBLAS_STATUS_SUCCESS;
  good = good && hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_16BF, N, M, N) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulPreference_t pref = nullptr;
  good = good && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
  const uint64_t no_ws = 0;
  good = good && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &no_ws,
                                                       sizeof(no_ws)) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulHeuristicResult_t res{};
  int got = 0;
  good = good && hipblasLtMatmulAlgoGetHeuristic(d.h, p.op, p.la, p.lb, p.lc, p.lc, pref, 1, &res, &got) ==
                     HIPBLAS_STATUS_SUCCESS && got > 0;
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (!good) {
    if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
    if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
    if (p.lc) hipblasLtMatrixLayoutDestroy(p.lc);
    if (p.op) hipblasLtMatmulDescDestroy(p.op);
    return nullptr;
  }
  p.algo = res.algo;
  d.plans.push_back(p);
  return &d.plans.back();
}

}  // namespace

hipError_t gemm_bf16_library(const void* A, const void* B, void* C, int M, int N, int K, hipStream_t stream) {
  if (M <= 0 || N <= 0 || K <= 0) return hipErrorNotSupported;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return hipErrorNotSupported;
  std::lock_guard<std::mutex> lock(g_blas_mu);
  DeviceBlas& d = g_blas[dev];
  if (!d.tried) {
    d.tried = true;
    if (hipblasLtCreate(&d.h) != HIPBLAS_STATUS_SUCCESS) d.h = nullptr;
  }
  if (!d.h) return hipErrorNotSupported;
  Plan* p = plan_for(d, M, N, K);
  if (!p) return hipErrorNotSupported;
  const float alpha = 1.f, beta = 0.f;
  if (hipblasLtMatmul(d.h, p->op, &alpha, B, p->la, A, p->lb, &beta, C, p->lc, C, p->lc, &p->algo, nullptr, 0,
                      stream) != HIPBLAS_STATUS_SUCCESS)
    return hipErrorNotSupported;
  return hipSuccess;
}

}  // namespace gdn
