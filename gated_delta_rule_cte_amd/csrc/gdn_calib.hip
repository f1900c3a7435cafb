// Measurement aids for the benchmark (not part of the GDN interface): a dense
// bf16 MFMA throughput kernel, so that achieved prefill rates can be set
// beside a measured matrix-core ceiling as well as the published one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_calib.h"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kAcc = 8;  // independent accumulators per wave (covers the dependent-issue latency)

// Each wave issues `iters` x kAcc v_mfma_f32_16x16x32_bf16 (16384 flop each)
// and writes one value per lane so nothing is optimised away.
__global__ __launch_bounds__(64) void mfma_bf16_kernel(int iters, float* sink) {
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(1e-3f * (float)(threadIdx.x + j));
    b[j] = (__bf16)(1e-3f * (float)(j + 1));
  }
  f4 c[kAcc];
  for (int i = 0; i < kAcc; ++i) c[i] = f4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < kAcc; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  sink[(size_t)blockIdx.x * 64 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

double gdn_calib_mfma_bf16_flops(int waves, int iters) { return (double)waves * iters * kAcc * 16384.0; }

int gdn_calib_mfma_bf16(int waves, int iters, float* sink, void* stream) {
  if (waves <= 0 || iters <= 0 || !sink) return -1;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3((unsigned)waves), dim3(64), 0, static_cast<hipStream_t>(stream), iters,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // extern "C"
