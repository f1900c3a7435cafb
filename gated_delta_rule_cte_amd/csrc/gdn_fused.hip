// Prefill with the decode step's gates and output norm around gdn_cte.
// "GDN CTE Kernel API Reference" (gdn_cte: q, k must arrive unit-length; the
// output is un-normalised, with no fused epilogue) and "GDN TKG Kernel API
// Reference" (summary: l2norm(q, k), beta = sigmoid(b),
// g = -exp(A_log) softplus(a + dt_bias), the 1/sqrt(K) query scale and
// RMSNormGated(out, z)).
//
// HBM-bound row passes around the chunked prefill:
//   l2norm_rows_kernel    q^, k^ = x / sqrt(sum x^2 + 1e-6), rounded to the compute type;
//   gates_kernel          beta and g per token of every value head (A_log, dt_bias by head);
//   (gdn_cte with scale = Dk^-1/2 on q^, k^, v, g, beta)
//   rms_gate_rows_kernel  y = w * o / sqrt(mean(o^2) + eps) * silu(z) over Dv, in place
//                         (or written token-major, with z read token-major).
// In bf16 the first two are folded into the prefill's chunk-local kernel
// (which holds every key row of its chunk anyway); they run as passes for
// fp32 and where that kernel cannot write the unit rows over the raw ones.
// A row of up to 128 elements is one group of 16 lanes, 8 elements per lane,
// reduced with lane shuffles; 16 rows per workgroup of 256 threads.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kRowThreads = 256;
constexpr int kRowsPerBlock = kRowThreads / 16;
constexpr float kL2Eps = 1e-6f;

__device__ __forceinline__ void ld8(const float* p, float* x) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void ld8(const __bf16* p, float* x) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void st8(float* p, const float* x) {
  reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void st8(__bf16* p, const float* x) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = f2bf(x[i]);
  *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, f);
}
// sum over the 16 lanes of this lane's row group
__device__ __forceinline__ float row_sum16(float v) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m, 16);
  return v;
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void l2norm_rows_kernel(const FusedPre f) {
  const long row = (long)blockIdx.x * kRowsPerBlock + threadIdx.x / 16;
  const int j = threadIdx.x & 15;
  if (row >= 2 * f.rows_qk) return;  // whole row groups leave together
  const bool is_k = row >= f.rows_qk;
  const long r = is_k ? row - f.rows_qk : row;
  const T* src = static_cast<const T*>(is_k ? f.k : f.q) + r * f.Dk;
  T* dst = static_cast<T*>(is_k ? f.kn : f.qn) + r * f.Dk;
  const bool valid = 8 * j < f.Dk;
  float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (valid) ld8(src + 8 * j, x);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
  const float inv = 1.0f / sqrtf(row_sum16(ss) + kL2Eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] *= inv;
  if (valid) st8(dst + 8 * j, x);
}

__global__ __launch_bounds__(kRowThreads) void gates_kernel(const FusedPre f) {
  const long i = (long)blockIdx.x * kRowThreads + threadIdx.x;
  if (i >= f.tokens_v) return;
  const int h = (int)((i / f.S) % f.Hv);
  f.beta[i] = sigmoidf_(f.b[i]);
  f.g[i] = -expf(f.A_log[h]) * softplusf_(f.a[i] + f.dt_bias[h]);
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void rms_gate_rows_kernel(const FusedPost f) {
  const long row = (long)blockIdx.x * kRowsPerBlock + threadIdx.x / 16;
  const int j = threadIdx.x & 15;
  if (row >= f.rows) return;
  T* o = static_cast<T*>(f.out) + row * f.Dv;
  // row = (b Hv + h) S + t; its token-major index is (b S + t) Hv + h
  long tok_row = row;
  if (f.out_tok) {
    const long bh = row / f.S, t = row - bh * f.S, b = bh / f.Hv, h = bh - b * f.Hv;
    tok_row = (b * f.S + t) * f.Hv + h;
  }
  const T* z = static_cast<const T*>(f.z) + (f.out_tok && f.z_token_major ? tok_row : row) * f.Dv;
  const bool valid = 8 * j < f.Dv;
  float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, zz[8], w[8];
  if (valid) {
    ld8(o + 8 * j, x);
    ld8(z + 8 * j, zz);
    ld8(f.norm_weight + 8 * j, w);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
  const float rinv = 1.0f / sqrtf(row_sum16(ss) / (float)f.Dv + f.rms_eps);
  if (valid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = w[i] * x[i] * rinv * (zz[i] * sigmoidf_(zz[i]));
    T* dst = f.out_tok ? static_cast<T*>(f.out_tok) + tok_row * f.Dv : o;  // token-major [B, S, Hv Dv]
    st8(dst + 8 * j, x);
  }
}

}  // namespace

hipError_t launch_fused_pre(const FusedPre& f, int dtype, hipStream_t stream) {
  const long rows = 2 * f.rows_qk;
  if (rows > 0) {
    const unsigned grid = (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
    if (dtype == 1)
      hipLaunchKernelGGL(l2norm_rows_kernel<__bf16>, dim3(grid), dim3(kRowThreads), 0, stream, f);
    else
      hipLaunchKernelGGL(l2norm_rows_kernel<float>, dim3(grid), dim3(kRowThreads), 0, stream, f);
  }
  if (f.tokens_v > 0)
    hipLaunchKernelGGL(gates_kernel, dim3((unsigned)((f.tokens_v + kRowThreads - 1) / kRowThreads)),
                       dim3(kRowThreads), 0, stream, f);
  return hipGetLastError();
}

hipError_t launch_fused_post(const FusedPost& f, int dtype, hipStream_t stream) {
  if (f.rows <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((f.rows + kRowsPerBlock - 1) / kRowsPerBlock);
  if (dtype == 1)
    hipLaunchKernelGGL(rms_gate_rows_kernel<__bf16>, dim3(grid), dim3(kRowThreads), 0, stream, f);
  else
    hipLaunchKernelGGL(rms_gate_rows_kernel<float>, dim3(grid), dim3(kRowThreads), 0, stream, f);
  return hipGetLastError();
}

}  // namespace gdn
