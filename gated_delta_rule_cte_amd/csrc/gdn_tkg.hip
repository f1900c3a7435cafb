// gdn_tkg: fused single-token gated delta-rule decode step.
// "GDN TKG Kernel API Reference", gdn_tkg (summary, parameters, Notes).
//
// One workgroup per head bh.  The step is a pair of mat-vecs over the head's
// [K, V] fp32 state plus a rank-1 update, so it is bound by HBM bandwidth:
// the state is read once and written once and everything else is O(K + V).
//
//   thread t of NT: float4 column group cg = t % 32 (columns 4cg..4cg+3)
//   and row group rg = t / 32 (rows rg, rg + NT/32, ...): 128 / (NT/32)
//   float4 of state in registers, loaded before the prologue so the loads are
//   in flight while wave 0 normalises q and k.  NT = 512 keeps 32 state
//   floats per thread and the kernel under 64 VGPRs: eight waves per SIMD,
//   so 1024 heads fill the chip in one round.  More heads than that are
//   split into launches of at most one round each (see launch_tkg).
//
//   r = S^T k^ and p = S^T q^ are reduced over the row groups through LDS in
//   a fixed order (bitwise reproducible; one thread per column, so few
//   registers are live next to the state), then per column
//     u = beta (v - alpha r),  S' = alpha S + k^ u^T,  o = alpha p + (k^.q^) u
//   which equals o = S'^T q^ without a second pass over the state.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kColGroups = 32;  // float4 column groups, V <= 128
constexpr float kL2Eps = 1e-6f;
// heads per round of the 512-thread form (four workgroups per CU)
constexpr long kOneRound = 4 * 256;
// buffer descriptor word 3 for raw (untyped, stride 0) buffers on gfx9-family parts
constexpr int kBufferFlags = 0x00020000;
// cache policy: non-temporal (the state is streamed exactly once each way)
constexpr int kNonTemporal = 2;

template <typename T>
__device__ __forceinline__ float4 load4(const T* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<__bf16>(const __bf16* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
}

template <typename T, int NT>
__global__ __launch_bounds__(NT, 4) void tkg_kernel(const TkgParams p) {
  constexpr int kThreads = NT;
  constexpr int kRowGroups = kThreads / kColGroups;  // 16 or 8
  constexpr int kRowsPerThread = 128 / kRowGroups;   // 8 or 16
  __shared__ float s_q[128];
  __shared__ float s_k[128];
  __shared__ float4 s_red[2][kRowGroups][kColGroups];  // partial S^T k^, S^T q^
  __shared__ float4 s_tot[2][kColGroups];              // their sums over row groups
  __shared__ float s_scal[3];  // alpha, beta, k^.q^

  const int bh = p.bh0 + (int)blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int cg = tid % kColGroups;
  const int rg = tid / kColGroups;
  const int K = p.K, V = p.V;
  const int bi = bh / p.Hv, h = bh - bi * p.Hv;
  const bool col_ok = 4 * cg < V;

  // The head's state through buffer descriptors: one 32-bit VGPR offset per
  // thread plus a uniform SGPR offset per row step keeps the row addresses
  // out of the VGPR budget.  Steps i with kRowGroups * i >= K hold no row
  // and are skipped (uniform); inside the last step, rows past K and threads
  // past the last column group land beyond the descriptor's range (loads
  // return zero, stores are dropped).
  const uint32_t head_bytes = (uint32_t)(K * V * 4);
  const __amdgpu_buffer_rsrc_t rin = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p.state_in + (size_t)bh * K * V), (short)0, head_bytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(
      p.state_out + (size_t)bh * K * V, (short)0, head_bytes, kBufferFlags);
  const uint32_t voff = col_ok ? (uint32_t)((rg * V + 4 * cg) * 4) : 0x40000000u;
  const uint32_t row_step = (uint32_t)(kRowGroups * V * 4);
  const int nrow = (K + kRowGroups - 1) / kRowGroups;

  // 1. this thread's state slab -> registers
  f4 s[kRowsPerThread];
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i)
    s[i] = (i < nrow) ? __builtin_amdgcn_raw_buffer_load_b128(rin, voff, i * row_step, kNonTemporal)
                      : f4{0.f, 0.f, 0.f, 0.f};

  // 2. prologue (wave 0): l2norm(q) / sqrt(K), l2norm(k), beta, g
  if (tid < kWave) {
    const size_t row = (size_t)bi * p.qk_bstride + (size_t)(h / p.head_div) * K;
    const T* q = static_cast<const T*>(p.q) + row;
    const T* k = static_cast<const T*>(p.k) + row;
    float q0 = lane < K ? to_f32<T>(q[lane]) : 0.f;
    float q1 = lane + kWave < K ? to_f32<T>(q[lane + kWave]) : 0.f;
    float k0 = lane < K ? to_f32<T>(k[lane]) : 0.f;
    float k1 = lane + kWave < K ? to_f32<T>(k[lane + kWave]) : 0.f;
    const float qq = wave_sum(q0 * q0 + q1 * q1);
    const float kk = wave_sum(k0 * k0 + k1 * k1);
    const float qs = (1.0f / sqrtf(qq + kL2Eps)) * (1.0f / sqrtf((float)K));
    const float ks = 1.0f / sqrtf(kk + kL2Eps);
    q0 *= qs; q1 *= qs; k0 *= ks; k1 *= ks;
    s_q[lane] = q0; s_q[lane + kWave] = q1;
    s_k[lane] = k0; s_k[lane + kWave] = k1;
    const float kq = wave_sum(q0 * k0 + q1 * k1);
    if (lane == 0) {
      const float beta = sigmoidf_(p.b[bh]);
      const float g = -expf(p.A_log[h]) * softplusf_(p.a[bh] + p.dt_bias[h]);
      s_scal[0] = expf(g);
      s_scal[1] = beta;
      s_scal[2] = kq;
    }
  }
  __syncthreads();

  // 3. partial S^T k^ and S^T q^ over this thread's rows
  float4 pr = make_float4(0.f, 0.f, 0.f, 0.f), pp = pr;
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int r = rg + kRowGroups * i;
    const float kr = s_k[r], qr = s_q[r];
    pr.x += s[i].x * kr; pr.y += s[i].y * kr; pr.z += s[i].z * kr; pr.w += s[i].w * kr;
    pp.x += s[i].x * qr; pp.y += s[i].y * qr; pp.z += s[i].z * qr; pp.w += s[i].w * qr;
  }
  s_red[0][rg][cg] = pr;
  s_red[1][rg][cg] = pp;
  __syncthreads();
  if (tid < 256) {
    // thread t sums one of the 2 x 128 columns over the row groups (fixed order)
    const float* red = reinterpret_cast<const float*>(s_red);
    const int which = tid / 128, col = tid % 128;
    float acc = red[(which * kRowGroups + 0) * 128 + col];
#pragma unroll
    for (int g = 1; g < kRowGroups; ++g) acc += red[(which * kRowGroups + g) * 128 + col];
    reinterpret_cast<float*>(s_tot)[which * 128 + col] = acc;
  }
  __syncthreads();
  const float4 R = s_tot[0][cg], P = s_tot[1][cg];

  // 4. u = beta (v - alpha r), o = alpha p + (k^.q^) u
  const float alpha = s_scal[0], beta = s_scal[1], kq = s_scal[2];
  float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
  if (col_ok) {
    const T* vrow = static_cast<const T*>(p.v) + (size_t)bi * p.v_bstride + (size_t)h * V;
    const float4 v = load4<T>(vrow + 4 * cg);
    u = make_float4(beta * (v.x - alpha * R.x), beta * (v.y - alpha * R.y),
                    beta * (v.z - alpha * R.z), beta * (v.w - alpha * R.w));
  }

  // 5. S' = alpha S + k^ u^T, written once (streaming stores)
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    if (i < nrow) {
      const float kr = s_k[rg + kRowGroups * i];
      const f4 o4 = {alpha * s[i].x + kr * u.x, alpha * s[i].y + kr * u.y,
                     alpha * s[i].z + kr * u.z, alpha * s[i].w + kr * u.w};
      __builtin_amdgcn_raw_buffer_store_b128(o4, rout, voff, i * row_step, kNonTemporal);
    }
  }

  // 6. RMSNormGated on row group 0 (lanes 0..31 of wave 0 hold all V columns)
  if (rg == 0) {
    const float4 o = make_float4(alpha * P.x + kq * u.x, alpha * P.y + kq * u.y,
                                 alpha * P.z + kq * u.z, alpha * P.w + kq * u.w);
    float ss = col_ok ? (o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w) : 0.f;
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    if (col_ok) {
      const float rinv = 1.0f / sqrtf(ss / (float)V + p.rms_eps);
      const float4 z = load4<T>(static_cast<const T*>(p.z) + (size_t)bh * V + 4 * cg);
      const float4 w = *reinterpret_cast<const float4*>(p.norm_weight + 4 * cg);
      bf16x4 y;
      y[0] = f2bf(w.x * o.x * rinv * (z.x * sigmoidf_(z.x)));
      y[1] = f2bf(w.y * o.y * rinv * (z.y * sigmoidf_(z.y)));
      y[2] = f2bf(w.z * o.z * rinv * (z.z * sigmoidf_(z.z)));
      y[3] = f2bf(w.w * o.w * rinv * (z.w * sigmoidf_(z.w)));
      *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + (size_t)bh * V + 4 * cg) = y;
    }
  }
}

}  // namespace

hipError_t launch_tkg(const TkgParams& p, int dtype, hipStream_t stream) {
  // One launch per round of the 512-thread form (at most 1024 heads, every
  // workgroup resident at once), the heads spread evenly over the launches.
  // All workgroups of a one-round launch start together, so the state reads
  // come first and the write-back after; in a two-round launch the second
  // round's reads meet the first round's writes.  At 2048 heads two launches
  // of 1024 took 44.9 us against 49.3 us for one launch of 256 threads and
  // about 50 us for one of 512.
  const int n = (int)((p.BH + kOneRound - 1) / kOneRound);
  if (n == 0) return hipSuccess;
  const int per = (p.BH + n - 1) / n;
  for (int h0 = 0; h0 < p.BH; h0 += per) {
    TkgParams q = p;
    q.bh0 = h0;
    const unsigned grid = (unsigned)(p.BH - h0 < per ? p.BH - h0 : per);
    if (dtype == 1)
      hipLaunchKernelGGL((tkg_kernel<__bf16, 512>), dim3(grid), dim3(512), 0, stream, q);
    else
      hipLaunchKernelGGL((tkg_kernel<float, 512>), dim3(grid), dim3(512), 0, stream, q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
