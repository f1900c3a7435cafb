// gdn_cte: chunk-parallel gated delta-rule prefill.
// "GDN CTE Kernel API Reference", gdn_cte (summary, parameters, returns, Notes).
//
// Chunk form (one value head, chunk of C tokens, state H at the chunk start,
// gam = inclusive cumsum of g_log inside the chunk, Gam = exp(gam)):
//   A[t,i] = beta_t (k_t.k_i) exp(gam_t - gam_i)  for i < t        (strict lower)
//   T      = (I + A)^-1                                            (unit lower)
//   X      = beta * (V - Gam * (K H))
//   U      = T X                           (the per-token "new values" u_t)
//   O      = scale (Gam * (Q H) + P U),  P[t,i] = (q_t.k_i) exp(gam_t - gam_i), i <= t
//   H'     = Gam_C H + (exp(gam_C - gam) * K)^T U
// which is the token recurrence S_t = exp(g_t)(I - beta_t k_t k_t^T) S_{t-1}
// + beta_t k_t v_t^T, o_t = scale S_t^T q_t rewritten exactly.  Every decay
// factor is exp of a non-positive number, so nothing overflows.
//
// Every state column evolves independently, so one workgroup owns one
// (batch, value head, DVT-column tile) and carries its [DK, DVT] slice of the
// fp32 state in MFMA accumulators across all chunks.  The chunk-local products
// (K K^T, Q K^T, T) are recomputed by each tile's workgroup.
//
// Per chunk (4 waves, LDS-staged, barriers between phases):
//   0  coalesced loads of the K, Q, V tiles; wave 0 scans g_log
//   1  K~^T = (exp(gam_C - gam) K)^T built in LDS; K K^T -> A, Q K^T -> P on
//      MFMA (lower blocks only); K H -> X; Q H -> O accumulators
//   2  T = (I + A)^-1: 16x16 diagonal blocks by forward substitution (one lane
//      per column), off-diagonal blocks T_ij = -T_ii sum_m A_im T_mj level by
//      level on fp32 MFMA
//   3  U = T X (MFMA)
//   4  O += P U -> out;  H = Gam_C H + K~^T U (MFMA into the state accumulators)
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<__bf16>(__bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = f2bf(a); v[1] = f2bf(b); v[2] = f2bf(c); v[3] = f2bf(d);
  *reinterpret_cast<bf16x4*>(p) = v;
}

template <typename T, int DK, int DVT, int C>
__global__ __launch_bounds__(kThreads) void cte_kernel(const CteParams p) {
  using V8 = Vec8<T>;
  using MM = Mfma<T>;
  constexpr int PAD = 16 / sizeof(T);   // 16 bytes of row padding against bank conflicts
  constexpr int LDK = DK + PAD;         // pitch of [*, DK] tiles (K, Q, H^T)
  constexpr int LDC = C + PAD;          // pitch of [*, C] tiles (K~^T, T, P, X^T, U^T)
  constexpr int LDV = DVT + PAD;        // pitch of the V tile
  constexpr int LDA = C + 1;            // pitch of the fp32 A and T tiles
  constexpr int NB = C / 16;            // 16-token blocks per chunk
  constexpr int NKB = DK / 16;
  constexpr int NVB = DVT / 16;
  constexpr int NHB = NKB * NVB;        // 16x16 blocks of the state tile
  constexpr int HPW = NHB / kWaves;     // state blocks per wave
  constexpr int NOT = NB * NVB;         // 16x16 output blocks per chunk
  constexpr int OPW = (NOT + kWaves - 1) / kWaves;
  static_assert(NHB % kWaves == 0, "state tile must split evenly over the waves");
  static_assert(C % 32 == 0 && DK % 32 == 0 && DVT % 16 == 0, "tile shape");

  __shared__ __align__(16) T sK[C * LDK];
  __shared__ __align__(16) T sQ[C * LDK];
  __shared__ __align__(16) T sKt[DK * LDC];
  __shared__ __align__(16) T sHt[DVT * LDK];
  __shared__ __align__(16) T sV[C * LDV];
  __shared__ __align__(16) T sT[C * LDC];
  __shared__ __align__(16) T sP[C * LDC];
  __shared__ __align__(16) T sXt[DVT * LDC];
  __shared__ __align__(16) T sUt[DVT * LDC];
  __shared__ float sA[C * LDA];
  __shared__ float sTf[C * LDA];
  __shared__ float sZ[kWaves][16 * 17];
  __shared__ float sGam[C];
  __shared__ float sBeta[C];

  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int lr = lane & 15;
  const int lg = lane >> 4;

  const int S = p.S, Dk = p.Dk, Dv = p.Dv, Hv = p.Hv;
  const int ntiles = (Dv + DVT - 1) / DVT;
  const int tile = blockIdx.x % ntiles;
  const int bh = blockIdx.x / ntiles;
  const int b = bh / Hv, h = bh - b * Hv;
  const int hk = h / (Hv / p.Hk);
  const int col0 = tile * DVT;
  const float scale = p.scale;

  const T* qg = static_cast<const T*>(p.q) + (size_t)(b * p.Hk + hk) * S * Dk;
  const T* kg = static_cast<const T*>(p.k) + (size_t)(b * p.Hk + hk) * S * Dk;
  const T* vg = static_cast<const T*>(p.v) + (size_t)bh * S * Dv;
  const float* gg = p.g + (size_t)bh * S;
  const float* bg = p.beta + (size_t)bh * S;
  T* og = static_cast<T*>(p.out) + (size_t)bh * S * Dv;
  float* stg = p.state + (size_t)bh * Dk * Dv;

  // upper blocks of T and P are never written: zero them once
  for (int i = tid; i < C * LDC; i += kThreads) {
    sT[i] = from_f32<T>(0.f);
    sP[i] = from_f32<T>(0.f);
  }
  for (int i = tid; i < C * LDA; i += kThreads) sTf[i] = 0.f;

  // state tile -> accumulators (wave w owns blocks hb = w + 4j)
  f4 hacc[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int hb = w + kWaves * j, kb = hb / NVB, vb = hb % NVB;
    const int c = col0 + 16 * vb + lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = 16 * kb + 4 * lg + r;
      hacc[j][r] = (p.has_initial_state && kk < Dk && c < Dv) ? stg[(size_t)kk * Dv + c] : 0.f;
    }
    T* dst = sHt + (16 * vb + lr) * LDK + 16 * kb + 4 * lg;
    store4<T>(dst, hacc[j][0], hacc[j][1], hacc[j][2], hacc[j][3]);
  }

  f4 oacc[OPW];

  for (int c0 = 0; c0 < S; c0 += C) {
    const int nvalid = min(C, S - c0);

    // ---------------------------------------------------------------- 0 loads
    for (int it = tid; it < C * (DK / 8); it += kThreads) {
      const int t = it / (DK / 8), c8 = (it % (DK / 8)) * 8;
      const bool ok = t < nvalid && c8 < Dk;
      const size_t off = (size_t)(c0 + t) * Dk + c8;
      (ok ? V8::load(kg + off) : V8::zero()).store(sK + t * LDK + c8);
      (ok ? V8::load(qg + off) : V8::zero()).store(sQ + t * LDK + c8);
    }
    for (int it = tid; it < C * (DVT / 8); it += kThreads) {
      const int t = it / (DVT / 8), c8 = (it % (DVT / 8)) * 8;
      const bool ok = t < nvalid && col0 + c8 < Dv;
      (ok ? V8::load(vg + (size_t)(c0 + t) * Dv + col0 + c8) : V8::zero()).store(sV + t * LDV + c8);
    }
    if (w == 0) {
      const bool ok = lane < nvalid;
      const float gl = ok ? gg[c0 + lane] : 0.f;
      const float be = ok ? bg[c0 + lane] : 0.f;
      const float gam = wave_inclusive_scan(gl, lane);
      if (lane < C) {
        sGam[lane] = gam;
        sBeta[lane] = be;
      }
    }
    __syncthreads();

    // ------------------------------------------------- 1 chunk-local products
    {
      const float gC = sGam[C - 1];
      for (int it = tid; it < C * (DK / 8); it += kThreads) {
        const int t = it % C, c8 = (it / C) * 8;
        const V8 kv = V8::load(sK + t * LDK + c8);
        const float d = __expf(gC - sGam[t]);
#pragma unroll
        for (int j = 0; j < 8; ++j) sKt[(c8 + j) * LDC + t] = from_f32<T>(kv.get(j) * d);
      }
    }
    {
      // K K^T (A, strict lower) and Q K^T (P, lower incl. diagonal), lower 16x16 blocks
      constexpr int NT1 = NB * (NB + 1) / 2;
      for (int task = w; task < 2 * NT1; task += kWaves) {
        const bool isA = task < NT1;
        int tt = isA ? task : task - NT1;
        int bi = 0;
        while (tt > bi) { tt -= bi + 1; ++bi; }
        const int bj = tt;
        const T* X = isA ? sK : sQ;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DK / 32; ++s) {
          const V8 a = V8::load(X + (16 * bi + lr) * LDK + 32 * s + 8 * lg);
          const V8 bb = V8::load(sK + (16 * bj + lr) * LDK + 32 * s + 8 * lg);
          acc = MM::mma(a, bb, acc);
        }
        const int ii = 16 * bj + lr;
        const float gi = sGam[ii];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * bi + 4 * lg + r;
          if (isA) {
            sA[t * LDA + ii] = (ii < t) ? sBeta[t] * acc[r] * __expf(sGam[t] - gi) : 0.f;
          } else {
            sP[t * LDC + ii] = from_f32<T>((ii <= t) ? scale * acc[r] * __expf(sGam[t] - gi) : 0.f);
          }
        }
      }
      // K H -> X (to LDS, transposed) and Q H -> O accumulators
#pragma unroll
      for (int j = 0; j < OPW; ++j) {
        const int ot = w + kWaves * j;
        if (ot < NOT) {
          const int rb = ot / NVB, vb = ot % NVB;
          f4 kh = {0.f, 0.f, 0.f, 0.f}, qh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < DK / 32; ++s) {
            const V8 hb = V8::load(sHt + (16 * vb + lr) * LDK + 32 * s + 8 * lg);
            kh = MM::mma(V8::load(sK + (16 * rb + lr) * LDK + 32 * s + 8 * lg), hb, kh);
            qh = MM::mma(V8::load(sQ + (16 * rb + lr) * LDK + 32 * s + 8 * lg), hb, qh);
          }
          const int c = 16 * vb + lr;
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * rb + 4 * lg + r;
            const float G = __expf(sGam[t]);
            x[r] = sBeta[t] * (to_f32<T>(sV[t * LDV + c]) - G * kh[r]);
            oacc[j][r] = scale * G * qh[r];
          }
          store4<T>(sXt + c * LDC + 16 * rb + 4 * lg, x[0], x[1], x[2], x[3]);
        }
      }
    }
    __syncthreads();

    // ------------------------------------------------------- 2 T = (I + A)^-1
    if (w == 0) {
      const int blk = lane >> 4, j = lane & 15;
      if (blk < NB) {
        const float* Ab = sA + 16 * blk * LDA + 16 * blk;
        float tc[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) tc[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int i = 1; i < 16; ++i) {
          float acc = 0.f;
#pragma unroll
          for (int m = 0; m < i; ++m) acc += Ab[i * LDA + m] * tc[m];
          if (i > j) tc[i] = -acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sTf[(16 * blk + i) * LDA + 16 * blk + j] = tc[i];
          sT[(16 * blk + i) * LDC + 16 * blk + j] = from_f32<T>(tc[i]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < NB; ++d) {
      const int bj = w, bi = w + d;
      if (bi < NB) {
        // Z = sum_{m=bj}^{bi-1} A_{bi,m} T_{m,bj}
        f4 z = {0.f, 0.f, 0.f, 0.f};
        for (int m = bj; m < bi; ++m) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float av = sA[(16 * bi + lr) * LDA + 16 * m + 4 * s + lg];
            const float tv = sTf[(16 * m + 4 * s + lg) * LDA + 16 * bj + lr];
            z = __builtin_amdgcn_mfma_f32_16x16x4f32(av, tv, z, 0, 0, 0);
          }
        }
        float* Zw = sZ[w];
#pragma unroll
        for (int r = 0; r < 4; ++r) Zw[(4 * lg + r) * 17 + lr] = z[r];
        wave_lds_sync();
        // T_{bi,bj} = -T_{bi,bi} Z
        f4 tz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float tv = sTf[(16 * bi + lr) * LDA + 16 * bi + 4 * s + lg];
          const float zv = Zw[(4 * s + lg) * 17 + lr];
          tz = __builtin_amdgcn_mfma_f32_16x16x4f32(tv, zv, tz, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * bi + 4 * lg + r;
          sTf[t * LDA + 16 * bj + lr] = -tz[r];
          sT[t * LDC + 16 * bj + lr] = from_f32<T>(-tz[r]);
        }
      }
      __syncthreads();
    }

    // ----------------------------------------------------------- 3 U = T X
#pragma unroll
    for (int j = 0; j < OPW; ++j) {
      const int ot = w + kWaves * j;
      if (ot < NOT) {
        const int rb = ot / NVB, vb = ot % NVB;
        f4 u = {0.f, 0.f, 0.f, 0.f};
        const int nks = (16 * (rb + 1) + 31) / 32;
        for (int s = 0; s < nks; ++s) {
          const V8 a = V8::load(sT + (16 * rb + lr) * LDC + 32 * s + 8 * lg);
          const V8 xb = V8::load(sXt + (16 * vb + lr) * LDC + 32 * s + 8 * lg);
          u = MM::mma(a, xb, u);
        }
        store4<T>(sUt + (16 * vb + lr) * LDC + 16 * rb + 4 * lg, u[0], u[1], u[2], u[3]);
      }
    }
    __syncthreads();

    // --------------------------------------- 4 outputs and the state update
#pragma unroll
    for (int j = 0; j < OPW; ++j) {
      const int ot = w + kWaves * j;
      if (ot < NOT) {
        const int rb = ot / NVB, vb = ot % NVB;
        f4 o = oacc[j];
        const int nks = (16 * (rb + 1) + 31) / 32;
        for (int s = 0; s < nks; ++s) {
          const V8 a = V8::load(sP + (16 * rb + lr) * LDC + 32 * s + 8 * lg);
          const V8 ub = V8::load(sUt + (16 * vb + lr) * LDC + 32 * s + 8 * lg);
          o = MM::mma(a, ub, o);
        }
        const int c = col0 + 16 * vb + lr;
        if (c < Dv) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * rb + 4 * lg + r;
            if (t < nvalid) og[(size_t)(c0 + t) * Dv + c] = from_f32<T>(o[r]);
          }
        }
      }
    }
    {
      const float GC = __expf(sGam[C - 1]);
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const int hb = w + kWaves * j, kb = hb / NVB, vb = hb % NVB;
        f4 hcur = hacc[j];
        hcur[0] *= GC; hcur[1] *= GC; hcur[2] *= GC; hcur[3] *= GC;
#pragma unroll
        for (int s = 0; s < C / 32; ++s) {
          const V8 a = V8::load(sKt + (16 * kb + lr) * LDC + 32 * s + 8 * lg);
          const V8 ub = V8::load(sUt + (16 * vb + lr) * LDC + 32 * s + 8 * lg);
          hcur = MM::mma(a, ub, hcur);
        }
        hacc[j] = hcur;
        store4<T>(sHt + (16 * vb + lr) * LDK + 16 * kb + 4 * lg, hcur[0], hcur[1], hcur[2], hcur[3]);
      }
    }
    __syncthreads();
  }

  // final state tile -> HBM (fp32)
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int hb = w + kWaves * j, kb = hb / NVB, vb = hb % NVB;
    const int c = col0 + 16 * vb + lr;
    if (c < Dv) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = 16 * kb + 4 * lg + r;
        if (kk < Dk) stg[(size_t)kk * Dv + c] = hacc[j][r];
      }
    }
  }
}

template <typename T, int DK, int DVT, int C>
hipError_t launch_one(const CteParams& p, hipStream_t stream) {
  const int ntiles = (p.Dv + DVT - 1) / DVT;
  const long grid = (long)p.B * p.Hv * ntiles;
  hipLaunchKernelGGL((cte_kernel<T, DK, DVT, C>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// number of compute units on the target (MI355X)
constexpr long kCUs = 256;

int pick_dvt(const CteParams& p, int max_dvt) {
#ifdef GDN_CTE_FORCE_DVT
  return GDN_CTE_FORCE_DVT;
#endif
  const long heads = (long)p.B * p.Hv;
  int dvt = 16;
  for (int cand = max_dvt; cand >= 16; cand /= 2) {
    const long tiles = (p.Dv + cand - 1) / cand;
    if (heads * tiles >= kCUs || cand == 16) { dvt = cand; break; }
  }
  // never wider than the (16-rounded) value dimension
  while (dvt > 16 && dvt / 2 >= ((p.Dv + 15) / 16) * 16) dvt /= 2;
  return dvt;
}

}  // namespace

hipError_t launch_cte(const CteParams& p, int dtype, hipStream_t stream) {
  if ((long)p.B * p.Hv == 0) return hipSuccess;
  const bool dk64 = p.Dk <= 64;
  if (dtype == 1) {
    const int dvt = pick_dvt(p, 64);
    if (dk64) {
      if (dvt == 64) return launch_one<__bf16, 64, 64, 64>(p, stream);
      if (dvt == 32) return launch_one<__bf16, 64, 32, 64>(p, stream);
      return launch_one<__bf16, 64, 16, 64>(p, stream);
    }
    if (dvt == 64) return launch_one<__bf16, 128, 64, 64>(p, stream);
    if (dvt == 32) return launch_one<__bf16, 128, 32, 64>(p, stream);
    return launch_one<__bf16, 128, 16, 64>(p, stream);
  }
  const int dvt = pick_dvt(p, 32);
  if (dk64) {
    if (dvt == 32) return launch_one<float, 64, 32, 32>(p, stream);
    return launch_one<float, 64, 16, 32>(p, stream);
  }
  if (dvt == 32) return launch_one<float, 128, 32, 32>(p, stream);
  return launch_one<float, 128, 16, 32>(p, stream);
}

}  // namespace gdn
