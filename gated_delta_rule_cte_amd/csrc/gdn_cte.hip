// gdn_cte: chunk-parallel gated delta-rule prefill.
// "GDN CTE Kernel API Reference", gdn_cte (summary, parameters, returns, Notes).
//
// Chunk form (one value head, chunk of C tokens, state H at the chunk start,
// gam = inclusive cumsum of g_log inside the chunk, Gam = exp(gam)):
//   A[t,i] = beta_t (k_t.k_i) exp(gam_t - gam_i)  for i < t        (strict lower)
//   T      = (I + A)^-1                                            (unit lower)
//   P[t,i] = scale (q_t.k_i) exp(gam_t - gam_i)   for i <= t
//   X      = beta * (V - Gam * (K H))
//   U      = T X                                   (the per-token new values)
//   O      = scale Gam * (Q H) + P U
//   H'     = Gam_C H + (exp(gam_C - gam) * K)^T U
// which is the token recurrence S_t = exp(g_t)(I - beta_t k_t k_t^T) S_{t-1}
// + beta_t k_t v_t^T, o_t = scale S_t^T q_t rewritten exactly.  Every decay
// factor is exp of a non-positive number, so nothing overflows.
//
// Two kernels:
//  1. cte_local_kernel, one workgroup per (batch, value head, chunk), all
//     chunks in parallel: K K^T and Q K^T on MFMA with the decays applied in
//     the epilogue, then (I + A)^-1 by blocked forward substitution (16x16
//     diagonal blocks one lane per column, off-diagonal blocks
//     T_ij = -T_ii sum_m A_im T_mj level by level on fp32 MFMA); T and P go to
//     the workspace with 16-byte stores.  Nothing here depends on the state.
//  2. cte_state_kernel, one workgroup per (batch, value head, DVT state
//     columns): the sequential pass over the chunks.  State columns evolve
//     independently, so the workgroup carries its [DK, DVT] fp32 slice in
//     MFMA accumulators.  Chunk data is prefetched into registers two chunks
//     ahead and staged into LDS at the end of the previous chunk, leaving
//     three barrier-separated phases per chunk on the critical path:
//     K H -> X, Q H | U = T X | O = scale Gam Q H + P U, H' = Gam_C H + K~^T U.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kC = 64;        // chunk length (one 16-row block per wave)
constexpr int kNB = kC / 16;  // 16-token blocks per chunk
constexpr int kAlgoNeumann = 1;  // intra-chunk inverse by the doubling Neumann product
constexpr float kL2Eps = 1e-6f;   // l2norm(x) = x / sqrt(sum x^2 + kL2Eps) in the folded prologue

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

template <typename T>
__device__ __forceinline__ void store2(T* p, float a, float b);
template <>
__device__ __forceinline__ void store2<float>(float* p, float a, float b) {
  *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
template <>
__device__ __forceinline__ void store2<__bf16>(__bf16* p, float a, float b) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, f2bf(a));
  const uint32_t hi = __builtin_bit_cast(uint16_t, f2bf(b));
  *reinterpret_cast<uint32_t*>(p) = lo | (hi << 16);
}

// T (bf16 or fp32) workspace of one (batch*value head, chunk): fp32, T then
// P, each [C][C]; bf16, the lower 16x16 blocks of T, then those of P, packed
// as 16-byte items (block in row-major lower order, row, half) in the order
// the state pass reads them
template <typename T>
__device__ __forceinline__ T* ws_chunk(void* ws, int bh, int NC, int c) {
  return static_cast<T*>(ws) + ((size_t)bh * NC + c) * 2 * kC * kC;
}

// ===========================================================================
// kernel 1: chunk-local products and the triangular inverse
// ===========================================================================
// One workgroup per (batch * value head, chunk).  LDS: the K and Q tiles are
// dead once the raw products sit in registers, so the fp32 A matrix reuses the
// K tile's bytes and the staged P block the Q tile's.
template <typename T, int DK, int ALGO>
__global__ __launch_bounds__(kThreads) void cte_local_kernel(const CteParams p) {
  using V8 = Vec8<T>;
  using MM = Mfma<T>;
  constexpr int C = kC, NB = kNB;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int LDK = DK + PAD;
  constexpr int LDC = C + PAD;
  constexpr int LDA = C + 4;                 // fp32 rows stay 16-byte aligned
  constexpr int NIT = C * (DK / 8) / kThreads;
  constexpr int kTileBytes = C * LDK * (int)sizeof(T);
  constexpr int kABytes = C * LDA * 4;
  constexpr int kPBytes = C * LDC * (int)sizeof(T);
  constexpr int kBufBytes = (2 * kTileBytes > kABytes + kPBytes) ? 2 * kTileBytes : kABytes + kPBytes;
  static_assert(NIT * kThreads == C * (DK / 8), "K/Q tile split");

  __shared__ __align__(16) char sbuf[kBufBytes];
  __shared__ __align__(16) float sTf[C * LDA];
  __shared__ float sZ[kWaves][16 * 17];
  __shared__ float sGam[C];
  __shared__ float sBeta[C];
  T* sK = reinterpret_cast<T*>(sbuf);
  T* sQ = reinterpret_cast<T*>(sbuf + kTileBytes);
  float* sA = reinterpret_cast<float*>(sbuf);           // after the raw products
  T* sPs = reinterpret_cast<T*>(sbuf + kABytes);         // staged P, after the raw products

  const int tid = threadIdx.x, w = tid / kWave, lane = tid & (kWave - 1);
  const int lr = lane & 15, lg = lane >> 4;
  const int S = p.S, Dk = p.Dk, Hk = p.Hk, Hv = p.Hv;
  const int NC = (S + C - 1) / C;
  // logical id = ((b * Hk + hk) * NC + c) * G + hh: the G value heads that
  // share a key head's chunk are neighbours (and so share an XCD's L2)
  const int G = Hv / Hk;
  const int lid = xcd_logical_id(blockIdx.x, (int)gridDim.x);
  const int hh = lid % G;
  const int nseg = p.c_end - p.c_begin;
  const int c = p.c_begin + (lid / G) % nseg;
  const int bhk = lid / (G * nseg);
  const int b = bhk / Hk, hk = bhk - b * Hk;
  const int h = hk * G + hh;
  const int bh = b * Hv + h;
  const int c0 = c * C, nvalid = min(C, S - c0);
  const float scale = p.scale;

  // K, Q chunk tiles (all loads issued before the first store); g, beta
  {
    const T* kg = static_cast<const T*>(p.k) + ((size_t)(b * Hk + hk) * S + c0) * Dk;
    const T* qg = static_cast<const T*>(p.q) + ((size_t)(b * Hk + hk) * S + c0) * Dk;
    V8 kr[NIT], qr[NIT];
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int it = tid + kThreads * i, t = it / (DK / 8), c8 = (it % (DK / 8)) * 8;
      const bool ok = t < nvalid && c8 < Dk;
      kr[i] = ok ? V8::load(kg + (size_t)t * Dk + c8) : V8::zero();
      qr[i] = ok ? V8::load(qg + (size_t)t * Dk + c8) : V8::zero();
    }
    float gl = 0.f, be = 0.f;
    if (w == 0 && lane < nvalid) {
      gl = p.g[(size_t)bh * S + c0 + lane];
      be = p.beta[(size_t)bh * S + c0 + lane];
    }
#pragma unroll
    for (int i = 0; i < NIT; ++i) {
      const int it = tid + kThreads * i, t = it / (DK / 8), c8 = (it % (DK / 8)) * 8;
      kr[i].store(sK + t * LDK + c8);
      qr[i].store(sQ + t * LDK + c8);
    }
    if (w == 0) {
      sGam[lane] = wave_inclusive_scan_dpp(gl);
      sBeta[lane] = be;
    }
  }
  __syncthreads();

  // raw K K^T for row block w and Q K^T for row block NB-1-w (lower blocks)
  const int rk = w, rq = NB - 1 - w;
  f4 kk[NB], qk[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    kk[j] = f4{0.f, 0.f, 0.f, 0.f};
    qk[j] = f4{0.f, 0.f, 0.f, 0.f};
    if (j <= rk) {
#pragma unroll
      for (int s = 0; s < DK / 32; ++s)
        kk[j] = MM::mma(V8::load(sK + (16 * rk + lr) * LDK + 32 * s + 8 * lg),
                        V8::load(sK + (16 * j + lr) * LDK + 32 * s + 8 * lg), kk[j]);
    }
    if (j <= rq) {
#pragma unroll
      for (int s = 0; s < DK / 32; ++s)
        qk[j] = MM::mma(V8::load(sQ + (16 * rq + lr) * LDK + 32 * s + 8 * lg),
                        V8::load(sK + (16 * j + lr) * LDK + 32 * s + 8 * lg), qk[j]);
    }
  }
  __syncthreads();  // K, Q tiles are dead from here on

  // decays: A (fp32) into the K tile's bytes, P (compute type) into the Q tile's
  {
    float gt[4], bt[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      gt[r] = sGam[16 * rk + 4 * lg + r];
      bt[r] = sBeta[16 * rk + 4 * lg + r];
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j <= rk) {
        const int i = 16 * j + lr;
        const float gi = sGam[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * rk + 4 * lg + r;
          sA[t * LDA + i] = (i < t) ? bt[r] * kk[j][r] * __expf(gt[r] - gi) : 0.f;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) gt[r] = sGam[16 * rq + 4 * lg + r];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j <= rq) {
        const int i = 16 * j + lr;
        const float gi = sGam[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * rq + 4 * lg + r;
          sPs[t * LDC + i] = from_f32<T>((i <= t) ? scale * qk[j][r] * __expf(gt[r] - gi) : 0.f);
        }
      }
    }
  }
  __syncthreads();

  if constexpr (ALGO == kAlgoNeumann) {
    // T = (I - A)(I + A^2)(I + A^4) ... (I + A^32), as in the bf16 kernel:
    // Pw <- Pw Pw, T <- T + T Pw, five times; wave w owns block row w of both
    // (blocks (w, j), j <= w), in accumulator form, and both are kept in row
    // form in LDS (Pw in sA, T in sTf) as the operands of the next products.
    f4 pw[NB], tt[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (j <= w)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = sA[(16 * w + 4 * lg + r) * LDA + 16 * j + lr];
          pw[j][r] = -a;
          tt[j][r] = (j == w && 4 * lg + r == lr) ? 1.f - a : -a;
        }
    __syncthreads();
    auto put = [&](float* dst, const f4* src) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (j <= w)
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[(16 * w + 4 * lg + r) * LDA + 16 * j + lr] = src[j][r];
    };
    put(sA, pw);
    put(sTf, tt);
    __syncthreads();
    // block (w, j) of X Y with X in row form (first operand) and Y in LDS
    auto prod = [&](const float* X, const float* Y, int j, f4 z) {
#pragma unroll
      for (int m = 0; m < NB; ++m)
        if (m >= j && m <= w)
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
            z = __builtin_amdgcn_mfma_f32_16x16x4f32(X[(16 * w + lr) * LDA + 16 * m + 4 * s4 + lg],
                                                     Y[(16 * m + 4 * s4 + lg) * LDA + 16 * j + lr], z, 0, 0, 0);
      return z;
    };
#pragma unroll 1
    for (int step = 1; step < 6; ++step) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (j <= w) pw[j] = prod(sA, sA, j, f4{0.f, 0.f, 0.f, 0.f});
      __syncthreads();
      put(sA, pw);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < NB; ++j)
        if (j <= w) tt[j] = prod(sTf, sA, j, tt[j]);
      __syncthreads();
      put(sTf, tt);
      __syncthreads();
    }
  } else {
    // diagonal 16x16 blocks of T: lane = (block, column), forward substitution
    if (w == 0) {
      const int blk = lane >> 4, j = lane & 15;
      const float* Ab = sA + 16 * blk * LDA + 16 * blk;
      float tc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) tc[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        float row[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(Ab + i * LDA + 4 * q);
          row[4 * q] = v.x; row[4 * q + 1] = v.y; row[4 * q + 2] = v.z; row[4 * q + 3] = v.w;
        }
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) acc += row[m] * tc[m];
        if (i > j) tc[i] = -acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sTf[(16 * blk + i) * LDA + 16 * blk + j] = tc[i];
    }
    __syncthreads();

    // off-diagonal blocks, one level (block distance d) at a time
#pragma unroll
    for (int d = 1; d < NB; ++d) {
      const int bj = w, bi = w + d;
      if (bi < NB) {
        f4 z = {0.f, 0.f, 0.f, 0.f};
        for (int m = bj; m < bi; ++m) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            z = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * bi + lr) * LDA + 16 * m + 4 * s + lg],
                                                     sTf[(16 * m + 4 * s + lg) * LDA + 16 * bj + lr], z, 0, 0, 0);
        }
        float* Zw = sZ[w];
#pragma unroll
        for (int r = 0; r < 4; ++r) Zw[(4 * lg + r) * 17 + lr] = z[r];
        wave_lds_sync();
        f4 tz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          tz = __builtin_amdgcn_mfma_f32_16x16x4f32(sTf[(16 * bi + lr) * LDA + 16 * bi + 4 * s + lg],
                                                    Zw[(4 * s + lg) * 17 + lr], tz, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) sTf[(16 * bi + 4 * lg + r) * LDA + 16 * bj + lr] = -tz[r];
      }
      __syncthreads();
    }
  }

  // T (lower blocks, rounded to the compute type) and P -> workspace, 16-byte stores
  T* Tg = ws_chunk<T>(p.ws, bh, NC, c);
  T* Pg = Tg + C * C;
#pragma unroll
  for (int i = 0; i < C * (C / 8) / kThreads; ++i) {
    const int it = tid + kThreads * i, t = it / (C / 8), c8 = (it % (C / 8)) * 8;
    if ((c8 >> 4) > (t >> 4)) continue;  // upper blocks are never read
    const float* src = sTf + t * LDA + c8;
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 bq = *reinterpret_cast<const float4*>(src + 4);
    V8 v;
    if constexpr (sizeof(T) == 2) {
      bf16x8 f;
      f[0] = f2bf(a.x); f[1] = f2bf(a.y); f[2] = f2bf(a.z); f[3] = f2bf(a.w);
      f[4] = f2bf(bq.x); f[5] = f2bf(bq.y); f[6] = f2bf(bq.z); f[7] = f2bf(bq.w);
      v.u = __builtin_bit_cast(uint4, f);
    } else {
      v.a = a;
      v.b = bq;
    }
    v.store(Tg + t * C + c8);
    V8::load(sPs + t * LDC + c8).store(Pg + t * C + c8);
  }
}

// ===========================================================================
// kernel 1, bf16: one wave per chunk
// ===========================================================================
// The same chunk-local products as above with no workgroup barrier: one
// wave computes a whole chunk, so many chunks are in flight per CU.
//  - With FUSE the decode step's prologue runs here first (the "GDN TKG
//    Kernel API Reference" summary: l2norm of q and k, beta = sigmoid(b),
//    g = -exp(A_log) softplus(a + dt_bias)): raw rows are made unit length in
//    the fragments and written once per key head and chunk for the state
//    pass, with beta and g.
//  - K and Q arrive straight from HBM as MFMA fragments (16 bytes per lane).
//  - A and P are produced transposed (the K rows of block j as the first
//    operand), so a lane holds 4 consecutive columns of one row and writes
//    them with one store.
//  - Lower 16x16 blocks of A and T are kept packed in LDS (row pitch of 20
//    floats: the row reads below hit 16 distinct bank groups).
//  - Diagonal blocks of T by forward substitution (lane = block, column);
//    off-diagonal blocks level by level, T_ij = -T_ii sum_m A_im T_mj, on
//    fp32 MFMA with a permuted contraction index (16x16x4 instruction s
//    takes index 4 (l / 16) + s): the first operand is 4 consecutive columns
//    of a row (one LDS read), the second is the accumulator layout itself, so
//    the partial sums and the T blocks never leave the registers.
constexpr int kLB = 20;         // fp32 row pitch of a packed 16x16 block
constexpr int kBlkF = 16 * kLB;  // floats per packed block
constexpr int kNTri = kNB * (kNB + 1) / 2;
constexpr int kTriItems = kNTri * 16 * 2;  // 16-byte bf16 items in the lower 16x16 blocks of a C x C tile

__device__ __forceinline__ constexpr int tri(int i, int j) { return i * (i + 1) / 2 + j; }

// sum over s of X[m][4 (l/16) + s] Y[4 (l/16) + s][n]: a4 = this lane's row
// segment of X, b = Y in the accumulator layout
__device__ __forceinline__ f4 mfma4_f32(float4 a4, f4 b, f4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.x, b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.y, b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.z, b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.w, b[3], c, 0, 0, 0);
  return c;
}

// One workgroup per (chunk, key head, NG * NH value heads of its GQA group):
// NG waves of NH value heads each, taken in turn.  The waves of a workgroup
// load the same K and Q rows (the second read hits the cache) and form the
// same raw K K^T and Q K^T; each head then gets its own beta and decays.
// The plain prefill runs one head per wave (NG = 2, NH = 1); the folded
// prologue runs one wave for both heads of a pair (NG = 1, NH = 2), since
// its unit rows replace the raw ones in place.  Each wave owns one LDS
// buffer of packed fp32 blocks that holds A, then T (the diagonal blocks of
// T replace A's once the substitution has read them, the rest once the
// levels are done), so two workgroups of two waves fit per SIMD pair and one
// wave's loads overlap another's inverse.  P goes from the accumulators
// straight to the workspace.
// (The Neumann series needs the power and the running product side by side:
// it keeps a second buffer.)
// FUSE: the decode step's prologue is folded in (raw q, k and gates in; unit
// rows of q, k and beta, g out for the state pass), see CteParams.
template <int DK, int NG, int NH, int ALGO, bool FUSE>
__global__ __launch_bounds__(kWave * NG) void cte_local1_kernel(const CteParams p) {
  using T = __bf16;
  using V8 = Vec8<T>;
  using MM = Mfma<T>;
  constexpr int C = kC, NB = kNB, NS = DK / 32;
  constexpr int kBufs = ALGO == kAlgoNeumann ? 2 : 1;

  __shared__ __align__(16) float sbuf[NG][kBufs][kNTri * kBlkF];
  __shared__ __align__(16) float sGamW[NG][C];
  __shared__ __align__(16) float sBetaW[NG][C];

  const int w = threadIdx.x >> 6;  // value heads hh0 + NH w .. + NH - 1 of the group
  const int lane = threadIdx.x & (kWave - 1), lr = lane & 15, lg = lane >> 4;
  float* const sA = sbuf[w][0];
  float* const sGam = sGamW[w];
  float* const sBeta = sBetaW[w];
  const int S = p.S, Dk = p.Dk, Hk = p.Hk, Hv = p.Hv;
  const int NC = (S + C - 1) / C;
  const int G = Hv / Hk;
  const int lid = xcd_logical_id(blockIdx.x, (int)gridDim.x);
  const int GN = G / (NG * NH);  // value-head groups per key head
  const int hh0 = (lid % GN) * NG * NH;
  const int nseg = p.c_end - p.c_begin;
  const int c = p.c_begin + (lid / GN) % nseg;
  const int bhk = lid / (GN * nseg);
  const int b = bhk / Hk, hk = bhk - b * Hk;
  const int bh0 = b * Hv + hk * G + hh0 + NH * w;  // this wave's first value head
  const int c0 = c * C;
  const uint32_t rem = (uint32_t)(S - c0);

  // K, Q fragments of all four row blocks; g, beta (lane = token)
  const size_t qk0 = ((size_t)(b * Hk + hk) * S + c0) * Dk;  // this chunk's first q / k element
  const auto rK = make_rsrc(static_cast<const T*>(FUSE ? p.k_raw : p.k) + qk0, rem * Dk * 2u);
  const auto rQ = make_rsrc(static_cast<const T*>(FUSE ? p.q_raw : p.q) + qk0, rem * Dk * 2u);
  V8 kf[NB][NS], qf[NB][NS];
  uint32_t foff[NS];  // byte offset of fragment s in row block 0 (row stride Dk * 2)
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int k8 = 32 * s + 8 * lg;
    foff[s] = k8 < Dk ? (uint32_t)(lr * Dk + k8) * 2u : kOOB;
  }
#pragma unroll
  for (int rb = 0; rb < NB; ++rb)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t off = foff[s] == kOOB ? kOOB : foff[s] + (uint32_t)(16 * rb * Dk) * 2u;
      kf[rb][s] = V8::bload(rK, off);
      qf[rb][s] = V8::bload(rQ, off);
    }
  float gln[NH], ben[NH];
  if constexpr (FUSE) {
    // Each row made unit length: lane (lr, lg) holds 8 columns of row
    // 16 rb + lr in each of its NS fragments, the rest of the row is in lanes
    // lr + 16 j.  One wave per key head and chunk writes the rows for the
    // state pass.
    auto unit_rows = [&](V8* f) {
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += f[s].get(e) * f[s].get(e);
      ss += __shfl_xor(ss, 16, kWave);
      ss += __shfl_xor(ss, 32, kWave);
      const float inv = 1.0f / sqrtf(ss + kL2Eps);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        bf16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = f2bf(f[s].get(e) * inv);
        f[s].u = __builtin_bit_cast(uint4, y);
      }
    };
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      unit_rows(kf[rb]);
      unit_rows(qf[rb]);
    }
    // The unit rows may be written over the raw ones (in place): every wave
    // of the workgroup has used its raw rows (the loads have returned) before
    // wave 0 writes.
    if constexpr (NG > 1) __syncthreads();
    if (hh0 == 0 && w == 0) {
      const auto wK = make_rsrc(static_cast<T*>(p.kn) + qk0, rem * Dk * 2u);
      const auto wQ = make_rsrc(static_cast<T*>(p.qn) + qk0, rem * Dk * 2u);
#pragma unroll
      for (int rb = 0; rb < NB; ++rb)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint32_t off = foff[s] == kOOB ? kOOB : foff[s] + (uint32_t)(16 * rb * Dk) * 2u;
          kf[rb][s].bstore(wK, off);
          qf[rb][s].bstore(wQ, off);
        }
    }
    // beta = sigmoid(b), g = -exp(A_log[h]) softplus(a + dt_bias[h]) for the
    // token of this lane; zero past the sequence end
    const bool tv = c0 + lane < S;
#pragma unroll
    for (int n = 0; n < NH; ++n) {
      const size_t row = (size_t)(bh0 + n) * S + c0;
      const int h = (bh0 + n) % Hv;
      const float bb = buf_load_f32(make_rsrc(p.b_raw + row, rem * 4u), (uint32_t)lane * 4u);
      const float aa = buf_load_f32(make_rsrc(p.a_raw + row, rem * 4u), (uint32_t)lane * 4u);
      gln[n] = tv ? -expf(p.A_log[h]) * softplusf_(aa + p.dt_bias[h]) : 0.f;
      ben[n] = tv ? sigmoidf_(bb) : 0.f;
      if (tv) {
        p.g_out[row + lane] = gln[n];
        p.beta_out[row + lane] = ben[n];
      }
    }
  } else {
#pragma unroll
    for (int n = 0; n < NH; ++n) {
      gln[n] = buf_load_f32(make_rsrc(p.g + (size_t)(bh0 + n) * S + c0, rem * 4u), (uint32_t)lane * 4u);
      ben[n] = buf_load_f32(make_rsrc(p.beta + (size_t)(bh0 + n) * S + c0, rem * 4u), (uint32_t)lane * 4u);
    }
  }

  // raw products of the lower blocks, transposed: lane holds row 16 i + lr,
  // columns 16 j + 4 lg .. +3 of K K^T and Q K^T
  f4 kkr[kNTri], qkr[kNTri];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j <= i; ++j) {
      f4 kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        kk = MM::mma(kf[j][s], kf[i][s], kk);
        qk = MM::mma(kf[j][s], qf[i][s], qk);
      }
      kkr[tri(i, j)] = kk;
      qkr[tri(i, j)] = qk;
    }
  const float scale = p.scale;

#pragma unroll
  for (int n = 0; n < NH; ++n) {
  const int bh = bh0 + n;
  if (n > 0) wave_lds_sync();  // the previous head's reads of the buffer are done
  sGam[lane] = wave_inclusive_scan_dpp(gln[n]);
  sBeta[lane] = ben[n];
  wave_lds_sync();

  // A (packed, fp32) and P (registers).  Below the diagonal block every
  // column precedes every row, so only the diagonal blocks are masked.
  f4 pacc[kNTri];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const float gt = sGam[16 * i + lr], bt = sBeta[16 * i + lr];
    const int t = 16 * i + lr;
#pragma unroll
    for (int j = 0; j <= i; ++j) {
      const f4 kk = kkr[tri(i, j)], qk = qkr[tri(i, j)];
      const float4 gs = *reinterpret_cast<const float4*>(&sGam[16 * j + 4 * lg]);
      const float gsv[4] = {gs.x, gs.y, gs.z, gs.w};
      float a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sc = 16 * j + 4 * lg + r;
        const float e = __expf(gt - gsv[r]);
        a[r] = (j < i || sc < t) ? bt * kk[r] * e : 0.f;
        pacc[tri(i, j)][r] = (j < i || sc <= t) ? scale * qk[r] * e : 0.f;
      }
      *reinterpret_cast<float4*>(&sA[tri(i, j) * kBlkF + lr * kLB + 4 * lg]) = make_float4(a[0], a[1], a[2], a[3]);
    }
  }
  wave_lds_sync();

  // T, left in sA (row form) in both branches
  if constexpr (ALGO == kAlgoNeumann) {
    // T = (I - A)(I + A^2)(I + A^4) ... (I + A^32): with Pw the running power
    // (-A)^(2^j), Pw <- Pw Pw and T <- T + T Pw, five times.  Every factor is
    // lower block-triangular, so block (i, j) of a product sums m = j..i.
    // Pw and T live in accumulator form (lane: rows 4 lg + r, column lr) and,
    // as the first operand of the next products, in row form: T in sA, Pw in
    // the second buffer.
    float* const sPw = sbuf[w][kBufs - 1];
    f4 pw[kNTri], tb[kNTri];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j <= i; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = sA[tri(i, j) * kBlkF + (4 * lg + r) * kLB + lr];
          pw[tri(i, j)][r] = -a;
          tb[tri(i, j)][r] = (i == j && 4 * lg + r == lr) ? 1.f - a : -a;
        }
    wave_lds_sync();
    auto put = [&](float* dst, const f4* src) {
#pragma unroll
      for (int q = 0; q < kNTri; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[q * kBlkF + (4 * lg + r) * kLB + lr] = src[q][r];
    };
    put(sPw, pw);
    put(sA, tb);
    wave_lds_sync();
#pragma unroll 1
    for (int step = 1; step < 6; ++step) {
      f4 np[kNTri];
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j) {
          f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = j; m <= i; ++m)
            z = mfma4_f32(*reinterpret_cast<const float4*>(&sPw[tri(i, m) * kBlkF + lr * kLB + 4 * lg]), pw[tri(m, j)], z);
          np[tri(i, j)] = z;
        }
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j <= i; ++j) {
          f4 z = tb[tri(i, j)];
#pragma unroll
          for (int m = j; m <= i; ++m)
            z = mfma4_f32(*reinterpret_cast<const float4*>(&sA[tri(i, m) * kBlkF + lr * kLB + 4 * lg]), np[tri(m, j)], z);
          tb[tri(i, j)] = z;
        }
#pragma unroll
      for (int q = 0; q < kNTri; ++q) pw[q] = np[q];
      wave_lds_sync();
      put(sPw, pw);
      put(sA, tb);
      wave_lds_sync();
    }
  } else {
    // diagonal blocks of T: lane = (block, column), forward substitution; T's
    // diagonal blocks then replace A's, which nothing reads again
    {
      const int blk = lane >> 4, j = lane & 15;
      float* const Ab = sA + tri(blk, blk) * kBlkF;
      float tc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) tc[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        float row[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 v = *reinterpret_cast<const float4*>(Ab + i * kLB + 4 * q);
          row[4 * q] = v.x; row[4 * q + 1] = v.y; row[4 * q + 2] = v.z; row[4 * q + 3] = v.w;
        }
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) acc += row[m] * tc[m];
        if (i > j) tc[i] = -acc;
      }
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < 16; ++i) Ab[i * kLB + j] = tc[i];
    }
    wave_lds_sync();

    // off-diagonal blocks level by level, T_ij = -T_ii sum_m A_im T_mj, in
    // the accumulator layout (lane: rows 4 lg + r, column lr); A_im (m < i)
    // and T_ii are both in sA now
    f4 tb[kNTri];
#pragma unroll
    for (int d = 0; d < NB; ++d)
#pragma unroll
      for (int r = 0; r < 4; ++r) tb[tri(d, d)][r] = sA[tri(d, d) * kBlkF + (4 * lg + r) * kLB + lr];
#pragma unroll
    for (int d = 1; d < NB; ++d) {
#pragma unroll
      for (int j = 0; j + d < NB; ++j) {
        const int i = j + d;
        f4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = j; m < i; ++m)
          z = mfma4_f32(*reinterpret_cast<const float4*>(&sA[tri(i, m) * kBlkF + lr * kLB + 4 * lg]), tb[tri(m, j)], z);
        const f4 tz = mfma4_f32(*reinterpret_cast<const float4*>(&sA[tri(i, i) * kBlkF + lr * kLB + 4 * lg]), z,
                                f4{0.f, 0.f, 0.f, 0.f});
        tb[tri(i, j)] = -tz;
      }
    }
    wave_lds_sync();  // every read of A's off-diagonal blocks is done
#pragma unroll
    for (int d = 1; d < NB; ++d)
#pragma unroll
      for (int j = 0; j + d < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) sA[tri(j + d, j) * kBlkF + (4 * lg + r) * kLB + lr] = tb[tri(j + d, j)][r];
  }
  wave_lds_sync();

  // lower blocks of T -> workspace in bf16, packed (item it = 32 block + 2
  // row + half holds 8 elements: the state pass reads them in this order, 1 KB
  // per instruction), 16-byte stores; then P, packed the same way after T
  T* Tg = ws_chunk<T>(p.ws, bh, NC, c);
  T* Pg = Tg + kTriItems * 8;
#pragma unroll
  for (int q = 0; q < kNTri * 32 / kWave; ++q) {
    const int it = lane + kWave * q, blk = it / 32, row = (it % 32) / 2, half = it % 2;
    const float* src = sA + blk * kBlkF + row * kLB + 8 * half;
    const float4 x0 = *reinterpret_cast<const float4*>(src);
    const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
    bf16x8 f;
    f[0] = f2bf(x0.x); f[1] = f2bf(x0.y); f[2] = f2bf(x0.z); f[3] = f2bf(x0.w);
    f[4] = f2bf(x1.x); f[5] = f2bf(x1.y); f[6] = f2bf(x1.z); f[7] = f2bf(x1.w);
    *reinterpret_cast<uint4*>(Tg + (size_t)it * 8) = __builtin_bit_cast(uint4, f);
  }
  // P straight from the accumulators: lane (lr, lg) of block b holds row
  // lr, columns 4 lg .. + 3, i.e. half lg / 2 of item 32 b + 2 lr + lg / 2,
  // so a block is one contiguous 512-byte store
#pragma unroll
  for (int b = 0; b < kNTri; ++b) {
    bf16x4 y;
    y[0] = f2bf(pacc[b][0]); y[1] = f2bf(pacc[b][1]); y[2] = f2bf(pacc[b][2]); y[3] = f2bf(pacc[b][3]);
    *reinterpret_cast<bf16x4*>(Pg + (size_t)(32 * b + 2 * lr) * 8 + 4 * lg) = y;
  }
  }  // value heads of this wave
}

// ===========================================================================
// kernel 2: the sequential state pass
// ===========================================================================
// Per chunk c, three phases separated by workgroup barriers (wave w owns the
// 16-token row block w of the chunk and the state blocks hb = w + 4j):
//   B  store the outputs of chunk c-1; K H -> X = beta (V - Gam K H) -> LDS;
//      Q H -> output accumulators
//   C  U = T X -> LDS twice: as is (for P U) and scaled by d_t =
//      exp(gam_C - gam_t) (for the state update, K~^T U = K^T (d U))
//   D  O = scale Gam Q H + P U -> LDS (stored in the next B);
//      H' = Gam_C H + K^T (d U) in the accumulators, bf16 copy -> LDS;
//      then chunk c+1 is staged from the registers it was prefetched into
//      during chunk c-1 (K into the other half of a double buffer, V, g scan,
//      beta into LDS; Q, T, P fragments stay in registers) and chunk c+2 is
//      prefetched.  The K^T operand of the state update is read from the
//      token-major K tile with transposed LDS reads.
// Every load and store goes through a buffer descriptor rebuilt per chunk
// (scalar work) whose base is the chunk start and whose range ends at the
// sequence end: per-thread offsets are loop invariant, and the hardware range
// check zero-fills (or drops) the rows past a ragged end.
template <typename T, int DK, int DVT>
__global__ __launch_bounds__(kThreads) void cte_state_kernel(const CteParams p) {
  using V8 = Vec8<T>;
  using MM = Mfma<T>;
  constexpr int C = kC;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int LDK = DK + PAD;
  constexpr int LDC = C + PAD;
  constexpr int LDV = DVT + PAD;
  constexpr int NKB = DK / 16, NVB = DVT / 16;
  constexpr int KG = DK / 32;                         // 32-column groups of K
  constexpr int HPW = NKB * NVB / kWaves;             // state blocks per wave
  constexpr int NKI = (C / 2) * (DK / 8) / kThreads;  // K token-pair items per thread
  constexpr int NVT = C * (DVT / 8);                  // V / O items
  constexpr int NV = (NVT + kThreads - 1) / kThreads;
  constexpr int NQ = DK / 32;                         // Q fragments per lane
  constexpr int KSTEPS = C / 32;
  constexpr uint32_t ES = sizeof(T);
  static_assert(NKB * NVB % kWaves == 0 && NKI * kThreads == (C / 2) * (DK / 8), "tile split");

  __shared__ __align__(16) T sKb[2][C * LDK];
  __shared__ __align__(16) T sV[C * LDV];
  __shared__ __align__(16) T sHt[DVT * LDK];
  __shared__ __align__(16) T sXt[DVT * LDC];
  __shared__ __align__(16) T sUt[DVT * LDC];
  __shared__ __align__(16) T sUd[DVT * LDC];
  __shared__ __align__(16) T sO[C * LDV];
  __shared__ float sGam[C];
  __shared__ float sBeta[C];

  const int tid = threadIdx.x, w = tid / kWave, lane = tid & (kWave - 1);
  const int lr = lane & 15, lg = lane >> 4;
  const int S = p.S, Dk = p.Dk, Dv = p.Dv, Hv = p.Hv;
  const int NC = (S + C - 1) / C;
  const int ntiles = (Dv + DVT - 1) / DVT;
  // logical id = (b * Hv + h) * ntiles + tile: the tiles of a head and the
  // value heads of a key head are neighbours (and so share an XCD's L2)
  const int lid = xcd_logical_id(blockIdx.x, (int)gridDim.x);
  const int tile = lid % ntiles;
  const int bh = lid / ntiles;
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

  // state tile -> accumulators; wave w owns blocks hb = w + 4j (kb = hb / NVB, vb = hb % NVB)
  f4 hacc[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int hb = w + kWaves * j, kb = hb / NVB, vb = hb % NVB;
    const int cc = col0 + 16 * vb + lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = 16 * kb + 4 * lg + r;
      hacc[j][r] = (p.has_initial_state && kk < Dk && cc < Dv) ? stg[(size_t)kk * Dv + cc] : 0.f;
    }
    store4<T>(sHt + (16 * vb + lr) * LDK + 16 * kb + 4 * lg, hacc[j][0], hacc[j][1], hacc[j][2], hacc[j][3]);
  }


  // ---- loop-invariant per-thread offsets (bytes from the chunk start)
  // K: item i = rows t0, t0+1 (t0 = 2 tp) at columns c8..c8+7
  int kt0[NKI], kc8[NKI];
  uint32_t vo_k[NKI];
#pragma unroll
  for (int i = 0; i < NKI; ++i) {
    const int rest = w + kWaves * i;
    kt0[i] = 2 * (lr + 16 * (rest / KG));
    kc8[i] = 8 * lg + 32 * (rest % KG);
    vo_k[i] = kc8[i] < Dk ? (uint32_t)(kt0[i] * Dk + kc8[i]) * ES : kOOB;
  }
  // T and P are only A operands of this wave's 16 rows: their fragments go
  // straight into registers; upper 16x16 blocks read as zero.  The compiler
  // may turn the s < nks guards below into EXEC masks, under which an MFMA
  // still executes: the fragments past a guard are those zeros, so such a
  // product adds nothing.
  const int nks = (16 * (w + 1) + 31) / 32;           // k-steps touching lower blocks
  uint32_t vo_t[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const int k8 = 32 * s + 8 * lg;
    vo_t[s] = (s < nks && (k8 >> 4) <= w) ? (uint32_t)((16 * w + lr) * C + k8) * ES : kOOB;
  }
  uint32_t vo_v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int it = tid + kThreads * i, t = it / (DVT / 8), c8 = (it % (DVT / 8)) * 8;
    vo_v[i] = (it < NVT && col0 + c8 < Dv) ? (uint32_t)(t * Dv + col0 + c8) * ES : kOOB;
  }
  uint32_t vo_q[NQ];
#pragma unroll
  for (int s = 0; s < NQ; ++s) {
    const int k8 = 32 * s + 8 * lg;
    vo_q[s] = k8 < Dk ? (uint32_t)((16 * w + lr) * Dk + k8) * ES : kOOB;
  }

  // ---- prefetch registers (one chunk)
  V8 pk0[NKI], pk1[NKI], ptf[KSTEPS], ppf[KSTEPS], pv[NV], pq[NQ];
  float pg = 0.f, pb = 0.f;
  auto prefetch = [&](int c) {
    const int c0 = c * C;
    const uint32_t rem = (uint32_t)(S - c0);
    const auto rK = make_rsrc(kg + (size_t)c0 * Dk, rem * Dk * ES);
    const auto rQ = make_rsrc(qg + (size_t)c0 * Dk, rem * Dk * ES);
    const auto rV = make_rsrc(vg + (size_t)c0 * Dv, rem * Dv * ES);
    const auto rW = make_rsrc(ws_chunk<T>(p.ws, bh, NC, c), 2 * C * C * ES);
    const auto rG = make_rsrc(gg + c0, rem * 4);
    const auto rB = make_rsrc(bg + c0, rem * 4);
#pragma unroll
    for (int i = 0; i < NKI; ++i) {
      pk0[i] = V8::bload(rK, vo_k[i]);
      pk1[i] = V8::bload(rK, vo_k[i] + (uint32_t)Dk * ES);
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      ptf[s] = V8::bload(rW, vo_t[s]);
      ppf[s] = V8::bload(rW, vo_t[s] + (uint32_t)(C * C) * ES);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) pv[i] = V8::bload(rV, vo_v[i]);
#pragma unroll
    for (int s = 0; s < NQ; ++s) pq[s] = V8::bload(rQ, vo_q[s]);
    pg = buf_load_f32(rG, (uint32_t)lane * 4u);
    pb = buf_load_f32(rB, (uint32_t)lane * 4u);
  };

  // ---- stage the prefetched chunk c into LDS (K[c & 1], V, g scan, beta)
  //      and registers (Q, T, P fragments)
  V8 qf[NQ], tf[KSTEPS], pf[KSTEPS];
  auto stage = [&](int c) {
    T* sK = sKb[c & 1];
#pragma unroll
    for (int i = 0; i < NKI; ++i) {
      const int t0 = kt0[i], c8 = kc8[i];
      pk0[i].store(sK + t0 * LDK + c8);
      pk1[i].store(sK + (t0 + 1) * LDK + c8);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int it = tid + kThreads * i, t = it / (DVT / 8), c8 = (it % (DVT / 8)) * 8;
      if (it < NVT) pv[i].store(sV + t * LDV + c8);
    }
#pragma unroll
    for (int s = 0; s < NQ; ++s) qf[s] = pq[s];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      tf[s] = ptf[s];
      pf[s] = ppf[s];
    }
    if (w == 0) {
      sGam[lane] = wave_inclusive_scan_dpp(pg);
      sBeta[lane] = pb;
    }
  };

  // outputs of chunk c sit in sO from its phase D until the next phase B
  auto flush_out = [&](int c) {
    const int c0 = c * C;
    const auto rO = make_rsrc(og + (size_t)c0 * Dv, (uint32_t)(S - c0) * Dv * ES);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int it = tid + kThreads * i, t = it / (DVT / 8), c8 = (it % (DVT / 8)) * 8;
      if (it < NVT) V8::load(sO + t * LDV + c8).bstore(rO, vo_v[i]);
    }
  };

  if (NC > 0) {
    prefetch(0);
    stage(0);
    if (NC > 1) prefetch(1);
  }
  __syncthreads();

  for (int c = 0; c < NC; ++c) {
    // ------------------------------------------------------------------- B
    if (c > 0) flush_out(c - 1);
    f4 oacc[NVB];
    float GC, dt[4];
    {
      float Gt[4], bt[4];
      const float gC = sGam[C - 1];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * w + 4 * lg + r;
        const float gt = sGam[t];
        Gt[r] = __expf(gt);
        dt[r] = __expf(gC - gt);
        bt[r] = sBeta[t];
      }
      GC = __expf(gC);
      const T* sK = sKb[c & 1];
      V8 kf[NQ];
#pragma unroll
      for (int s = 0; s < NQ; ++s) kf[s] = V8::load(sK + (16 * w + lr) * LDK + 32 * s + 8 * lg);
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f4 kh = {0.f, 0.f, 0.f, 0.f}, qh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
          const V8 hb = V8::load(sHt + (16 * vb + lr) * LDK + 32 * s + 8 * lg);
          kh = MM::mma(kf[s], hb, kh);
          qh = MM::mma(qf[s], hb, qh);
        }
        const int cc = 16 * vb + lr;
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * w + 4 * lg + r;
          x[r] = bt[r] * (to_f32<T>(sV[t * LDV + cc]) - Gt[r] * kh[r]);
          oacc[vb][r] = scale * Gt[r] * qh[r];
        }
        store4<T>(sXt + cc * LDC + 16 * w + 4 * lg, x[0], x[1], x[2], x[3]);
      }
    }
    __syncthreads();

    // ------------------------------------------------------------------- C
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      f4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        if (s < nks) u = MM::mma(tf[s], V8::load(sXt + (16 * vb + lr) * LDC + 32 * s + 8 * lg), u);
      const int off = (16 * vb + lr) * LDC + 16 * w + 4 * lg;
      store4<T>(sUt + off, u[0], u[1], u[2], u[3]);
      store4<T>(sUd + off, dt[0] * u[0], dt[1] * u[1], dt[2] * u[2], dt[3] * u[3]);
    }
    __syncthreads();

    // ------------------------------------------------------------------- D
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      f4 o = oacc[vb];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        if (s < nks) o = MM::mma(pf[s], V8::load(sUt + (16 * vb + lr) * LDC + 32 * s + 8 * lg), o);
#pragma unroll
      for (int r = 0; r < 4; ++r) sO[(16 * w + 4 * lg + r) * LDV + 16 * vb + lr] = from_f32<T>(o[r]);
    }
    {
      const T* sK = sKb[c & 1];
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const int hb = w + kWaves * j, kb = hb / NVB, vb = hb % NVB;
        f4 hc = hacc[j];
        hc[0] *= GC; hc[1] *= GC; hc[2] *= GC; hc[3] *= GC;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
          hc = MM::mma(lds_tr_frag(sK, LDK, 32 * s, 16 * kb, lane),
                       V8::load(sUd + (16 * vb + lr) * LDC + 32 * s + 8 * lg), hc);
        hacc[j] = hc;
        store4<T>(sHt + (16 * vb + lr) * LDK + 16 * kb + 4 * lg, hc[0], hc[1], hc[2], hc[3]);
      }
    }
    if (c + 1 < NC) {
      stage(c + 1);
      if (c + 2 < NC) prefetch(c + 2);
    }
    __syncthreads();
  }
  if (NC > 0) flush_out(NC - 1);

  // final state tile -> HBM (fp32)
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int hb = w + kWaves * j, kb = hb / NVB, vb = hb % NVB;
    const int cc = col0 + 16 * vb + lr;
    if (cc < Dv) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = 16 * kb + 4 * lg + r;
        if (kk < Dk) stg[(size_t)kk * Dv + cc] = hacc[j][r];
      }
    }
  }
}

// ===========================================================================
// kernel 2, bf16: the same sequential pass with four data-mover waves
// ===========================================================================
// Eight waves per workgroup.  Waves 0-3 compute as above (wave w owns row
// block w of the chunk and the state blocks w + 4j, and forms scale Gam Q H
// of its row block next to K H) but issue no global memory instruction inside
// the chunk loop; waves 4-7 move data and finish the outputs.  The movers hold
// two register sets of operands and write each into LDS as soon as the
// compute phase that read the previous copy has passed its barrier, then load
// the same operand of a later chunk, so every load has two chunks of time to
// arrive and the memory pipeline's issue stalls fall on the movers:
//   segment 1  compute: B          movers: K(c+1) -> LDS (K double buffered),
//                                  load K(c+3); outputs of c-1 -> HBM
//   barrier
//   segment 2  compute: C          movers: V, g scan, beta, Q of c+1 -> LDS,
//                                  load those of c+3
//   barrier
//   segment 3  compute: D          movers: O = scale Gam Q H + P U of chunk c
//                                  (P in registers) -> LDS; load P(c+2)
//   barrier
// Only the lower 16x16 blocks of T and P are moved (the packed workspace
// layout).  The compute waves load their own T fragments from it, one
// chunk ahead: each 16-byte piece is used by one wave only, so staging T
// through LDS would only add LDS writes, which run at half the read rate.
// element index of (row t, column k) in a K tile: KSW = XOR-swizzled
// 16-byte granules (granule k/8 of row t lives at granule (k/8) ^ swz(t)),
// else a plain row pitch
__device__ __forceinline__ int k_swz(int t) { return 2 * (t & 3) + ((t >> 2) & 1) + 8 * ((t >> 3) & 1); }
template <bool KSW, int PITCH>
__device__ __forceinline__ int kidx(int t, int k) {
  if constexpr (KSW) return t * PITCH + ((((k >> 3) ^ k_swz(t)) << 3) | (k & 7));
  else return t * PITCH + k;
}
// the transposed fragment of lds_tr_frag, read from a K tile in either layout:
// lane l -> K[r0 + 8 (l / 16) + j][c0 + l % 16], j = 0..7
template <bool KSW, int PITCH>
__device__ __forceinline__ Vec8<__bf16> k_tr_frag(const __bf16* m, int r0, int c0, int lane) {
  const int L = lane & 15, g = lane >> 4;
  const int r = r0 + 8 * g + (L >> 2), c = c0 + 4 * (L & 3);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(m + kidx<KSW, PITCH>(r, c)));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(m + kidx<KSW, PITCH>(r + 4, c)));
  Vec8<__bf16> v;
  v.u = make_uint4((uint16_t)a[0] | (uint32_t)(uint16_t)a[1] << 16, (uint16_t)a[2] | (uint32_t)(uint16_t)a[3] << 16,
                   (uint16_t)b[0] | (uint32_t)(uint16_t)b[1] << 16, (uint16_t)b[2] | (uint32_t)(uint16_t)b[3] << 16);
  return v;
}


template <int DK, int DVT, int MW>
__global__ __launch_bounds__((kWaves + MW) * kWave) void cte_state_ws_kernel(const CteParams p) {
  using T = __bf16;
  using V8 = Vec8<T>;
  using MM = Mfma<T>;
  constexpr int C = kC;
  constexpr int PAD = 8;
  constexpr int LDK = DK + PAD;
  constexpr int LDC = C + PAD;
  constexpr int LDV = DVT + PAD;
  constexpr int NKB = DK / 16, NVB = DVT / 16;
  constexpr int HPW = NKB * NVB / kWaves;                // state blocks per compute wave
  constexpr int NQ = DK / 32;                            // Q / K fragments per lane
  constexpr int KSTEPS = C / 32;
  constexpr int kMovers = MW * kWave;                    // mover threads
  constexpr int kAll = (kWaves + MW) * kWave;
  constexpr int NKQ = C * (DK / 8) / kMovers;            // K or Q items per mover thread
  constexpr int NVT = C * (DVT / 8);                     // V / O items
  constexpr int NVI = (NVT + kMovers - 1) / kMovers;
  constexpr uint32_t ES = 2;
  static_assert(NKB * NVB % kWaves == 0 && NKQ * kMovers == C * (DK / 8), "tile split");
  static_assert(kTriItems % kWave == 0 && NVT % kWave == 0, "T and V items end on a wave boundary");
  static_assert(MW == kWaves, "mover wave mw holds the Q and P rows of row block mw");

  // K tile: for DK = 128 unpadded 256-byte rows whose 16-byte granules are
  // XOR-swizzled by row, so the row-fragment reads (16 rows, one granule), the
  // transposed reads (rows r..r+3 and r+8..r+11, two granules) and the
  // row-contiguous stores each touch 16 distinct bank groups; DK = 64 keeps a
  // padded row.
  constexpr bool KSW = DK == 128;
  constexpr int LDKS = KSW ? DK : LDK;
  __shared__ __align__(16) T sK[2][C * LDKS];
  __shared__ __align__(16) T sQ[C * LDKS];  // Q of the chunk whose outputs the movers form
  __shared__ __align__(16) float sQH[kWaves * NVB * kWave * 4];  // scale Gam Q H, row block w, from wave w
  __shared__ __align__(16) T sV[C * LDV];
  __shared__ __align__(16) T sHt[DVT * LDK];
  __shared__ __align__(16) T sXt[DVT * LDC];
  __shared__ __align__(16) T sUt[DVT * LDC];
  __shared__ __align__(16) T sUd[DVT * LDC];
  __shared__ __align__(16) T sO[C * LDV];
  __shared__ __align__(16) float sEG[C];   // exp(gam_t)
  __shared__ __align__(16) float sED[C];   // exp(gam_C - gam_t)
  __shared__ __align__(16) float sBeta[C];

  const int tid = threadIdx.x, w = tid / kWave, lane = tid & (kWave - 1);
  const int lr = lane & 15, lg = lane >> 4;
  const bool mover = w >= kWaves;
  const int mt = tid - kThreads;  // mover thread index (movers only)
  const int S = p.S, Dk = p.Dk, Dv = p.Dv, Hv = p.Hv;
  const int NC = (S + C - 1) / C;
  const int c_begin = p.c_begin, c_end = p.c_end;  // this launch's chunks
  const int ntiles = (Dv + DVT - 1) / DVT;
  const int lid = xcd_logical_id(blockIdx.x, (int)gridDim.x);
  const int tile = lid % ntiles;
  const int bh = lid / ntiles;
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


  f4 hacc[HPW];
  if (!mover) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int hb = w + kWaves * j, kb = hb / NVB, vb = hb % NVB;
      const int cc = col0 + 16 * vb + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = 16 * kb + 4 * lg + r;
        hacc[j][r] = (p.has_initial_state && kk < Dk && cc < Dv) ? stg[(size_t)kk * Dv + cc] : 0.f;
      }
      store4<T>(sHt + (16 * vb + lr) * LDK + 16 * kb + 4 * lg, hacc[j][0], hacc[j][1], hacc[j][2], hacc[j][3]);
    }
  }


  // ---- mover state: loop-invariant offsets (bytes from the chunk start) and
  //      LDS element offsets of every item, and the in-flight registers
  uint32_t vo_kq[NKQ], vo_v[NVI];
  int lo_kq[NKQ], lo_v[NVI];
#pragma unroll
  for (int i = 0; i < NKQ; ++i) {
    const int it = mt + kMovers * i, t = it / (DK / 8), c8 = 8 * (it % (DK / 8));
    vo_kq[i] = c8 < Dk ? (uint32_t)(t * Dk + c8) * ES : kOOB;
    lo_kq[i] = kidx<KSW, LDKS>(t, c8);
  }
#pragma unroll
  for (int i = 0; i < NVI; ++i) {
    const int it = mt + kMovers * i, t = it / (DVT / 8), c8 = 8 * (it % (DVT / 8));
    vo_v[i] = (it < NVT && col0 + c8 < Dv) ? (uint32_t)(t * Dv + col0 + c8) * ES : kOOB;
    lo_v[i] = it < NVT ? t * LDV + c8 : 0;
  }
  // The outputs are finished by the movers, off the state chain: mover wave
  // mw owns rows 16 mw .. +15.  Q is staged in LDS like K (whole 1 KB runs
  // per load instruction; compute wave mw reads its row fragments for
  // Q H); the P fragments (the MFMA first operand of P U) sit in the mover's
  // registers, loaded from the workspace.
  const int mw = w - kWaves;
  const int mnks = (16 * (mw + 1) + 31) / 32;  // k-steps of P touching lower blocks
  uint32_t vo_pf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    // packed lower blocks: row 16 mw + lr, columns k8 .. + 7 are item
    // 32 tri(mw, k8 / 16) + 2 lr + (k8 / 8) % 2; upper blocks read as zero
    // (so an MFMA past the s < mnks guard, which may compile to an EXEC mask
    // under which it still executes, adds nothing)
    const int k8 = 32 * s + 8 * lg, bj = k8 >> 4;
    vo_pf[s] = (s < mnks && bj <= mw) ? (uint32_t)(32 * (mw * (mw + 1) / 2 + bj) + 2 * lr + ((k8 >> 3) & 1)) * 16u
                                       : kOOB;
  }
  // two register sets: the set of chunk c holds P(c) and the Q, K, V, g,
  // beta, T of chunk c+1, so each load is issued two chunks before its use
  struct Regs {
    V8 K[NKQ], Q[NKQ], Pf[KSTEPS], V[NVI];
    float g, b;
  };
  Regs rs0, rs1;

  // descriptors of chunk c (range 0 past the last chunk: the loads read zero)
  // (chunks outside [c_begin, c_end) read zero and drop their stores)
  auto rem_bytes = [&](int c, int row_elems) -> uint32_t {
    const int r = S - c * C;
    return (c >= c_begin && c < c_end && r > 0) ? (uint32_t)r * (uint32_t)row_elems * ES : 0u;
  };
  auto ld_k = [&](Regs& m, int c) {
    const auto r = make_rsrc(kg + (size_t)c * C * Dk, rem_bytes(c, Dk));
#pragma unroll
    for (int i = 0; i < NKQ; ++i) m.K[i] = V8::bload(r, vo_kq[i]);
  };
  auto ld_p = [&](Regs& m, int c) {
    const auto r = make_rsrc(ws_chunk<T>(p.ws, bh, NC, c) + kTriItems * 8, c < c_end ? (uint32_t)kTriItems * 16u : 0u);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) m.Pf[s] = V8::bload(r, vo_pf[s]);
  };
  auto ld_q = [&](Regs& m, int c) {
    const auto r = make_rsrc(qg + (size_t)c * C * Dk, rem_bytes(c, Dk));
#pragma unroll
    for (int i = 0; i < NKQ; ++i) m.Q[i] = V8::bload(r, vo_kq[i]);
  };
  auto ld_vg = [&](Regs& m, int c) {
    const auto rv = make_rsrc(vg + (size_t)c * C * Dv, rem_bytes(c, Dv));
#pragma unroll
    for (int i = 0; i < NVI; ++i) m.V[i] = V8::bload(rv, vo_v[i]);
    const uint32_t nb = rem_bytes(c, 2);  // fp32 per token
    m.g = buf_load_f32(make_rsrc(gg + c * C, nb), (uint32_t)lane * 4u);
    m.b = buf_load_f32(make_rsrc(bg + c * C, nb), (uint32_t)lane * 4u);
  };
  auto ld_all = [&](Regs& m, int c) {  // P(c) and the rest of chunk c+1
    ld_p(m, c);
    ld_q(m, c + 1);
    ld_k(m, c + 1);
    ld_vg(m, c + 1);
  };
  auto st_k = [&](const Regs& m, int slot) {
#pragma unroll
    for (int i = 0; i < NKQ; ++i) m.K[i].store(sK[slot] + lo_kq[i]);
  };
  auto st_q = [&](const Regs& m) {
#pragma unroll
    for (int i = 0; i < NKQ; ++i) m.Q[i].store(sQ + lo_kq[i]);
  };
  auto st_vg = [&](const Regs& m) {
#pragma unroll
    for (int i = 0; i < NVI; ++i)
      if (mt + kMovers * i < NVT) m.V[i].store(sV + lo_v[i]);
    if (w == kWaves) {
      const float gam = wave_inclusive_scan_dpp(m.g);
      const float gamC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gam), C - 1));
      sEG[lane] = __expf(gam);
      sED[lane] = __expf(gamC - gam);
      sBeta[lane] = m.b;
    }
  };
  // unconditional, so that every path issues the same vector memory
  // instructions (exact waits): items past the tile and chunks outside
  // [0, NC) are dropped by the range check
  auto flush_out = [&](int c) {
    const auto ro = make_rsrc(og + (ptrdiff_t)c * C * Dv, rem_bytes(c, Dv));
#pragma unroll
    for (int i = 0; i < NVI; ++i) V8::load(sO + lo_v[i]).bstore(ro, vo_v[i]);
  };
  auto out_pu = [&](f4* oacc, const V8* pf) {
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      f4 o = oacc[vb];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        if (s < mnks) o = MM::mma(pf[s], V8::load(sUt + (16 * vb + lr) * LDC + 32 * s + 8 * lg), o);
#pragma unroll
      for (int r = 0; r < 4; ++r) sO[(16 * mw + 4 * lg + r) * LDV + 16 * vb + lr] = from_f32<T>(o[r]);
    }
  };
  // one chunk of mover work; m is the set of chunk c, refilled for chunk c+2.
  // The outputs: compute wave w leaves scale Gam Q H of row block w in LDS
  // during B (H of chunk c is in LDS then); mover wave w adds P U once U is
  // there.
  auto mover_chunk = [&](Regs& m, int c) {
    st_k(m, (c + 1) & 1);
    ld_k(m, c + 3);
    flush_out(c - 1);
    __syncthreads();  // end of B
    st_vg(m);
    ld_vg(m, c + 3);
    st_q(m);  // Q(c+1): every mover's Q(c) reads passed the barrier above
    ld_q(m, c + 3);
    __syncthreads();  // end of C
    f4 oacc[NVB];
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) oacc[vb] = *reinterpret_cast<const f4*>(sQH + ((mw * NVB + vb) * kWave + lane) * 4);
    out_pu(oacc, m.Pf);
    ld_p(m, c + 2);
    __syncthreads();  // end of D
  };

  if (mover) {
    // The two roles run separate code from here on, with the same barrier
    // sequence, so the load-to-use waits of each are counted on its own
    // instruction stream.
    __syncthreads();  // initial state staged
    ld_k(rs0, c_begin);
    ld_q(rs0, c_begin);
    ld_vg(rs0, c_begin);
    st_k(rs0, c_begin & 1);
    st_q(rs0);
    st_vg(rs0);
    ld_all(rs0, c_begin);
    ld_all(rs1, c_begin + 1);
    __syncthreads();  // chunk 0 staged
    // an even number of chunks: the padding chunk of an odd count only moves
    // zeros
    for (int c = c_begin; c < c_end; c += 2) {
      mover_chunk(rs0, c);
      mover_chunk(rs1, c + 1);
    }
    flush_out(c_begin + ((c_end - c_begin + 1) & ~1) - 1);
    return;
  }

  __syncthreads();  // initial state staged
  __syncthreads();  // chunk 0 staged
  const int nks = (16 * (w + 1) + 31) / 32;  // k-steps touching lower blocks
  // T fragments of row block w straight from the packed workspace (lane
  // (lr, lg) of k-step s: block j = 2 s + lg / 2, half lg % 2 of row lr, one
  // 512-byte run per block); blocks above the diagonal read zero, as the
  // s < nks guard of U = T X relies on (it may compile to an EXEC mask, under
  // which an MFMA still executes)
  uint32_t vo_tf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const int j = 2 * s + (lg >> 1);
    vo_tf[s] = j <= w ? (uint32_t)(32 * (w * (w + 1) / 2 + j) + 2 * lr + (lg & 1)) * 16u : kOOB;
  }
  auto ld_tf = [&](V8* tf, int c) {
    const auto r = make_rsrc(ws_chunk<T>(p.ws, bh, NC, c), c < c_end ? (uint32_t)kTriItems * 16u : 0u);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) tf[s] = V8::bload(r, vo_tf[s]);
  };
  V8 tfa[KSTEPS], tfb[KSTEPS];
  // A padding chunk past the end (odd NC) is computed like any other: its
  // operands are zeros, exp(gam) = 1 and beta = 0, so the state is unchanged
  // and its outputs fall outside the range check.
  auto compute_chunk = [&](int c, const V8* tf, V8* tfn) {
    const T* sKc = sK[c & 1];
    float GC, dt[4];
    // ------------------------------------------------------------------- B
    {
      // K H -> X = beta (V - Gam K H) -> LDS
      const float4 eg = *reinterpret_cast<const float4*>(&sEG[16 * w + 4 * lg]);
      const float4 ed = *reinterpret_cast<const float4*>(&sED[16 * w + 4 * lg]);
      const float4 be = *reinterpret_cast<const float4*>(&sBeta[16 * w + 4 * lg]);
      const float Gt[4] = {eg.x, eg.y, eg.z, eg.w}, bt[4] = {be.x, be.y, be.z, be.w};
      dt[0] = ed.x; dt[1] = ed.y; dt[2] = ed.z; dt[3] = ed.w;
      GC = sEG[C - 1];
      // and the outputs' first part, scale Gam Q H of row block w (the same
      // state operands), left in LDS for mover wave w
      V8 kf[NQ], qf[NQ];
#pragma unroll
      for (int s = 0; s < NQ; ++s) {
        kf[s] = V8::load(sKc + kidx<KSW, LDKS>(16 * w + lr, 32 * s + 8 * lg));
        qf[s] = V8::load(sQ + kidx<KSW, LDKS>(16 * w + lr, 32 * s + 8 * lg));
      }
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        f4 kh = {0.f, 0.f, 0.f, 0.f}, qh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
          const V8 hf = V8::load(sHt + (16 * vb + lr) * LDK + 32 * s + 8 * lg);
          kh = MM::mma(kf[s], hf, kh);
          qh = MM::mma(qf[s], hf, qh);
        }
        *reinterpret_cast<f4*>(sQH + ((w * NVB + vb) * kWave + lane) * 4) =
            f4{scale * Gt[0] * qh[0], scale * Gt[1] * qh[1], scale * Gt[2] * qh[2], scale * Gt[3] * qh[3]};
        const uint2 v4 = lds_tr4(sV, LDV, 16 * w + 4 * lg, 16 * vb, lane);  // V[16 w + 4 lg + r][16 vb + lr]
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = bt[r] * (bf4_get(v4, r) - Gt[r] * kh[r]);
        store4<T>(sXt + (16 * vb + lr) * LDC + 16 * w + 4 * lg, x[0], x[1], x[2], x[3]);
      }
    }
    __syncthreads();

    // ------------------------------------------------------------------- C
    // U = T X -> LDS as is and scaled by d_t
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      f4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        if (s < nks)
          u = MM::mma(tf[s],
                      V8::load(sXt + (16 * vb + lr) * LDC + 32 * s + 8 * lg), u);
      const int off = (16 * vb + lr) * LDC + 16 * w + 4 * lg;
      store4<T>(sUt + off, u[0], u[1], u[2], u[3]);
      store4<T>(sUd + off, dt[0] * u[0], dt[1] * u[1], dt[2] * u[2], dt[3] * u[3]);
    }
    __syncthreads();

    // ------------------------------------------------------------------- D
    // H' = Gam_C H + K^T (d U)
    ld_tf(tfn, c + 1);
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int hb = w + kWaves * j, kb = hb / NVB, vb = hb % NVB;
      f4 hc = hacc[j];
      hc[0] *= GC; hc[1] *= GC; hc[2] *= GC; hc[3] *= GC;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        hc = MM::mma(k_tr_frag<KSW, LDKS>(sKc, 32 * s, 16 * kb, lane),
                     V8::load(sUd + (16 * vb + lr) * LDC + 32 * s + 8 * lg), hc);
      hacc[j] = hc;
      store4<T>(sHt + (16 * vb + lr) * LDK + 16 * kb + 4 * lg, hc[0], hc[1], hc[2], hc[3]);
    }
    __syncthreads();
  };
  ld_tf(tfa, c_begin);
  for (int c = c_begin; c < c_end; c += 2) {
    compute_chunk(c, tfa, tfb);
    compute_chunk(c + 1, tfb, tfa);
  }


#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int hb = w + kWaves * j, kb = hb / NVB, vb = hb % NVB;
    const int cc = col0 + 16 * vb + lr;
    if (cc < Dv) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = 16 * kb + 4 * lg + r;
        if (kk < Dk) stg[(size_t)kk * Dv + cc] = hacc[j][r];
      }
    }
  }
}

// one workgroup per (chunk, key head, pair of value heads) when the GQA group
// is even, else per (chunk, value head); one wave per value head, or with the
// folded prologue one wave for the pair
constexpr int local1_ng(int Hk, int Hv) { return (Hv / Hk) % 2 == 0 ? 2 : 1; }

template <int DK, int NG, int NH, bool FUSE>
void launch_local1_as(const CteParams& p, long wgs, bool neu, hipStream_t stream) {
  if (neu)
    hipLaunchKernelGGL((cte_local1_kernel<DK, NG, NH, kAlgoNeumann, FUSE>), dim3((unsigned)wgs), dim3(NG * kWave), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((cte_local1_kernel<DK, NG, NH, 0, FUSE>), dim3((unsigned)wgs), dim3(NG * kWave), 0, stream, p);
}

template <int DK, bool FUSE>
hipError_t launch_local1(const CteParams& p, long grid1, hipStream_t stream) {
  const bool neu = p.algo == kAlgoNeumann;
  if (local1_ng(p.Hk, p.Hv) == 1)
    launch_local1_as<DK, 1, 1, FUSE>(p, grid1, neu, stream);
  else if constexpr (FUSE)
    launch_local1_as<DK, 1, 2, FUSE>(p, grid1 / 2, neu, stream);  // one wave rewrites each key head's rows
  else
    launch_local1_as<DK, 2, 1, FUSE>(p, grid1 / 2, neu, stream);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_local(const CteParams& p, hipStream_t stream) {
  const long grid1 = (long)p.B * p.Hv * (p.c_end - p.c_begin);
  if (grid1 == 0) return hipSuccess;
  const bool neu = p.algo == kAlgoNeumann;
  if constexpr (sizeof(T) == 2) {
    if (p.q_raw) return launch_local1<DK, true>(p, grid1, stream);
    return launch_local1<DK, false>(p, grid1, stream);
  } else if (neu)
    hipLaunchKernelGGL((cte_local_kernel<T, DK, kAlgoNeumann>), dim3((unsigned)grid1), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((cte_local_kernel<T, DK, 0>), dim3((unsigned)grid1), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int DK, int DVT>
hipError_t launch_state(const CteParams& p, hipStream_t stream) {
  const long grid2 = (long)p.B * p.Hv * ((p.Dv + DVT - 1) / DVT);
  constexpr int MW = 4;
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((cte_state_ws_kernel<DK, DVT, MW>), dim3((unsigned)grid2), dim3((kWaves + MW) * kWave), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((cte_state_kernel<T, DK, DVT>), dim3((unsigned)grid2), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int DK, int DVT>
hipError_t launch_pair(const CteParams& p0, hipStream_t stream) {
  CteParams p = p0;
  p.c_begin = 0;
  p.c_end = (p.S + kC - 1) / kC;
  const hipError_t e = launch_local<T, DK>(p, stream);
  if (e != hipSuccess) return e;
  return launch_state<T, DK, DVT>(p, stream);
}

// number of compute units on the target (MI355X)
constexpr long kCUs = 256;

// widest state tile that still gives every CU a workgroup
int pick_dvt(const CteParams& p, int max_dvt) {
  const long heads = (long)p.B * p.Hv;
  int dvt = 16;
  for (int cand = max_dvt; cand >= 16; cand /= 2) {
    if (heads * ((p.Dv + cand - 1) / cand) >= kCUs || cand == 16) {
      dvt = cand;
      break;
    }
  }
  while (dvt > 16 && dvt / 2 >= ((p.Dv + 15) / 16) * 16) dvt /= 2;
  return dvt;
}

}  // namespace

size_t cte_workspace_bytes(int B, int Hv, int S, int dtype) {
  const size_t NC = (size_t)((S + kC - 1) / kC);
  return (size_t)B * Hv * NC * 2 * kC * kC * (dtype == 1 ? 2 : 4);
}

bool fused_inplace_ok(int Hk, int Hv) { return Hv / Hk == local1_ng(Hk, Hv); }

hipError_t launch_cte(const CteParams& p, int dtype, hipStream_t stream) {
  if ((long)p.B * p.Hv == 0) return hipSuccess;
  if (p.q_raw && dtype != 1) return hipErrorInvalidValue;  // the folded prologue is bf16 only
  const bool dk64 = p.Dk <= 64;
  if (dtype == 1) {
    const int dvt = pick_dvt(p, 64);
    if (dk64) {
      if (dvt == 64) return launch_pair<__bf16, 64, 64>(p, stream);
      if (dvt == 32) return launch_pair<__bf16, 64, 32>(p, stream);
      return launch_pair<__bf16, 64, 16>(p, stream);
    }
    if (dvt == 64) return launch_pair<__bf16, 128, 64>(p, stream);
    if (dvt == 32) return launch_pair<__bf16, 128, 32>(p, stream);
    return launch_pair<__bf16, 128, 16>(p, stream);
  }
  // fp32 tiles are twice the bytes: with DK = 128 only the 16-column state
  // tile fits the 160 KB of LDS
  if (dk64) {
    if (pick_dvt(p, 32) == 32) return launch_pair<float, 64, 32>(p, stream);
    return launch_pair<float, 64, 16>(p, stream);
  }
  return launch_pair<float, 128, 16>(p, stream);
}

}  // namespace gdn
