// Prefill counterpart of the decode layer: in_proj over S tokens, the causal
// depthwise conv1d over the sequence, then the prefill with the decode gates
// and output norm.  "GDN Block TKG Kernel API Reference" (summary: in_proj ->
// conv + silu + slide-window state -> q|k|v split -> GQA -> the GDN step)
// read for a whole sequence, with "GDN CTE Kernel API Reference" gdn_cte as
// the recurrence.
//
//   gemm_bf16_kernel     [M, H] x [H, N] on bf16 MFMA 16x16x32 (the q|k|v and
//                        z projections), 128x128 tiles, K step 64 double-
//                        buffered in LDS, weights read with transposing LDS
//                        reads, outputs staged through LDS for 16-byte stores;
//   proj_ab_kernel       the a and b projections (N = Hv, a multiple of 16
//                        up to 64) on MFMA, one workgroup per 16 token rows;
//   proj_narrow_kernel   the same for other Hv, one wave per token;
//   conv_split_kernel    conv + silu over the sequence, split into head-major
//                        q, k, v, rounded to bf16;
//   conv_window_kernel   the conv window after the last token, and a, b moved
//                        to head-major fp32 when they came from the GEMMs.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kGThreads = 256;
constexpr int kGBM = 128, kGBN = 128, kGBK = 64;
constexpr int kGLA = kGBK + 8;  // A tile pitch: 144-byte rows, conflict-free 16-byte fragment reads
constexpr int kGLB = kGBN + 8;  // B tile pitch: 272-byte rows for the transposed reads
constexpr int kGLC = kGBN + 8;  // output staging pitch
constexpr int kGItems = kGBM * kGBK / 8 / kGThreads;  // 16-byte pieces per thread per tile (4)
static_assert(kGBM * kGBK == kGBK * kGBN, "A and B tiles hold the same number of pieces");
static_assert(kGBM * kGLC <= 2 * kGBM * kGLA, "output staging fits the A buffers");

__global__ __launch_bounds__(kGThreads) void gemm_bf16_kernel(const GemmParams g) {
  using V8 = Vec8<__bf16>;
  using MM = Mfma<__bf16>;
  __shared__ __align__(16) __bf16 sA[2 * kGBM * kGLA];
  __shared__ __align__(16) __bf16 sB[2 * kGBK * kGLB];

  const int tid = threadIdx.x, w = tid / kWave, lane = tid & (kWave - 1);
  const int lr = lane & 15, lg = lane >> 4;
  const int M = g.M, K = g.K;
  const int ntm = (M + kGBM - 1) / kGBM;
  // neighbouring logical tiles share an M band (the same activation rows);
  // the products' tiles follow one another
  int lid = xcd_logical_id((int)blockIdx.x, (int)gridDim.x);
  int pi = 0;
  for (; pi + 1 < g.nprob; ++pi) {
    const int nt = ntm * ((g.N[pi] + kGBN - 1) / kGBN);
    if (lid < nt) break;
    lid -= nt;
  }
  const int N = g.N[pi];
  const int ntn = (N + kGBN - 1) / kGBN;
  const int m0 = (lid / ntn) * kGBM, n0 = (lid % ntn) * kGBN;
  const int wm = 64 * (w >> 1), wn = 64 * (w & 1);

  const auto rA = make_rsrc(g.A, (uint32_t)((size_t)M * K * 2));
  const auto rB = make_rsrc(g.B[pi], (uint32_t)((size_t)K * N * 2));
  uint32_t voA[kGItems], voB[kGItems];
  int loA[kGItems], loB[kGItems];
#pragma unroll
  for (int i = 0; i < kGItems; ++i) {
    const int it = tid + kGThreads * i;
    const int ar = it / (kGBK / 8), ak = 8 * (it % (kGBK / 8));
    voA[i] = m0 + ar < M ? (uint32_t)((m0 + ar) * K + ak) * 2u : kOOB;
    loA[i] = ar * kGLA + ak;
    const int bk = it / (kGBN / 8), bn = 8 * (it % (kGBN / 8));
    voB[i] = n0 + bn < N ? (uint32_t)(bk * N + n0 + bn) * 2u : kOOB;
    loB[i] = bk * kGLB + bn;
  }
  V8 ra[kGItems], rb[kGItems];
  auto load = [&](int kt) {
    const uint32_t da = (uint32_t)(kt * kGBK) * 2u, db = (uint32_t)(kt * kGBK) * (uint32_t)N * 2u;
#pragma unroll
    for (int i = 0; i < kGItems; ++i) {
      ra[i] = V8::bload(rA, voA[i] == kOOB ? kOOB : voA[i] + da);
      rb[i] = V8::bload(rB, voB[i] == kOOB ? kOOB : voB[i] + db);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kGItems; ++i) {
      ra[i].store(sA + buf * kGBM * kGLA + loA[i]);
      rb[i].store(sB + buf * kGBK * kGLB + loB[i]);
    }
  };
  f4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int nkt = K / kGBK;
  load(0);
  stage(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load(kt + 1);
    const __bf16* a = sA + buf * kGBM * kGLA;
    const __bf16* bt = sB + buf * kGBK * kGLB;
#pragma unroll
    for (int s = 0; s < kGBK / 32; ++s) {
      V8 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = V8::load(a + (wm + 16 * i + lr) * kGLA + 32 * s + 8 * lg);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = lds_tr_frag(bt, kGLB, 32 * s, wn + 16 * j, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = MM::mma(af[i], bf[j], acc[i][j]);
    }
    if (kt + 1 < nkt) stage(buf ^ 1);
    __syncthreads();
  }
  // outputs: accumulators -> bf16 tile in LDS -> 16-byte row pieces
  __bf16* sc = sA;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[(wm + 16 * i + 4 * lg + r) * kGLC + wn + 16 * j + lr] = f2bf(acc[i][j][r]);
  __syncthreads();
  const auto rC = make_rsrc(g.C[pi], (uint32_t)((size_t)M * N * 2));
#pragma unroll
  for (int i = 0; i < kGBM * kGBN / 8 / kGThreads; ++i) {
    const int it = tid + kGThreads * i, r = it / (kGBN / 8), c8 = 8 * (it % (kGBN / 8));
    const uint32_t off = (m0 + r < M && n0 + c8 < N) ? (uint32_t)((m0 + r) * N + n0 + c8) * 2u : kOOB;
    V8::load(sc + r * kGLC + c8).bstore(rC, off);
  }
}

// out[m, n] = bf16(sum_k A[m, k] W[k, n]) widened to fp32, written head-major
// [B, Hv, S] (m = b S + t, n = head), for the two narrow projections a and b.
// One wave per token row: lane l takes k = l, l + 64, ...; eight columns per
// pass, reduced across the wave with lane shuffles.
__global__ __launch_bounds__(kGThreads) void proj_narrow_kernel(const NarrowParams p) {
  const int wv = (int)((blockIdx.x * kGThreads + threadIdx.x) / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  if (wv >= p.M) return;
  const int b = wv / p.S, t = wv - b * p.S;
  const __bf16* x = static_cast<const __bf16*>(p.A) + (size_t)wv * p.K;
#pragma unroll 1
  for (int which = 0; which < 2; ++which) {
    const __bf16* W = static_cast<const __bf16*>(which ? p.Wb : p.Wa);
    float* out = which ? p.out_b : p.out_a;
#pragma unroll 1
    for (int n0 = 0; n0 < p.N; n0 += 8) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int k = lane; k < p.K; k += kWave) {
        const float xv = bf2f(x[k]);
        const __bf16* wr = W + (size_t)k * p.N + n0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (n0 + j < p.N) acc[j] += xv * bf2f(wr[j]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = acc[j];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
        acc[j] = v;
      }
      if (lane < 8 && n0 + lane < p.N) {
        float v = acc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j)
          if (lane == j) v = acc[j];
        out[((size_t)b * p.N + n0 + lane) * p.S + t] = bf2f(f2bf(v));
      }
    }
  }
}

// The same two narrow projections on bf16 MFMA 16x16x32, for Hv = 16 NBA
// (NBA <= 4): one workgroup per 16 token rows, its eight waves taking the
// k-steps of 32 in turn (wave w: steps w, w + 8, ...).  Per step a wave takes
// the hidden operand (row lr, columns 8 lg .. + 7) straight from global
// memory and copies the step's 32 weight rows of W_a and W_b into its own
// LDS tile, to read them back transposed as MFMA operands (one tile per
// wave: a wave's LDS operations run in order, so the next step's copy
// cannot overtake this step's reads); the pieces of the next kAbAhead - 1
// steps are in flight while one is used.  The eight partial sums meet in
// LDS at the end; wave 0 adds them in a fixed order, rounds to bf16 and
// writes head-major fp32 like proj_narrow_kernel.  Hidden is read once, the
// weights (2 K Hv bf16) once per workgroup, mostly from L2.  At 4096 tokens,
// H = 2048, Hv = 32: 10.0 us against 2 x 11.4 us for the two products in
// the vendor library (four waves, or more steps in flight: 10-12 us).
constexpr int kAbRows = 16;
constexpr int kAbWaves = 8;
constexpr int kAbAhead = 2;  // k-steps in flight per wave
template <int NBA>
__global__ __launch_bounds__(kAbWaves * kWave) void proj_ab_kernel(const NarrowParams p) {
  constexpr int N = 16 * NBA;            // columns per matrix
  constexpr int LW = N + 8;              // weight tile pitch (8-byte aligned rows)
  // a step's 32 rows of one matrix are 32 N / 8 = 64 NBA pieces of 16
  // bytes: lane l takes pieces l + 64 i, i < NBA (row, piece of the row)
  using V8 = Vec8<__bf16>;
  __shared__ __align__(16) __bf16 sW[kAbWaves][2][32 * LW];         // [wave][matrix]
  __shared__ __align__(16) float sR[kAbWaves - 1][2 * NBA][kWave * 4];  // partial sums of waves 1..7
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1), lr = lane & 15, lg = lane >> 4;
  const int m0 = blockIdx.x * kAbRows;
  const int K = p.K, kst = K / 32;
  // steps per wave, padded to a multiple of kAbAhead (steps past K read zeros)
  const int nj = ((kst + kAbWaves - 1) / kAbWaves + kAbAhead - 1) / kAbAhead * kAbAhead;
  const auto rA = make_rsrc(p.A, (uint32_t)((size_t)p.M * K * 2));
  const auto rW0 = make_rsrc(p.Wa, (uint32_t)((size_t)K * N * 2));
  const auto rW1 = make_rsrc(p.Wb, (uint32_t)((size_t)K * N * 2));
  const uint32_t ao = m0 + lr < p.M ? (uint32_t)(((size_t)(m0 + lr) * K + 8 * lg) * 2) : kOOB;
  uint32_t wo[NBA];  // byte offset of the lane's pieces within a step's rows
  int lo[NBA];       // and their place in the weight tile
#pragma unroll
  for (int i = 0; i < NBA; ++i) {
    const int h = lane + kWave * i, r = h / (N / 8), g = h % (N / 8);
    wo[i] = (uint32_t)((r * N + 8 * g) * 2);
    lo[i] = r * LW + 8 * g;
  }
  V8 a[kAbAhead], wv[kAbAhead][2][NBA];
  auto load = [&](int j, int u) {  // this wave's j-th step into ring slot u
    const int ks = w + kAbWaves * j;
    const bool in = ks < kst;
    const uint32_t kb = (uint32_t)(ks * 32);
    a[u] = V8::bload(rA, (ao == kOOB || !in) ? kOOB : ao + kb * 2u);
#pragma unroll
    for (int i = 0; i < NBA; ++i) {
      const uint32_t off = in ? wo[i] + kb * (uint32_t)(N * 2) : kOOB;
      wv[u][0][i] = V8::bload(rW0, off);
      wv[u][1][i] = V8::bload(rW1, off);
    }
  };
  f4 acc[2 * NBA];
#pragma unroll
  for (int j = 0; j < 2 * NBA; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
  __bf16(*tile)[32 * LW] = sW[w];
#pragma unroll
  for (int u = 0; u < kAbAhead; ++u) load(u, u);
  for (int j0 = 0; j0 < nj; j0 += kAbAhead) {
#pragma unroll
    for (int u = 0; u < kAbAhead; ++u) {
#pragma unroll
      for (int mat = 0; mat < 2; ++mat)
#pragma unroll
        for (int i = 0; i < NBA; ++i) wv[u][mat][i].store(tile[mat] + lo[i]);
#pragma unroll
      for (int mat = 0; mat < 2; ++mat)
#pragma unroll
        for (int nb = 0; nb < NBA; ++nb)
          acc[mat * NBA + nb] = Mfma<__bf16>::mma(a[u], lds_tr_frag(tile[mat], LW, 0, 16 * nb, lane), acc[mat * NBA + nb]);
      load(j0 + u + kAbAhead, u);
    }
  }
  if (w > 0) {
#pragma unroll
    for (int j = 0; j < 2 * NBA; ++j) *reinterpret_cast<f4*>(&sR[w - 1][j][lane * 4]) = acc[j];
  }
  __syncthreads();
  if (w != 0) return;
  // lane (lr, lg) holds rows m0 + 4 lg + r, column 16 nb + lr of each matrix
#pragma unroll
  for (int j = 0; j < 2 * NBA; ++j) {
    f4 v = acc[j];
#pragma unroll
    for (int q = 0; q < kAbWaves - 1; ++q) {
      const f4 o = *reinterpret_cast<const f4*>(&sR[q][j][lane * 4]);
      v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
    }
    float* out = j < NBA ? p.out_a : p.out_b;
    const int n = 16 * (j % NBA) + lr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 4 * lg + r;
      if (m < p.M) {
        const int b = m / p.S, t = m - b * p.S;
        out[((size_t)b * N + n) * p.S + t] = bf2f(f2bf(v[r]));
      }
    }
  }
}

// conv + silu over the sequence for 8 channels and a block of kConvTok tokens
// (the window slides in registers, so each input row is read once, plus the
// K_win - 1 rows before the block), then the split: channels [0, key_dim) ->
// q, [key_dim, 2 key_dim) -> k, the rest of conv_dim -> v, all head-major
// bf16.  Eight tokens keep the kernel at 109 VGPRs, four waves per SIMD, so a
// 4096-token sequence is two even rounds of workgroups (sixteen tokens took
// 149 VGPRs, three waves per SIMD and 1.34 rounds: 44.7 against 33.9 us).
constexpr int kConvTok = 8;

__device__ __forceinline__ void unpack8(uint4 u, float* e) {
  const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    e[2 * q] = __uint_as_float(wd[q] << 16);
    e[2 * q + 1] = __uint_as_float(wd[q] & 0xFFFF0000u);
  }
}

template <int KW>
__global__ __launch_bounds__(kGThreads) void conv_split_kernel(const ConvSplitParams p) {
  const int gconv = p.conv_dim / 8;
  const int ntb = (p.S + kConvTok - 1) / kConvTok;
  const long gid = (long)blockIdx.x * kGThreads + threadIdx.x;
  if (gid >= (long)p.B * ntb * gconv) return;
  const int grp = (int)(gid % gconv);
  const long btb = gid / gconv;
  const int b = (int)(btb / ntb), t0 = (int)(btb - (long)b * ntb) * kConvTok;
  const int t1 = min(t0 + kConvTok, p.S);
  {
    const int c = 8 * grp;
    const __bf16* mixed = static_cast<const __bf16*>(p.mixed) + (size_t)b * p.S * p.conv_dim + c;
    const __bf16* st = static_cast<const __bf16*>(p.conv_state) + ((size_t)b * p.conv_dim + c) * p.K_win;
    constexpr int Kw = KW;
    // taps and the window (entries of [state | tokens]); token t uses entries t+1 .. t+Kw
    float wt[8][KW], win[8][KW];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        wt[q][j] = p.conv_weight[(size_t)(c + q) * Kw + j];
        win[q][j] = 0.f;
      }
    // entries t0+1 .. t0+Kw-1 into slots 0 .. Kw-2
#pragma unroll
    for (int j = 0; j < KW - 1; ++j) {
      const int i = t0 + 1 + j;
      float e[8];
      if (i < Kw) {
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = bf2f(st[q * Kw + i]);
      } else {
        unpack8(*reinterpret_cast<const uint4*>(mixed + (size_t)(i - Kw) * p.conv_dim), e);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) win[q][j] = e[q];
    }
    __bf16* dst;
    size_t dstride;
    if (c < p.key_dim) {
      const int h = c / p.Dk, d = c - h * p.Dk;
      dst = static_cast<__bf16*>(p.q) + (((size_t)b * p.Hk + h) * p.S) * p.Dk + d;
      dstride = p.Dk;
    } else if (c < 2 * p.key_dim) {
      const int cc = c - p.key_dim, h = cc / p.Dk, d = cc - h * p.Dk;
      dst = static_cast<__bf16*>(p.k) + (((size_t)b * p.Hk + h) * p.S) * p.Dk + d;
      dstride = p.Dk;
    } else {
      const int cc = c - 2 * p.key_dim, h = cc / p.Dv, d = cc - h * p.Dv;
      dst = static_cast<__bf16*>(p.v) + (((size_t)b * p.Hv + h) * p.S) * p.Dv + d;
      dstride = p.Dv;
    }
    uint4 rows[kConvTok];  // the block's token rows, all requested before the first use
#pragma unroll
    for (int u = 0; u < kConvTok; ++u)
      rows[u] = t0 + u < t1 ? *reinterpret_cast<const uint4*>(mixed + (size_t)(t0 + u) * p.conv_dim)
                            : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < kConvTok; ++u) {
      const int t = t0 + u;
      if (t >= t1) break;
      // newest entry t + Kw is token t
      float e[8];
      unpack8(rows[u], e);
      bf16x8 f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < KW; ++j) acc += wt[q][j] * (j == KW - 1 ? e[q] : win[q][j]);
        f[q] = f2bf(acc * sigmoidf_(acc));
      }
      *reinterpret_cast<uint4*>(dst + (size_t)t * dstride) = __builtin_bit_cast(uint4, f);
      // slide: slots 0 .. Kw-2 take entries t+2 .. t+Kw
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int j = 0; j + 1 < KW - 1; ++j) win[q][j] = win[q][j + 1];
        if constexpr (KW >= 2) win[q][KW - 2] = e[q];  // the newest entry
      }
    }
  }
}

// a and b, [2][B*S, Hv] bf16 token-major -> [B, Hv, S] fp32 (Hv % 8 == 0):
// item id is one token's 8 heads, one 16-byte load; neighbouring items are
// the next heads, then the next token, so a wave reads 1 KB in one piece and
// each of its 8 stores writes 4 runs of 16 tokens
__device__ __forceinline__ void ab_move(const ConvSplitParams& p, long id) {
  const int g8 = p.Hv / 8;
  if (id >= 2L * p.B * p.S * g8) return;
  const int hg = (int)(id % g8);
  const long tok = id / g8;  // (which * B + b) * S + t
  const int which = (int)(tok / ((long)p.B * p.S));
  const long bt = tok - (long)which * p.B * p.S;
  const int b = (int)(bt / p.S), t = (int)(bt - (long)b * p.S);
  const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const __bf16*>(p.ab_tok) + tok * p.Hv + 8 * hg);
  float e[8];
  unpack8(x, e);
  float* out = (which ? p.b_head : p.a_head) + ((size_t)b * p.Hv + 8 * hg) * p.S + t;
#pragma unroll
  for (int q = 0; q < 8; ++q) out[(size_t)q * p.S] = e[q];
}

// the window after the last token: the last K_win entries of [window | tokens]
// (each thread reads its whole row before writing, so it may update in place);
// the threads past B * conv_dim move a and b to head-major
__global__ __launch_bounds__(kGThreads) void conv_window_kernel(const ConvSplitParams p) {
  const long gid = (long)blockIdx.x * kGThreads + threadIdx.x;
  if (gid >= (long)p.B * p.conv_dim) {
    if (p.ab_tok) ab_move(p, gid - (long)p.B * p.conv_dim);
    return;
  }
  const int b = (int)(gid / p.conv_dim), c = (int)(gid - (long)b * p.conv_dim);
  const __bf16* st = static_cast<const __bf16*>(p.conv_state) + gid * p.K_win;
  const __bf16* mixed = static_cast<const __bf16*>(p.mixed);
  __bf16 e[8];
  for (int i = 0; i < p.K_win; ++i) {
    const int idx = p.S + i;
    e[i] = idx < p.K_win ? st[idx] : mixed[((size_t)b * p.S + (idx - p.K_win)) * p.conv_dim + c];
  }
  __bf16* out = static_cast<__bf16*>(p.conv_state_out) + gid * p.K_win;
  for (int i = 0; i < p.K_win; ++i) out[i] = e[i];
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& g, hipStream_t stream) {
  long tiles = 0;
  for (int i = 0; i < g.nprob; ++i) tiles += (long)((g.M + kGBM - 1) / kGBM) * ((g.N[i] + kGBN - 1) / kGBN);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)tiles), dim3(kGThreads), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_proj_ab(const NarrowParams& p, hipStream_t stream) {
  if (p.N % 16 != 0 || p.N > 64 || p.K % 32 != 0) return hipErrorNotSupported;
  if (p.M == 0) return hipSuccess;
  const dim3 grid((unsigned)((p.M + kAbRows - 1) / kAbRows));
  switch (p.N / 16) {
    case 1: hipLaunchKernelGGL((proj_ab_kernel<1>), grid, dim3(kAbWaves * kWave), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((proj_ab_kernel<2>), grid, dim3(kAbWaves * kWave), 0, stream, p); break;
    case 3: hipLaunchKernelGGL((proj_ab_kernel<3>), grid, dim3(kAbWaves * kWave), 0, stream, p); break;
    default: hipLaunchKernelGGL((proj_ab_kernel<4>), grid, dim3(kAbWaves * kWave), 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_proj_narrow(const NarrowParams& p, hipStream_t stream) {
  if (p.M == 0) return hipSuccess;
  const long waves_per_block = kGThreads / kWave;
  hipLaunchKernelGGL(proj_narrow_kernel, dim3((unsigned)((p.M + waves_per_block - 1) / waves_per_block)),
                     dim3(kGThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_conv_split(const ConvSplitParams& p, hipStream_t stream) {
  const long ntb = (p.S + kConvTok - 1) / kConvTok;
  const long n = (long)p.B * ntb * (p.conv_dim / 8);
  if (n > 0) {
    const dim3 grid((unsigned)((n + kGThreads - 1) / kGThreads)), block(kGThreads);
    switch (p.K_win) {
      case 1: hipLaunchKernelGGL(conv_split_kernel<1>, grid, block, 0, stream, p); break;
      case 2: hipLaunchKernelGGL(conv_split_kernel<2>, grid, block, 0, stream, p); break;
      case 3: hipLaunchKernelGGL(conv_split_kernel<3>, grid, block, 0, stream, p); break;
      case 4: hipLaunchKernelGGL(conv_split_kernel<4>, grid, block, 0, stream, p); break;
      case 5: hipLaunchKernelGGL(conv_split_kernel<5>, grid, block, 0, stream, p); break;
      case 6: hipLaunchKernelGGL(conv_split_kernel<6>, grid, block, 0, stream, p); break;
      case 7: hipLaunchKernelGGL(conv_split_kernel<7>, grid, block, 0, stream, p); break;
      default: hipLaunchKernelGGL(conv_split_kernel<8>, grid, block, 0, stream, p); break;
    }
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long nw = (long)p.B * p.conv_dim + (p.ab_tok ? 2L * p.B * p.S * (p.Hv / 8) : 0);
  if (nw > 0)
    hipLaunchKernelGGL(conv_window_kernel, dim3((unsigned)((nw + kGThreads - 1) / kGThreads)), dim3(kGThreads), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace gdn
