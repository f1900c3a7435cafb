// gdn_block_tkg, stage 1: the in_proj matmuls with the depthwise causal conv1d
// decode fused into the epilogue.
// "GDN Block TKG Kernel API Reference", gdn_block_tkg: summary (in_proj
// matmuls -> conv + silu + slide-window state -> split / GQA -> decode step),
// parameters W_in_*, conv_weight, conv_state.
//
// Y[B, N] = hidden[B, H] x [W_in_qkv | W_in_z | W_in_a | W_in_b] is a skinny
// GEMM (M = batch) that streams each weight byte once, so it is bound by HBM
// bandwidth.  One workgroup owns 64 output columns of one weight matrix and
// 64 batch rows and walks H in steps of 128 on bf16 MFMA (16x16x32).  The
// weight tile arrives N-contiguous and is transposed while it is written to
// LDS, so both MFMA operands are read as contiguous 16-byte fragments.
//
// Epilogue per output element (b, n), all results rounded to bf16:
//   q|k|v column c:  window = [state[b,c,1:], y];  act = silu(sum_j w[c,j] window[j])
//                    -> activation buffer, window -> conv_state_out
//   z column:        -> z buffer
//   a / b column:    rounded to bf16, widened to fp32 -> a / b buffers
// Stage 2 is the decode-step kernel reading these buffers with the GQA map.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 64;   // batch rows per workgroup
constexpr int kBN = 64;   // output columns per workgroup
constexpr int kBK = 128;  // hidden-dimension step
constexpr int kLD = kBK + 8;

__global__ __launch_bounds__(kThreads) void block_proj_kernel(const BlockParams p) {
  __shared__ __align__(16) __bf16 sH[kBM * kLD];
  __shared__ __align__(16) __bf16 sWt[kBN * kLD];

  const int tid = threadIdx.x;
  const int w = tid / kWave, lane = tid & (kWave - 1), lr = lane & 15, lg = lane >> 4;
  const int key_dim = p.Hk * p.Dk, value_dim = p.Hv * p.Dv;
  const int conv_dim = 2 * key_dim + value_dim;
  const int nt_qkv = (conv_dim + kBN - 1) / kBN;
  const int nt_z = (value_dim + kBN - 1) / kBN;

  int tile = blockIdx.x, seg, ncols;
  const __bf16* W;
  if (tile < nt_qkv) {
    seg = 0; ncols = conv_dim; W = static_cast<const __bf16*>(p.W_qkv);
  } else if ((tile -= nt_qkv) < nt_z) {
    seg = 1; ncols = value_dim; W = static_cast<const __bf16*>(p.W_z);
  } else {
    tile -= nt_z; seg = 2; ncols = 2 * p.Hv; W = nullptr;
  }
  const int n0 = tile * kBN;
  const int m0 = blockIdx.y * kBM;
  const int H = p.H, B = p.B;
  const __bf16* hid = static_cast<const __bf16*>(p.hidden);

  f4 acc[kBN / 16];
#pragma unroll
  for (int nb = 0; nb < kBN / 16; ++nb) acc[nb] = f4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < H; k0 += kBK) {
    // hidden tile [64 rows][128 k]
    for (int it = tid; it < kBM * (kBK / 8); it += kThreads) {
      const int m = it / (kBK / 8), k8 = (it % (kBK / 8)) * 8;
      const Vec8<__bf16> v = (m0 + m < B) ? Vec8<__bf16>::load(hid + (size_t)(m0 + m) * H + k0 + k8)
                                          : Vec8<__bf16>::zero();
      v.store(sH + m * kLD + k8);
    }
    // weight tile [128 k][64 n] -> transposed [64 n][128 k]
    for (int it = tid; it < kBK * (kBN / 8); it += kThreads) {
      const int k = it / (kBN / 8), n8 = (it % (kBN / 8)) * 8;
      const int n = n0 + n8;
      uint16_t e[8];
      if (seg < 2) {
        if (n < ncols) {
          const uint4 u = *reinterpret_cast<const uint4*>(W + (size_t)(k0 + k) * ncols + n);
          e[0] = u.x & 0xFFFF; e[1] = u.x >> 16; e[2] = u.y & 0xFFFF; e[3] = u.y >> 16;
          e[4] = u.z & 0xFFFF; e[5] = u.z >> 16; e[6] = u.w & 0xFFFF; e[7] = u.w >> 16;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) e[j] = 0;
        }
      } else {
        const uint16_t* Wa = static_cast<const uint16_t*>(p.W_a);
        const uint16_t* Wb = static_cast<const uint16_t*>(p.W_b);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = n + j;
          e[j] = c < p.Hv ? Wa[(size_t)(k0 + k) * p.Hv + c]
                          : (c < 2 * p.Hv ? Wb[(size_t)(k0 + k) * p.Hv + c - p.Hv] : (uint16_t)0);
        }
      }
      uint16_t* dst = reinterpret_cast<uint16_t*>(sWt);
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[(n8 + j) * kLD + k] = e[j];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kBK / 32; ++s) {
      const Vec8<__bf16> a = Vec8<__bf16>::load(sH + (16 * w + lr) * kLD + 32 * s + 8 * lg);
#pragma unroll
      for (int nb = 0; nb < kBN / 16; ++nb) {
        const Vec8<__bf16> bfr = Vec8<__bf16>::load(sWt + (16 * nb + lr) * kLD + 32 * s + 8 * lg);
        acc[nb] = Mfma<__bf16>::mma(a, bfr, acc[nb]);
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds Y[m0 + 16w + 4lg + r][n0 + 16nb + lr]
#pragma unroll
  for (int nb = 0; nb < kBN / 16; ++nb) {
    const int n = n0 + 16 * nb + lr;
    if (n >= ncols) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * w + 4 * lg + r;
      if (m >= B) continue;
      const __bf16 y = f2bf(acc[nb][r]);
      if (seg == 0) {
        const int KW = p.K_win;
        const __bf16* st = static_cast<const __bf16*>(p.conv_state_in) + ((size_t)m * conv_dim + n) * KW;
        __bf16* so = static_cast<__bf16*>(p.conv_state_out) + ((size_t)m * conv_dim + n) * KW;
        const float* cw = p.conv_weight + (size_t)n * KW;
        __bf16 win[8];
        for (int j = 0; j + 1 < KW; ++j) win[j] = st[j + 1];
        win[KW - 1] = y;
        float sum = 0.f;
        for (int j = 0; j < KW; ++j) sum += cw[j] * bf2f(win[j]);
        for (int j = 0; j < KW; ++j) so[j] = win[j];
        static_cast<__bf16*>(p.ws_conv_out)[(size_t)m * conv_dim + n] = f2bf(sum * sigmoidf_(sum));
      } else if (seg == 1) {
        static_cast<__bf16*>(p.ws_z)[(size_t)m * value_dim + n] = y;
      } else if (n < p.Hv) {
        p.ws_a[(size_t)m * p.Hv + n] = bf2f(y);
      } else {
        p.ws_b[(size_t)m * p.Hv + n - p.Hv] = bf2f(y);
      }
    }
  }
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

BlockWorkspace block_workspace_layout(int B, int Hk, int Hv, int Dk, int Dv) {
  BlockWorkspace L;
  const size_t conv_dim = 2 * (size_t)Hk * Dk + (size_t)Hv * Dv;
  L.conv_out = 0;
  L.z = L.conv_out + round256((size_t)B * conv_dim * 2);
  L.a = L.z + round256((size_t)B * Hv * Dv * 2);
  L.b = L.a + round256((size_t)B * Hv * 4);
  L.total = L.b + round256((size_t)B * Hv * 4);
  return L;
}

hipError_t launch_block_proj(const BlockParams& p, hipStream_t stream) {
  const int key_dim = p.Hk * p.Dk, value_dim = p.Hv * p.Dv;
  const int conv_dim = 2 * key_dim + value_dim;
  const int tiles = (conv_dim + kBN - 1) / kBN + (value_dim + kBN - 1) / kBN + (2 * p.Hv + kBN - 1) / kBN;
  const dim3 grid(tiles, (p.B + kBM - 1) / kBM);
  hipLaunchKernelGGL(block_proj_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gdn
