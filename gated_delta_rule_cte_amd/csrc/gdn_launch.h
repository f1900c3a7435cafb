// Internal launch interface between the C-ABI layer (gdn_api.cpp) and the
// kernels.  Arguments are validated before any of these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// records a message for gdn_last_error() (printf format) and returns `code`
int set_error(int code, const char* fmt, ...);

// ---------------------------------------------------------------- decode step
struct TkgParams {
  // q/k row of head bh = b * Hv + h starts at base + b * qk_bstride + (h / head_div) * K
  const void* q;
  const void* k;
  long qk_bstride;
  int head_div;
  // v row: v + b * v_bstride + h * V ; z row: z + bh * V
  const void* v;
  long v_bstride;
  const void* z;
  const float* b;
  const float* a;
  const float* A_log;
  const float* dt_bias;
  const float* norm_weight;
  const float* state_in;
  float* state_out;
  void* out;  // bf16 [BH, V]
  int BH, Hv, K, V;
  float rms_eps;
  int bh0;  // first head of a launch (set by launch_tkg)
};
// dtype: 0 fp32, 1 bf16 (q, k, v, z)
hipError_t launch_tkg(const TkgParams& p, int dtype, hipStream_t stream);

// ---------------------------------------------------------------- prefill
struct CteParams {
  const void* q;    // [B, Hk, S, Dk]
  const void* k;
  const void* v;    // [B, Hv, S, Dv]
  const float* g;   // [B, Hv, S]
  const float* beta;
  float* state;     // [B, Hv, Dk, Dv]
  void* out;        // [B, Hv, S, Dv]
  int B, Hk, Hv, S, Dk, Dv;
  int has_initial_state;
  float scale;
  // chunks [c_begin, c_end) of 64 tokens handled by this launch (the
  // workspace layout and the token indexing always span the whole sequence)
  int c_begin, c_end;
  // intra-chunk inverse: 0 blocked forward substitution, 1 Neumann series
  // summed by doubling
  int algo;
  // scratch: per (batch * value head, chunk of 64 tokens) the inverse T and
  // the decayed Q K^T block P, each [64][64] in the compute type
  void* ws;
  // The decode step's prologue folded into the chunk-local kernel (bf16
  // only; NULL q_raw = off).  That kernel then reads raw q_raw, k_raw (the
  // layout of q, k), writes each row made unit length, x / sqrt(sum x^2 +
  // 1e-6) rounded to bf16, to qn, kn, and writes beta = sigmoid(b_raw) and
  // g = -exp(A_log[h]) softplus(a_raw + dt_bias[h]) per token to g_out,
  // beta_out.  q, k, g, beta must point at qn, kn, g_out, beta_out, which
  // the state pass reads.  qn, kn may alias q_raw, k_raw only when one
  // workgroup serves all value heads of a key head (fused_inplace_ok).
  const void* q_raw;
  const void* k_raw;
  const float* b_raw;
  const float* a_raw;
  const float* A_log;
  const float* dt_bias;
  void* qn;
  void* kn;
  float* g_out;
  float* beta_out;
};
// true when the folded prologue may write its unit rows over q_raw, k_raw
bool fused_inplace_ok(int Hk, int Hv);
size_t cte_workspace_bytes(int B, int Hv, int S, int dtype);
hipError_t launch_cte(const CteParams& p, int dtype, hipStream_t stream);

// ------------------------------------- prefill with the decode gates and norm
struct FusedPre {
  const void* q;              // raw [B, Hk, S, Dk], compute type
  const void* k;
  void* qn;                   // unit rows out, same layout and type
  void* kn;
  const float* b;             // [B, Hv, S]
  const float* a;
  const float* A_log;         // [Hv]
  const float* dt_bias;
  float* g;                   // [B, Hv, S] out
  float* beta;
  long rows_qk;               // B * Hk * S
  long tokens_v;              // B * Hv * S
  int S, Hv, Dk;
};
struct FusedPost {
  void* out;                  // [B, Hv, S, Dv] compute type, normalised in place
  const void* z;              // same layout
  const float* norm_weight;   // [Dv]
  long rows;                  // B * Hv * S
  int Dv;
  float rms_eps;
  // when not NULL the result goes here token-major, [B, S, Hv * Dv], and `out`
  // is only read
  void* out_tok;
  int S, Hv;
  // with out_tok: z is token-major too, [B, S, Hv * Dv]
  int z_token_major;
};
hipError_t launch_fused_pre(const FusedPre& f, int dtype, hipStream_t stream);
hipError_t launch_fused_post(const FusedPost& f, int dtype, hipStream_t stream);

// ----------------------------------------------- prefill layer (bf16 only)
// up to four products sharing the left operand, C_p[M, N_p] = A[M, K] B_p[K, N_p]
// (bf16 row-major, N_p % 8 == 0, K % 64 == 0), in one launch
struct GemmParams {
  const void* A;
  int M, K, nprob;
  const void* B[4];
  void* C[4];
  int N[4];
};
hipError_t launch_gemm_bf16(const GemmParams& g, hipStream_t stream);
// C[M, N] = A[M, K] B[K, N], row-major bf16 (leading dimensions K, N, N), fp32
// accumulation, through the vendor GEMM library; hipErrorNotSupported when
// the library cannot take the product (nothing was queued then)
hipError_t gemm_bf16_library(const void* A, const void* B, void* C, int M, int N, int K, hipStream_t stream);
struct NarrowParams {
  const void* A;             // [M, K] bf16, M = B * S token rows
  const void* Wa;            // [K, N] bf16
  const void* Wb;
  float* out_a;              // [B, N, S] fp32 (bf16-rounded values)
  float* out_b;
  int M, N, K, S;
};
hipError_t launch_proj_narrow(const NarrowParams& p, hipStream_t stream);
// the same on MFMA; hipErrorNotSupported (nothing queued) unless N % 16 == 0,
// N <= 64 and K % 32 == 0
hipError_t launch_proj_ab(const NarrowParams& p, hipStream_t stream);
struct ConvSplitParams {
  const void* mixed;         // [B * S, conv_dim] bf16 (the q|k|v projection)
  const float* conv_weight;  // [conv_dim, K_win]
  const void* conv_state;    // [B, conv_dim, K_win] bf16, oldest first
  void* conv_state_out;      // same shape; may be conv_state
  void* q;                   // [B, Hk, S, Dk] bf16
  void* k;
  void* v;                   // [B, Hv, S, Dv] bf16
  // when not NULL (Hv % 8 == 0 only): the a and b projections token-major,
  // [2][B * S, Hv] bf16, moved to a_head / b_head ([B, Hv, S] fp32)
  const void* ab_tok;
  float* a_head;
  float* b_head;
  int B, S, conv_dim, value_dim, key_dim, Hk, Hv, Dk, Dv, K_win;
};
hipError_t launch_conv_split(const ConvSplitParams& p, hipStream_t stream);

// ---------------------------------------------------------------- decode layer
struct BlockParams {
  const void* hidden;      // [B, H] bf16
  const void* W_qkv;       // [H, conv_dim] bf16
  const void* W_z;         // [H, value_dim]
  const void* W_a;         // [H, Hv]
  const void* W_b;         // [H, Hv]
  const float* conv_weight;  // [conv_dim, K_win]
  const void* conv_state_in;  // [B, conv_dim, K_win] bf16
  void* conv_state_out;
  // workspace slices
  void* ws_conv_out;  // [B, conv_dim] bf16
  void* ws_z;         // [B, value_dim] bf16
  float* ws_a;        // [B, Hv]
  float* ws_b;        // [B, Hv]
  int B, H, Hk, Hv, Dk, Dv, K_win;
};
struct BlockWorkspace {
  size_t conv_out, z, a, b, total;  // byte offsets and total size
};
BlockWorkspace block_workspace_layout(int B, int Hk, int Hv, int Dk, int Dv);
hipError_t launch_block_proj(const BlockParams& p, hipStream_t stream);

}  // namespace gdn
