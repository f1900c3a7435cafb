/*
 * libgdn: gated delta-rule (GDN) prefill and decode on AMD Instinct MI355X
 * (gfx950, CDNA4).  Plain C ABI: device pointers, sizes and a HIP stream.
 *
 * The recurrence, per value head h with an fp32 state S in R^{Dk x Dv}
 * (the gated delta rule of Yang, Kautz & Hatamizadeh, "Gated Delta Networks",
 * ICLR 2025, which the pages below name as the computation):
 *
 *     S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * Conventions shared by every entry point
 *   - Every pointer is a device pointer owned by the caller.  The library never
 *     allocates, frees or synchronises; it only launches kernels, in order, on
 *     `stream` (a hipStream_t; NULL is the null stream).  (One exception:
 *     gdn_block_cte runs its projections through hipBLASLt, whose handle is
 *     created on the first call on each device and, with a plan per GEMM
 *     shape, kept until the process ends.)  Launches are asynchronous: a
 *     kernel fault shows up at the caller's next synchronisation.
 *   - Tensors are dense, row-major in the printed index order, and every
 *     pointer must be 16-byte aligned.
 *   - bf16 data is IEEE bfloat16 (upper half of an fp32), passed as void*.
 *   - The return value is GDN_OK (0) or a negative GDN_ERR_* code.  On an error
 *     nothing is launched and no output is touched; gdn_last_error() then
 *     returns a message naming the failed check (per calling thread).
 *   - Input values are not validated (unit-length q/k for the prefill,
 *     beta in (0,1), g < 0 are the caller's contract).
 *   - Calls on one stream are ordered; calls that share an output buffer on
 *     different streams race.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { GDN_F32 = 0, GDN_BF16 = 1 };

/* status codes */
enum {
  GDN_OK = 0,
  GDN_ERR_NULL = -1,        /* a required pointer is NULL                      */
  GDN_ERR_SHAPE = -2,       /* a dimension is out of range or inconsistent     */
  GDN_ERR_DTYPE = -3,       /* unsupported element type                        */
  GDN_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                */
  GDN_ERR_ALIAS = -5,       /* an output overlaps an input it may not overlap  */
  GDN_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required         */
  GDN_ERR_UNSUPPORTED = -7, /* a valid request this library does not implement */
  GDN_ERR_LAUNCH = -8,      /* the HIP runtime rejected a launch               */
  GDN_ERR_DEVICE = -9       /* the current device is not a gfx950 GPU          */
};

/* Intra-chunk inverse T = (I + A)^-1 for gdn_cte ("GDN CTE Kernel API
 * Reference", gdn_cte: parameter algorithm, which names a default method and
 * a Neumann-series alternative).  A is strictly lower triangular, so both
 * methods are exact up to rounding:
 *   GDN_CTE_ALGO_DEFAULT  blocked forward substitution, 16x16 diagonal blocks
 *                         by scalar substitution, off-diagonal blocks level by
 *                         level on fp32 MFMA;
 *   GDN_CTE_ALGO_NEUMANN  the Neumann series summed by doubling,
 *                         T = (I - A)(I + A^2)(I + A^4) ... (I + A^32) for
 *                         64-token chunks (A^64 = 0), ten block-triangular
 *                         fp32 MFMA products per chunk.
 * Both accept every shape and state form gdn_cte accepts; results agree to
 * fp32 rounding of T. */
enum { GDN_CTE_ALGO_DEFAULT = 0, GDN_CTE_ALGO_NEUMANN = 1 };

/* Largest head dimension (Dk, Dv, K, V) any entry point accepts. */
#define GDN_MAX_HEAD_DIM 128

/*
 * gdn_cte - chunk-parallel prefill.
 * "GDN CTE Kernel API Reference", gdn_cte: parameters query, key, value,
 * g_log, beta, scale, recurrent_state; returns; Notes; Dimensions.
 *
 *   query, key   [B, Hk, S, Dk]  token-major, element type `dtype`; each
 *                                token's q and k must have unit L2 norm.
 *   value        [B, Hv, S, Dv]  element type `dtype`.
 *   g_log        [B, Hv, S] fp32 per-token log decay (negative).
 *   beta         [B, Hv, S] fp32 per-token write strength in (0, 1).
 *   scale        query scale (typically 1/sqrt(Dk)), applied on the device.
 *   recurrent_state [B, Hv, Dk, Dv] fp32, in/out.  has_initial_state != 0:
 *                read as the initial state and overwritten in place with the
 *                final state.  has_initial_state == 0: never read (the
 *                recurrence starts from zero) and receives the final state.
 *   out          [B, Hv, S, Dv]  element type `dtype`, head-major, the
 *                un-normalised o_t (no output epilogue).  Must not overlap
 *                any input or recurrent_state.
 *   dtype        GDN_BF16 or GDN_F32: the type of query, key, value and out,
 *                and the MFMA operand type.  Accumulation, the decay cumsum,
 *                the triangular solve and the state are fp32 either way.
 *   algorithm    GDN_CTE_ALGO_DEFAULT or GDN_CTE_ALGO_NEUMANN (see above);
 *                anything else -> GDN_ERR_UNSUPPORTED.
 *   workspace    device scratch of gdn_cte_workspace_size() bytes, 256-byte
 *                aligned, disjoint from every other argument (may be NULL when
 *                that size is 0).  It holds, per value head and chunk of 64
 *                tokens, the intra-chunk inverse (I + A)^-1 and the decayed
 *                query-key block, 2 * 64 * 64 elements of `dtype`; its contents
 *                are undefined after the call.  NULL or too small ->
 *                GDN_ERR_WORKSPACE.
 * Constraints: 1 <= Dk, Dv <= 128 and multiples of 8; Hv % Hk == 0 (value head
 * h reads key/query head h / (Hv / Hk)); S >= 0 with no divisibility
 * requirement (a ragged last chunk is handled) and S * 256 * sizeof(dtype)
 * below 2^31 (about 4M bf16 tokens per call; longer sequences are chained
 * through recurrent_state); B, Hk >= 1.
 */
int gdn_cte(const void* query, const void* key, const void* value,
            const float* g_log, const float* beta, float scale,
            float* recurrent_state, int has_initial_state, void* out,
            int B, int Hk, int Hv, int S, int Dk, int Dv, int dtype,
            int algorithm, void* workspace, size_t workspace_bytes,
            void* stream);

size_t gdn_cte_workspace_size(int B, int Hk, int Hv, int S, int Dk, int Dv,
                              int dtype);

/* Bytes of the fixed device scratch gdn_cte_noalloc uses (per GPU). */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * gdn_cte_noalloc - gdn_cte for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The arguments, results and checks are gdn_cte's; the workspace
 * is instead a fixed array of GDN_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU, held until the process ends.  Nothing is allocated or freed.
 *   - A call whose gdn_cte_workspace_size() exceeds that size returns
 *     GDN_ERR_WORKSPACE (nothing launched); gdn_cte with a caller-owned
 *     workspace has no such limit.
 *   - Every call on a GPU uses that GPU's one array: calls that overlap in
 *     time on one GPU (different streams, or host threads racing to one
 *     stream's queue) race on it and give wrong results.  The array needs no
 *     clearing: each call writes every byte it later reads.
 *   - All of gdn_cte's argument checks run before the first HIP call; on its
 *     first call on a device the entry point then looks up the array's
 *     address on that device (GDN_ERR_DEVICE if it cannot).
 */
int gdn_cte_noalloc(const void* query, const void* key, const void* value,
                    const float* g_log, const float* beta, float scale,
                    float* recurrent_state, int has_initial_state, void* out,
                    int B, int Hk, int Hv, int S, int Dk, int Dv, int dtype,
                    int algorithm, void* stream);

/*
 * gdn_cte_fused - chunked prefill with the decode step's gates and output norm.
 * The steps either side of gdn_cte: "GDN CTE Kernel API Reference", gdn_cte
 * (Notes: q, k must arrive unit-length; return: the output is un-normalised,
 * with no fused epilogue) and "GDN TKG Kernel API Reference", gdn_tkg (summary:
 * l2norm(q, k), beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias), the
 * 1/sqrt(K) query scale, RMSNormGated(out, z)).
 *
 *   q, k         [B, Hk, S, Dk] element type `dtype`, RAW (not normalised).
 *   v, z         [B, Hv, S, Dv] element type `dtype`.
 *   b, a         [B, Hv, S] fp32 raw beta input (pre-sigmoid) and gate input
 *                (pre-softplus), per token of every value head.
 *   A_log, dt_bias [Hv] fp32, indexed by value head.
 *   norm_weight  [Dv] fp32 RMSNormGated weight.
 *   recurrent_state, has_initial_state, algorithm: as for gdn_cte.
 *   out          [B, Hv, S, Dv] element type `dtype`: RMSNormGated(o, z) with
 *                o the un-normalised prefill output rounded to `dtype`.  Must
 *                not overlap any input, recurrent_state or the workspace.
 *   rms_eps      RMSNormGated epsilon (>= 0; the page gives none; 1e-6 typical).
 *   workspace    gdn_cte_fused_workspace_size() bytes, 256-byte aligned and
 *                disjoint from every other argument: the normalised q, k, the
 *                per-token g and beta, and gdn_cte's own workspace.
 * Computes q^ = l2norm(q), k^ = l2norm(k) (epsilon 1e-6 inside the square
 * root, rounded to `dtype`), beta = sigmoid(b), g = -exp(A_log[h])
 * softplus(a + dt_bias[h]), then gdn_cte(q^, k^, v, g, beta, scale = Dk^-1/2),
 * then out = norm_weight * o / sqrt(mean_Dv(o^2) + rms_eps) * silu(z).
 * Constraints: those of gdn_cte.  Errors as for gdn_cte.
 */
int gdn_cte_fused(const void* q, const void* k, const void* v, const float* b,
                  const float* a, const float* A_log, const float* dt_bias,
                  const void* z, const float* norm_weight, float* recurrent_state,
                  int has_initial_state, void* out, int B, int Hk, int Hv, int S,
                  int Dk, int Dv, int dtype, int algorithm, float rms_eps,
                  void* workspace, size_t workspace_bytes, void* stream);

size_t gdn_cte_fused_workspace_size(int B, int Hk, int Hv, int S, int Dk,
                                    int Dv, int dtype);

/*
 * gdn_tkg - fused single-token decode step.
 * "GDN TKG Kernel API Reference", gdn_tkg: summary, parameters, returns,
 * Notes, Dimensions.
 *
 *   q, k         [BH, K] element type `dtype`, RAW (not normalised), already
 *                expanded to value heads.  BH = B * num_v_heads with heads
 *                cycling fastest within a batch.
 *   v, z         [BH, V] element type `dtype`.
 *   b, a         [BH] fp32 raw beta input (pre-sigmoid) and gate input
 *                (pre-softplus).
 *   A_log, dt_bias [num_v_heads] fp32, indexed by bh % num_v_heads.
 *   norm_weight  [V] fp32 RMSNormGated weight (gamma).
 *   state_in     [BH, K, V] fp32 incoming state.
 *   state_out    [BH, K, V] fp32 updated state; may be exactly state_in
 *                (updated in place), must not partially overlap it.
 *   out          [BH, V] bf16: RMSNormGated(o, z).
 *   rms_eps      epsilon of RMSNormGated (the page gives none; 1e-6 typical).
 * The step computes q^ = l2norm(q)/sqrt(K), k^ = l2norm(k) (epsilon 1e-6 inside
 * the square root), beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias),
 * S' = exp(g)(I - beta k^ k^T) S + beta k^ v^T, o = S'^T q^,
 * out = norm_weight * o / sqrt(mean(o^2) + rms_eps) * silu(z).
 * Constraints: 1 <= K, V <= 128, multiples of 8; BH % num_v_heads == 0.
 */
int gdn_tkg(const void* q, const void* k, const void* v, const float* b,
            const float* a, const float* A_log, const float* dt_bias,
            const void* z, const float* norm_weight, const float* state_in,
            float* state_out, void* out, int BH, int num_v_heads, int K, int V,
            int dtype, float rms_eps, void* stream);

/*
 * gdn_block_tkg - fused decode layer: in_proj matmuls -> depthwise causal
 * conv1d decode (conv + silu + window slide) -> split q|k|v and GQA repeat ->
 * the gdn_tkg step -> [B, 1, value_dim].
 * "GDN Block TKG Kernel API Reference", gdn_block_tkg: summary, parameters,
 * returns, Notes, Dimensions.  All of B, H and the head counts come from the
 * arguments.
 *
 *   hidden       [B, 1, H] bf16.
 *   W_in_qkv     [H, conv_dim] bf16 (nn.Linear.weight transposed),
 *                conv_dim = 2 * key_dim + value_dim, columns packed q | k | v.
 *   W_in_z       [H, value_dim] bf16.
 *   W_in_a, W_in_b [H, num_v_heads] bf16.
 *   conv_weight  [conv_dim, K_win] fp32 depthwise taps; tap K_win-1 multiplies
 *                the newest input.
 *   conv_state_in  [B, conv_dim, K_win] bf16 window, oldest first.
 *   A_log, dt_bias [num_v_heads] fp32;  norm_weight [head_v_dim] fp32.
 *   recurrent_state_in [B, num_v_heads, head_k_dim, head_v_dim] fp32.
 *   out          [B, 1, value_dim] bf16.
 *   conv_state_out [B, conv_dim, K_win] bf16: the slid window; may be exactly
 *                conv_state_in.
 *   recurrent_state_out: as recurrent_state_in; may be exactly it.
 *   workspace    gdn_block_tkg_workspace_size() bytes of device scratch for
 *                the activations between the projection and the decode step.
 * Stage boundaries are bf16: the projections and the conv output are rounded
 * to bf16; a and b are widened to fp32 for the gate.
 * Constraints: H % 128 == 0; num_v_heads % num_k_heads == 0; head dims
 * 8..128, multiples of 8; 1 <= K_win <= 8; B >= 0; H * conv_dim * 2,
 * B * H * 2 and B * conv_dim * K_win * 2 below 2^31 bytes.
 */
int gdn_block_tkg(const void* hidden, const void* W_in_qkv, const void* W_in_z,
                  const void* W_in_a, const void* W_in_b,
                  const float* conv_weight, const void* conv_state_in,
                  const float* A_log, const float* dt_bias,
                  const float* norm_weight, const float* recurrent_state_in,
                  void* out, void* conv_state_out, float* recurrent_state_out,
                  int B, int H, int num_k_heads, int num_v_heads,
                  int head_k_dim, int head_v_dim, int K_win, float rms_eps,
                  void* workspace, size_t workspace_bytes, void* stream);

size_t gdn_block_tkg_workspace_size(int B, int H, int num_k_heads,
                                    int num_v_heads, int head_k_dim,
                                    int head_v_dim, int K_win);

/*
 * gdn_block_cte - prefill layer: the decode layer's steps over S tokens.
 * "GDN Block TKG Kernel API Reference", gdn_block_tkg (summary: in_proj ->
 * depthwise causal conv1d with its window -> q|k|v split and GQA repeat -> the
 * GDN step) with the conv run along the sequence and gdn_cte_fused as the step
 * ("GDN CTE Kernel API Reference", gdn_cte).  bf16 only.
 *
 *   hidden       [B, S, H] bf16.
 *   W_in_qkv, W_in_z, W_in_a, W_in_b, conv_weight, A_log, dt_bias,
 *   norm_weight  as for gdn_block_tkg.
 *   conv_state_in [B, conv_dim, K_win] bf16: the window before token 0, oldest
 *                first.  Per channel the inputs extend it; token t convolves
 *                the K_win entries ending at its own input (tap K_win-1).
 *   recurrent_state_in [B, Hv, Dk, Dv] fp32 state before token 0.
 *   out          [B, S, value_dim] bf16: RMSNormGated(o_t, z_t) per token.
 *   conv_state_out [B, conv_dim, K_win] bf16: the window after the last token
 *                (may be exactly conv_state_in).
 *   recurrent_state_out: the state after the last token (may be exactly
 *                recurrent_state_in).
 *   algorithm    intra-chunk inverse, as for gdn_cte.
 *   workspace    gdn_block_cte_workspace_size() bytes, 256-byte aligned,
 *                disjoint from every other argument: the projections, the
 *                head-major conv outputs, gates and the prefill scratch.
 * The q|k|v and z projections are plain GEMMs and run on hipBLASLt (no
 * workspace); a product the library declines runs on this library's own MFMA
 * GEMM.  The narrow a and b projections run on this library's own kernel
 * (num_v_heads a multiple of 16 up to 64; other counts join the GEMMs or,
 * when not a multiple of 8, a per-token kernel).
 * Stage boundaries are bf16 as in gdn_block_tkg; q, k are normalised to unit
 * rows (rounded to bf16) and scaled by Dk^-1/2 inside the prefill.
 * Constraints: those of gdn_block_tkg, plus S >= 0 and every buffer below
 * 2^31 bytes (B*S*H*2, B*S*conv_dim*2, H*conv_dim*2, ...).
 */
int gdn_block_cte(const void* hidden, const void* W_in_qkv, const void* W_in_z,
                  const void* W_in_a, const void* W_in_b,
                  const float* conv_weight, const void* conv_state_in,
                  const float* A_log, const float* dt_bias,
                  const float* norm_weight, const float* recurrent_state_in,
                  void* out, void* conv_state_out, float* recurrent_state_out,
                  int B, int S, int H, int num_k_heads, int num_v_heads,
                  int head_k_dim, int head_v_dim, int K_win, int algorithm,
                  float rms_eps, void* workspace, size_t workspace_bytes,
                  void* stream);

size_t gdn_block_cte_workspace_size(int B, int S, int H, int num_k_heads,
                                    int num_v_heads, int head_k_dim,
                                    int head_v_dim, int K_win);

/* Human-readable name of a status code (static storage). */
const char* gdn_status_string(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char* gdn_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
