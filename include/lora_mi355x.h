/*
 * lora_mi355x.h - C ABI of the fused LoRA MLP / QKV projections on MI355X (gfx950).
 *
 * What is computed (the pages' titles and sections):
 *   - Opake, "Model Patches and Kernels", section "Fused LoRA operations":
 *     the LoRA linear x @ W.T + x @ A @ B * s (opake_lora_w), the fused
 *     Q+K+V call sharing one input (opake_lora_qkv) and the fused
 *     gate+up+down call with the activation (opake_lora_mlp). Fusion applies
 *     only without active LoRA dropout and, for the MLP, without bias.
 *   - Same page, "Activation functions": SwiGLU silu(gate)*up, GeGLU with
 *     the tanh approximation gelu_tanh(gate)*up and the exact (erf) GeGLU
 *     gelu(gate)*up; the backward of the
 *     activation reads the upstream gradient, gate and up and writes the two
 *     input gradients in one pass.
 *   - Same page, "Rotary position embeddings (RoPE)": RoPE applied to Q and K
 *     together, grouped-query attention with different Q and K head counts,
 *     following RoFormer.
 *   - Same page, "Fused linear cross-entropy", key design decisions: frozen
 *     weights get no weight gradient (base W here is frozen: no dW).
 *   - Axolotl, "monkeypatch.lora_kernels", "apply_lora_kernel_patches" note
 *     (no dropout, no bias) and "original_apply_qkv" (hidden_states
 *     [batch, seq, hidden] -> (query, key, value)).
 *
 * Conventions (readings where the pages leave a step open):
 *   - Storage is PEFT / nn.Linear, row-major: W [out, in], A [r, in], B [out, r],
 *     so L(Z) = Z W^T + s (Z A^T) B^T and T = Z A^T is [N, r].
 *   - Tokens are rows n = b*seq + s; X is [n_tokens, hidden] row-major.
 *   - RoPE pairs column j with j + head_dim/2 of a head (half split), angle
 *     = s * theta^(-2j/head_dim) evaluated in double precision, s = n mod seq.
 *   - Q is [batch, n_q, seq, head_dim], K and V are [batch, n_kv, seq, head_dim].
 *   - n_tokens = 0 (batch = 0 for QKV) is a valid call: the forward writes
 *     nothing, the backward writes dA = 0 and dB = 0 (empty sums).  Per-token
 *     tensors (X, Y, G, U, T, Q, K, V, their gradients, Pn, rinv) may then be
 *     NULL; weights, adapters and dA / dB may not.
 *   - One dtype per call (LORA_F32 or LORA_BF16) for X, W, A, B, the upstream
 *     gradients and every output except T (always float32). Accumulation is
 *     float32; each stored value is rounded once (round-to-nearest-even).
 *
 * Ownership and execution:
 *   - Every pointer is caller-owned device memory; the library never
 *     allocates, frees or synchronises. Work is enqueued on the caller's HIP
 *     stream (NULL = the default stream) and the call returns at once.
 *   - Forward writes the tensors the backward needs (G, U, T); the caller
 *     keeps them alive between the two calls, as an autograd context would.
 *   - The workspace is scratch owned by the caller, sized by the query
 *     functions; its contents need not be initialised and are garbage after
 *     the call. Two calls may not share one workspace concurrently.
 *   - Results are bitwise reproducible run to run (fixed-order reductions).
 *
 * Errors: no exception crosses the ABI. Every entry point returns one of the
 * LORA_* status codes below; arguments are validated on the host before any
 * device work, so an error return means nothing was enqueued (except
 * LORA_ERR_HIP, which reports a failed launch). lora_last_error_message()
 * gives a thread-local description of the last non-OK return.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define LORA_OK 0
#define LORA_ERR_NULL 1          /* a required pointer is NULL */
#define LORA_ERR_SHAPE 2         /* non-positive size, odd head_dim, n_q % n_kv != 0, ... */
#define LORA_ERR_UNSUPPORTED 3   /* dtype / activation / rank / head_dim not supported */
#define LORA_ERR_WORKSPACE 4     /* workspace smaller than the query function's size */
#define LORA_ERR_HIP 5           /* HIP runtime or launch error */

/* ---- enums ------------------------------------------------------------- */
#define LORA_F32 0
#define LORA_BF16 1

#define LORA_SWIGLU 0            /* silu(gate) * up */
#define LORA_GEGLU_TANH 1        /* gelu_tanh(gate) * up */
#define LORA_GEGLU_ERF 2         /* gelu(gate) * up, exact GELU g * Phi(g) with the error function */

#define LORA_MAX_RANK 16         /* largest adapter rank the kernels are built for */

/* One adapted projection: frozen base W [out, in], adapter A [r, in],
 * B [out, r] (same dtype as the call), scale s (alpha / r), and an optional
 * frozen base-layer bias [out] (same dtype; NULL for none).  The bias is
 * added in the forward only and gets no gradient.  The QKV and single-linear
 * calls accept it (Opake, "Model Patches and Kernels", "Fused LoRA
 * operations": the fused QKV call allows frozen base biases); the MLP call
 * requires NULL (its fusion is for bias-free projections) and returns
 * LORA_ERR_UNSUPPORTED otherwise. */
typedef struct {
  const void* W;
  const void* A;
  const void* B;
  float scale;
  const void* bias;
} lora_proj_t;

/* LoRA MLP: gate/up [hidden -> inter], GLU, down [inter -> hidden]. */
typedef struct {
  int64_t n_tokens;   /* N = batch * seq, >= 0 */
  int32_t hidden;     /* h */
  int32_t inter;      /* i */
  int32_t rank;       /* r, 1..LORA_MAX_RANK */
  int32_t dtype;      /* LORA_F32 | LORA_BF16 */
  int32_t act;        /* LORA_SWIGLU | LORA_GEGLU_TANH | LORA_GEGLU_ERF */
  int32_t reserved;   /* must be 0 */
} lora_mlp_desc_t;

/* LoRA QKV: X [batch*seq, hidden] -> Q, K, V head-split, RoPE on Q and K. */
typedef struct {
  int32_t batch;      /* >= 0 (0: empty batch) */
  int32_t seq;
  int32_t hidden;
  int32_t n_q;        /* query heads */
  int32_t n_kv;       /* key/value heads; n_q % n_kv == 0 (GQA) */
  int32_t head_dim;   /* d: 64 or 128 */
  int32_t rank;       /* r, 1..LORA_MAX_RANK */
  int32_t dtype;      /* LORA_F32 | LORA_BF16 */
  double rope_theta;  /* RoPE base theta > 0 */
} lora_qkv_desc_t;

/* One LoRA linear (e.g. an attention output projection): X [N, in] -> Y [N, out]. */
typedef struct {
  int64_t n_tokens;      /* N >= 0 */
  int32_t in_features;   /* in */
  int32_t out_features;  /* out */
  int32_t rank;          /* r, 1..LORA_MAX_RANK */
  int32_t dtype;         /* LORA_F32 | LORA_BF16 */
} lora_linear_desc_t;

/* ---- workspace queries (pass: 0 = forward, 1 = backward) ---------------- */
size_t lora_mlp_workspace_bytes(const lora_mlp_desc_t* desc, int pass);
size_t lora_qkv_workspace_bytes(const lora_qkv_desc_t* desc, int pass);
/* The linear forward needs workspace only when few output tiles leave the
 * GPU underfilled (small n_tokens: the K range is then split over several
 * workgroups); when the query returns 0 the workspace may be NULL. */
size_t lora_linear_workspace_bytes(const lora_linear_desc_t* desc, int pass);

/*
 * MLP forward.  Defined by Opake, "Model Patches and Kernels", section "Fused
 * LoRA operations" (opake_lora_mlp: gate, up and down LoRA projections with
 * the activation between them) and section "Activation functions" (SwiGLU
 * silu(gate) * up, GeGLU gelu_tanh(gate) * up or gelu(gate) * up).
 *   X [N, h]; gate, up: W [i, h], A [r, h], B [i, r]; down: W [h, i], A [r, i], B [h, r].
 *   Writes Y [N, h] = L_d(H) with H = phi(G) * U, and the saved tensors
 *   G = L_g(X), U = L_u(X) [N, i] (pre-activation, call dtype) and
 *   T [3, N, r] float32 = (X A_g^T, X A_u^T, H A_d^T).
 */
int lora_mlp_fwd(const lora_mlp_desc_t* desc, const void* X,
                 const lora_proj_t* gate, const lora_proj_t* up, const lora_proj_t* down,
                 void* Y, void* G, void* U, void* T,
                 void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * MLP backward for the loss <dY, Y>, base weights frozen.  Defined by the
 * same passages as the forward (Opake, "Model Patches and Kernels", "Fused
 * LoRA operations": the autograd pair of opake_lora_mlp; "Activation
 * functions": the activation backward reads the upstream gradient, gate and
 * up and writes both input gradients; "Fused linear cross-entropy", key design
 * decisions: frozen weights get no weight gradient).
 *   dY [N, h]; X, G, U, T as written by lora_mlp_fwd; same projections.
 *   Writes dX [N, h] and the adapter gradients dA_* [r, in], dB_* [out, r]
 *   (call dtype, float32 accumulation).
 */
int lora_mlp_bwd(const lora_mlp_desc_t* desc, const void* dY, const void* X,
                 const void* G, const void* U, const void* T,
                 const lora_proj_t* gate, const lora_proj_t* up, const lora_proj_t* down,
                 void* dX, void* dA_gate, void* dB_gate, void* dA_up, void* dB_up,
                 void* dA_down, void* dB_down,
                 void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * QKV forward.  Defined by Opake, "Model Patches and Kernels", section "Fused
 * LoRA operations" (opake_lora_qkv: the Q, K and V LoRA projections of one
 * input in one call) and section "Rotary position embeddings (RoPE)" (RoPE
 * on Q and K together, grouped-query head counts), and by Axolotl,
 * "monkeypatch.lora_kernels", "original_apply_qkv" (hidden states in, query,
 * key and value out).
 *   X [batch*seq, h]; q: W [n_q*d, h], A [r, h], B [n_q*d, r]; k, v: W [n_kv*d, h], ...
 *   Writes Q [batch, n_q, seq, d], K, V [batch, n_kv, seq, d] (RoPE on Q and K)
 *   and T [3, N, r] float32 = (X A_q^T, X A_k^T, X A_v^T).
 */
int lora_qkv_fwd(const lora_qkv_desc_t* desc, const void* X,
                 const lora_proj_t* q, const lora_proj_t* k, const lora_proj_t* v,
                 void* Q, void* K, void* V, void* T,
                 void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * QKV backward for the loss <dQ,Q> + <dK,K> + <dV,V>, base weights frozen.
 * Defined by the same passages as the forward (the autograd pair of
 * opake_lora_qkv; the RoPE backward is the transposed rotation) and by "Fused
 * linear cross-entropy", key design decisions (no gradient for frozen W).
 *   dQ, dK, dV in the layouts of Q, K, V; X and T as for the forward.
 *   Writes dX [N, h] and dA_* [r, h], dB_* [out, r].
 */
int lora_qkv_bwd(const lora_qkv_desc_t* desc, const void* dQ, const void* dK, const void* dV,
                 const void* X, const void* T,
                 const lora_proj_t* q, const lora_proj_t* k, const lora_proj_t* v,
                 void* dX, void* dA_q, void* dB_q, void* dA_k, void* dB_k, void* dA_v, void* dB_v,
                 void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * QKV forward that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid it).  Same arguments, results and errors as
 * lora_qkv_fwd without the workspace pair: its scratch (the RoPE cos / sin
 * table, lora_qkv_workspace_bytes(desc, 0) bytes) lives in a static device
 * array of lora_qkv_fwd_noalloc_max_scratch_bytes() bytes (4 MiB: seq *
 * head_dim up to 524288) that each GPU holds until the process ends.  Larger
 * shapes return LORA_ERR_WORKSPACE before any device call.  Every call on one
 * GPU shares that GPU's array (nothing in it needs to start at zero; each call
 * rewrites the table before use), so calls that overlap on one GPU, on
 * different streams or from different threads, race.  The stream must belong
 * to the current device.
 */
int lora_qkv_fwd_noalloc(const lora_qkv_desc_t* desc, const void* X,
                         const lora_proj_t* q, const lora_proj_t* k, const lora_proj_t* v,
                         void* Q, void* K, void* V, void* T, void* hip_stream);
size_t lora_qkv_fwd_noalloc_max_scratch_bytes(void);

/* Per-head RMSNorm of Q and K (q_norm / k_norm) between the projection and
 * RoPE: each head x [head_dim] becomes x / sqrt(mean(x^2) + eps) * w, with
 * one weight vector w [head_dim] (call dtype) for all Q heads and one for all
 * K heads.  Weights are frozen (no gradient).  For Gemma-style (1 + w) norms
 * pass 1 + w. */
typedef struct {
  const void* q_weight;   /* [head_dim] */
  const void* k_weight;   /* [head_dim] */
  float eps;              /* >= 0 */
} lora_qk_norm_t;

/*
 * LoRA QKV forward with q/k norm (Opake, "Model Patches and Kernels",
 * "Fused LoRA operations" and "Model compatibility": the Qwen3 / Gemma3
 * attention wrappers keep q_norm / k_norm under QKV fusion; Zhang & Sennrich
 * RMSNorm).  As lora_qkv_fwd, with the norm applied to each Q and K head after
 * the bias and before RoPE.  It also writes, for the backward:
 *   Pn   [N, (n_q + n_kv) * head_dim]  the Q|K projections before the norm (call dtype);
 *   rinv [N, n_q + n_kv] float32       1 / sqrt(mean(x^2) + eps) per token and head.
 * The norm weights and Pn must be 16-byte aligned (LORA_ERR_UNSUPPORTED otherwise).
 * Workspace: lora_qkv_workspace_bytes(desc, 0).
 */
int lora_qkv_norm_fwd(const lora_qkv_desc_t* desc, const void* X,
                      const lora_proj_t* q, const lora_proj_t* k, const lora_proj_t* v,
                      const lora_qk_norm_t* norm, void* Q, void* K, void* V, void* T, void* Pn, float* rinv,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Backward of lora_qkv_norm_fwd: as lora_qkv_bwd, pulling R^T dQ and R^T dK
 * back through the norm with the saved Pn and rinv.  dQ, dK, dV, Pn and the
 * norm weights must be 16-byte aligned.  Workspace: lora_qkv_workspace_bytes(desc, 1).
 */
int lora_qkv_norm_bwd(const lora_qkv_desc_t* desc, const void* dQ, const void* dK, const void* dV,
                      const void* X, const void* T, const void* Pn, const float* rinv,
                      const lora_proj_t* q, const lora_proj_t* k, const lora_proj_t* v,
                      const lora_qk_norm_t* norm,
                      void* dX, void* dA_q, void* dB_q, void* dA_k, void* dB_k, void* dA_v, void* dB_v,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * LoRA linear forward (Opake, "Model Patches and Kernels", "Fused LoRA
 * operations": the single adapted projection, opake_lora_w; Axolotl,
 * "monkeypatch.lora_kernels", original_apply_o for the attention output).
 *   X [N, in]; proj: W [out, in], A [r, in], B [out, r].
 *   Writes Y [N, out] = X W^T + s (X A^T) B^T and T [N, r] float32 = X A^T.
 */
int lora_linear_fwd(const lora_linear_desc_t* desc, const void* X, const lora_proj_t* proj,
                    void* Y, void* T, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * LoRA linear backward for the loss <dY, Y>, W frozen.
 *   dY [N, out]; X and T as for the forward.
 *   Writes dX [N, in], dA [r, in], dB [out, r] (call dtype, float32 accumulation).
 */
int lora_linear_bwd(const lora_linear_desc_t* desc, const void* dY, const void* X, const void* T,
                    const lora_proj_t* proj, void* dX, void* dA, void* dB,
                    void* workspace, size_t workspace_bytes, void* hip_stream);

/* ---- diagnostics --------------------------------------------------------- */
const char* lora_status_string(int status);
const char* lora_last_error_message(void);   /* thread-local; "" after success */
const char* lora_version(void);

/*
 * Per-kernel timing with HIP events (off by default). While enabled, every
 * kernel launch is bracketed by two events recorded on the call's stream.
 * lora_timing_query synchronises those events and returns the summed
 * duration and launch count of the named kernel since the last reset;
 * lora_kernel_names lists the names (comma separated).
 */
int lora_timing_enable(int on);
int lora_timing_reset(void);
int lora_timing_query(const char* kernel, double* total_ms, int* launches);
const char* lora_kernel_names(void);

#ifdef __cplusplus
}
#endif
#endif /* LORA_MI355X_H */
