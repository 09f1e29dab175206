/*
 * libmoe -- MoE layer forward on one AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every pointer argument is a DEVICE pointer unless marked (host).
 * The caller owns every buffer (inputs, outputs and the workspace); the
 * library never allocates or frees memory, never synchronises the stream and
 * keeps no state between calls (except the wait limit of
 * moe_set_split_wait). Every call validates its arguments on the
 * host and then only enqueues kernels on `stream` (a hipStream_t passed as
 * void*; NULL means the default stream); results are ready once the stream
 * reaches that point. Nothing but kernel launches reaches the stream (the
 * split GEMMs' ready flags are cleared by a kernel, not a memset), so a call
 * may be captured into a HIP graph; each replay recomputes everything from
 * the buffers' contents at replay time. No C++ exception crosses this
 * boundary.
 *
 * Layer (sources cited by page title and section):
 *   y[t] = sum_{j < k, kept} w[t][j] * SwiGLU_{e(t,j)}(x[t]) + shared(x[t])
 *   "FFN, SwiGLU and MoE" (bjdmk.com) sec. 3 (router r = W_r x, softmax,
 *   top-k, weighted sum of the selected experts) and sec. 2 (SwiGLU);
 *   "moe f&b compute flow" (Echo's blog): Router -> Dispatch -> FFN ->
 *   Combine; "ops-transformer MoE operator on Ascend NPU" (gitcode.csdn.net):
 *   the MoEForward sketch, capacity (pitfall 1), FP32 routing (pitfall 3);
 *   "DeepSeek-V4.1-Flash fine-grained MoE (5A)" (openarchlab.com) sec. 1 and
 *   3: selection by score + bias, raw sqrt(softplus) weights, SwiGLU clamp,
 *   FP4 routed experts and one shared expert.
 *
 * Layouts (row-major, no padding):
 *   x        [T][D]      act dtype (MOE_F32 or MOE_BF16)
 *   W_r      [D][E]      fp32
 *   bias     [E]         fp32
 *   W_gate, W_up [E][D][F]  and  W_down [E][F][D]   w dtype F32 or BF16
 *   MXFP4 weights keep the logical [E][K][N] matrix but are stored by
 *     32-element K-blocks (the MX scaling blocks), block-major: codes uint8
 *     [E][K/32][N][16] (the 16 bytes of block b of column n; element 2i of
 *     the block in the low nibble of byte i, 2i+1 in the high nibble),
 *     e8m0 scales uint8 [E][K/32][N] (scale 2^(s-127), s = 255 not
 *     allowed); for gate/up K = D, N = F; for down K = F, N = D (OCP MX
 *     v1.0 e2m1 + e8m0). Block-major storage puts one K-block of
 *     consecutive columns in consecutive bytes, so the GEMM's per-step
 *     copies read whole cache lines.
 *   Shared expert: Ws_gate, Ws_up [D][shared_F], Ws_down [shared_F][D], bf16.
 *   topk_idx int32 [T][k], topk_w fp32 [T][k]   (slot 0 = largest key)
 *   counts   int32 [E]      pairs routed to each expert, before capacity
 *   offsets  int32 [E+1]    kept segment starts; offsets[E] = kept pairs A
 *   slot_pos int32 [T][k]   row of (t, j) in the segments, -1 if dropped
 *   perm_token int32 [T*k]  token of each segment row (rows < A written)
 *   x_perm   [T*k][D] act dtype  H [T*k][F] act dtype  y_perm [T*k][D] fp32
 *   (MOE_MXFP4_A8: x_perm and H hold MXFP8 rows, e4m3 codes uint8
 *   [T*k][W] (W = D for x_perm, F for H) followed by e8m0 scales uint8
 *   [ceil(W/512)][T*k][16] -- the scale of row r, block b at
 *   ((b/16)*T*k + r)*16 + b%16, so that 8 GEMM steps of a row's scales are
 *   one 16-byte piece -- in the same bf16-sized buffers)
 *   y        [T][D]   act dtype
 * Every device pointer must be 16-byte aligned.
 *
 * Errors: functions return MOE_OK (0) or a negative moe_status. Invalid
 * arguments are rejected before anything is enqueued. MOE_ERR_HIP means a
 * launch failed; moe_last_hip_error() then returns the hipError_t of the
 * calling thread's last failure.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

/* MOE_MXFP4_A8: the MXFP4 weights of MOE_MXFP4 (same layout), with the
 * routed experts' activation operands (the x rows and H) quantised to
 * MXFP8 (OCP MX v1.0: e4m3 elements, one e8m0 scale per 32 values along
 * K) so that the products run on the block-scaled MFMA. The pages store the
 * routed experts in FP4 and say nothing of the activations; this mode is an
 * opt-in addition. The quantisation of a block of 32 values v: exponent
 * X = floor(log2 max|v|) - 8, clamped to [-127, 127] (-127 for a zero
 * block); element = e4m3 of v / 2^X, ties to even, saturated at +-448. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2, MOE_MXFP4_A8 = 3 } moe_dtype;

typedef enum {
  MOE_GATE_SOFTMAX = 0,       /* p = softmax(logit + bias) over all E */
  MOE_GATE_SIGMOID = 1,       /* w = 1/(1+exp(-logit)) */
  MOE_GATE_SQRT_SOFTPLUS = 2  /* w = sqrt(softplus(logit)) */
} moe_gating;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad size or mode */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels cover */
  MOE_ERR_WORKSPACE = -3,    /* workspace missing or smaller than needed */
  MOE_ERR_HIP = -4,          /* a HIP launch failed */
  MOE_ERR_SCRATCH = -5       /* size beyond the fixed scratch of moe_dispatch_noalloc */
} moe_status;

typedef enum {
  MOE_WS_DISPATCH = 0,
  MOE_WS_EXPERT_FFN = 1,
  MOE_WS_FORWARD = 2,
  MOE_WS_ROUTE = 3
} moe_ws_kind;

/* Layer configuration (host struct, read during the call only).
 *   T tokens (B*S flattened), D model width, E routed experts, F expert
 *   width, top_k experts per token (1 <= top_k <= min(E, 16)).
 *   gating    moe_gating.
 *   renorm    1: divide the k selected weights by their sum (the module's
 *             top-k renormalisation in "FFN, SwiGLU and MoE" sec. 3).
 *   capacity  <= 0: unlimited; else each expert keeps at most `capacity`
 *             pairs, the earliest tokens first ("ops-transformer" pitfall 1).
 *   clamp     <= 0: none; else gate and up pre-activations are clamped to
 *             [-clamp, clamp] before SiLU(gate)*up ("DeepSeek-V4.1-Flash"
 *             sec. 1, 3), in routed and shared experts.
 *   act_dtype MOE_F32 (then w_dtype MOE_F32) or MOE_BF16 (then w_dtype
 *             MOE_BF16, MOE_MXFP4 or MOE_MXFP4_A8; MOE_MXFP4_A8 needs D
 *             and F multiples of 64).
 *   shared_F  0: no shared expert; else the width of one always-on bf16
 *             SwiGLU expert added with weight 1 (requires MOE_BF16). */
typedef struct moe_cfg {
  int32_t T, D, E, F, top_k;
  int32_t gating;
  int32_t renorm;
  int32_t capacity;
  float clamp;
  int32_t act_dtype, w_dtype;
  int32_t shared_F;
} moe_cfg;

/* Expert weights (host struct of device pointers). S_* are the e8m0 scale
 * arrays for MXFP4 (NULL otherwise). Ws_* are the shared expert's (NULL
 * when shared_F == 0). */
typedef struct moe_weights {
  const void *W_gate, *W_up, *W_down;
  const uint8_t *S_gate, *S_up, *S_down;
  const void *Ws_gate, *Ws_up, *Ws_down;
} moe_weights;

/* Bytes of workspace a call needs (host out-parameter `bytes`).
 * MOE_WS_DISPATCH for moe_dispatch (per-chunk expert counts),
 * MOE_WS_EXPERT_FFN for moe_expert_ffn / _gate_up / _down (the device tile
 * map and, with bf16 activations, 64 MiB of fp32 partial sums plus two
 * banks of ready flags for the GEMM tiles that are split along K, and with
 * MOE_MXFP4_A8 the MXFP8 copy of x that a gathered gate/up reads),
 * MOE_WS_ROUTE for moe_route_screened (0 where it runs the exact router),
 * MOE_WS_FORWARD for moe_forward (all of the above plus H, y_perm, x_perm for fp32
 * activations only, the MXFP8 copy of x for MOE_MXFP4_A8 and, with a
 * shared expert, its H and output). A workspace carries state only within
 * one call; calls that run concurrently need separate workspaces. */
int moe_workspace_size(const moe_cfg* cfg, int kind, size_t* bytes);

/* Router ("FFN, SwiGLU and MoE" sec. 3; "ops-transformer" MoEForward steps
 * 1-2, optimisation 2, pitfall 3; "DeepSeek-V4.1-Flash" sec. 1, 3;
 * "MoE routing: Top-K, Expert-Choice and Sigmoid Gating").
 *   logit[t][e] = fp32 fused multiply-add chain over d = 0..D-1 of
 *                 x[t][d]*W_r[d][e], starting from +0 (bit-reproducible);
 *   key = logit + bias[e] (bias may be NULL = 0); the k largest keys in
 *   descending order, equal keys to the lower expert index, go to topk_idx;
 *   topk_w by the gating mode (softmax uses the keys, sigmoid and
 *   sqrt-softplus the raw logits), renormalised when cfg->renorm.
 *   logits [T][E] fp32 is an optional output (NULL: not written). */
int moe_route(const moe_cfg* cfg, const void* x, const float* W_r, const float* bias,
              int32_t* topk_idx, float* topk_w, float* logits, void* stream);

/* moe_route without the logits output, for many experts: the same
 * topk_idx and topk_w, bit for bit, with most of the fp32 chains skipped.
 * An estimate of every logit on the bf16 MFMA (x times bf16(W_r)) with a
 * rigorous bound eps_t on its distance from the defined fp32 chain (from
 * ||x_t||, the norms of W_r's columns and of their bf16 residuals, and the
 * fp32 accumulation error bound D u / (1 - D u) of the chain and, with a
 * safety factor, of the MFMA) keeps, per token, the experts whose estimated
 * key is within 2 eps_t of the k-th largest: the exact top k is always
 * among them ("ops-transformer" pitfall 3: the router is FP32; its
 * performance comparison counts routing among the overheads). Only their
 * exact chains run; selection and weights then use the exact router's
 * code. Used with bf16 activations, E >= 128 and any gating except softmax
 * without renormalisation; otherwise this call runs the exact router
 * (workspace size 0). Workspace: MOE_WS_ROUTE. moe_forward takes this path
 * whenever it applies. */
int moe_route_screened(const moe_cfg* cfg, const void* x, const float* W_r, const float* bias,
                       int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream);

/* Dispatch ("moe f&b compute flow" Dispatch; "ops-transformer" MoEForward
 * step 3 GetTokensForExpert/Gather, pitfall 1). Groups the (t, j) pairs by
 * expert, token order inside each expert; pairs whose rank within their
 * expert reaches cfg->capacity are dropped. Writes counts, offsets,
 * slot_pos, perm_token and copies each kept pair's x row to x_perm (with
 * MOE_MXFP4_A8: the row's MXFP8 quantisation, quantised once per token).
 * x_perm may be NULL: then no row is copied (for callers that gather the
 * rows through perm_token, as moe_expert_gate_up_gathered does).
 * Integer outputs are deterministic and bit-exact. T = 0: counts and
 * offsets are written as zeros and nothing else is enqueued. */
int moe_dispatch(const moe_cfg* cfg, const int32_t* topk_idx, const void* x, int32_t* counts,
                 int32_t* offsets, int32_t* slot_pos, int32_t* perm_token, void* x_perm,
                 void* ws, size_t ws_bytes, void* stream);

/* moe_dispatch for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the per-chunk expert
 * counts in a fixed 1 MiB device array of the library instead of a
 * caller's workspace. Limit: E * ceil(T / 256) <= 262144 (e.g. E = 1024
 * with T up to 65536), else MOE_ERR_SCRATCH and nothing is enqueued. It
 * calls no allocating routine. Each GPU holds its own copy of the array
 * until the process ends, and every call on that GPU shares it: calls that
 * overlap on one GPU (other streams, other threads) race. Nothing in it
 * needs clearing between calls. */
int moe_dispatch_noalloc(const moe_cfg* cfg, const int32_t* topk_idx, const void* x,
                         int32_t* counts, int32_t* offsets, int32_t* slot_pos,
                         int32_t* perm_token, void* x_perm, void* stream);

/* Routed experts ("FFN, SwiGLU and MoE" sec. 2; "ops-transformer"
 * optimisation 3, one launch over all experts' irregular segments):
 * for every kept row r of expert e's segment,
 *   H[r] = SiLU(clampL(x_perm[r] W_gate[e])) * clampL(x_perm[r] W_up[e])
 *          (rounded to the act dtype), y_perm[r] = H[r] W_down[e] (fp32).
 * With MOE_MXFP4_A8, x_perm is the MXFP8 x_perm that moe_dispatch writes
 * and H is stored as MXFP8 (computed in fp32, then quantised).
 * Rows r >= offsets[E] are not written. */
int moe_expert_ffn(const moe_cfg* cfg, const void* x_perm, const int32_t* offsets,
                   const moe_weights* w, void* H, float* y_perm, void* ws, size_t ws_bytes,
                   void* stream);

/* The two halves of moe_expert_ffn, for callers that schedule or time them
 * separately. moe_expert_gate_up writes H only; moe_expert_down reads H and
 * writes y_perm. Both take the same workspace as moe_expert_ffn. */
int moe_expert_gate_up(const moe_cfg* cfg, const void* x_perm, const int32_t* offsets,
                       const moe_weights* w, void* H, void* ws, size_t ws_bytes, void* stream);
int moe_expert_down(const moe_cfg* cfg, const void* H, const int32_t* offsets,
                    const moe_weights* w, float* y_perm, void* ws, size_t ws_bytes, void* stream);

/* moe_expert_gate_up reading its rows from x itself: routed row r is row
 * perm_token[r] of x [T][D] ("ops-transformer" MoEForward gathers each
 * expert's tokens; here the gather happens inside the GEMM's copies, so no
 * dispatched copy x_perm is written). bf16 activations only
 * (MOE_ERR_UNSUPPORTED otherwise); with MOE_MXFP4_A8 x is first quantised
 * to MXFP8 once per token, into the workspace. The same kernels and
 * results as moe_forward's gate/up stage. Workspace: MOE_WS_EXPERT_FFN. */
int moe_expert_gate_up_gathered(const moe_cfg* cfg, const void* x, const int32_t* perm_token,
                                const int32_t* offsets, const moe_weights* w, void* H, void* ws,
                                size_t ws_bytes, void* stream);

/* Shared expert ("DeepSeek-V4.1-Flash" sec. 1, 3): the same SwiGLU with
 * the bf16 weights Ws_* on every token. H_shared [T][shared_F] bf16 is
 * scratch owned by the caller; y_shared [T][D] fp32. */
int moe_shared_expert(const moe_cfg* cfg, const void* x, const moe_weights* w, void* H_shared,
                      float* y_shared, void* stream);

/* Combine ("moe f&b compute flow" Combine; "ops-transformer" Scatter and
 * WeightedSum; "FFN, SwiGLU and MoE" sec. 3):
 *   y[t] = sum over j ascending with slot_pos[t][j] >= 0 of
 *          topk_w[t][j] * y_perm[slot_pos[t][j]]  (+ y_shared[t] if not NULL),
 * accumulated in fp32, stored in the act dtype (round to nearest even). */
int moe_combine(const moe_cfg* cfg, const float* y_perm, const int32_t* slot_pos,
                const float* topk_w, const float* y_shared, void* y, void* stream);

/* The whole layer: route, dispatch, routed experts, shared expert (when
 * cfg->shared_F > 0) and combine, enqueued back to back with no host
 * synchronisation. topk_idx, topk_w, counts and offsets are optional
 * outputs (NULL: kept in the workspace). With bf16 activations the gate/up
 * GEMM fetches each routed row from x through perm_token, so the
 * dispatched copy x_perm is never written; the results are the same as
 * those of the stage entry points. T = 0: the optional counts and offsets
 * are written as zeros and nothing else is enqueued. */
int moe_forward(const moe_cfg* cfg, const void* x, const float* W_r, const float* bias,
                const moe_weights* w, void* y, int32_t* topk_idx, float* topk_w,
                int32_t* counts, int32_t* offsets, void* ws, size_t ws_bytes, void* stream);

/* MXFP8 quantisation of bf16 rows, the activation format of MOE_MXFP4_A8
 * (OCP MX v1.0 conversion, as stated at MOE_MXFP4_A8): x [rows][K] bf16 ->
 * e4m3 codes uint8 [rows][K] and e8m0 scales uint8 [rows][K/32], one scale
 * per 32 consecutive values of a row. K must be a positive multiple of 32
 * and rows >= 0; inputs are expected to be finite. */
int moe_quantize_mxfp8(const void* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                       void* stream);

/* Split-tile hand-off of the grouped GEMMs (bf16 activations). The tiles
 * of a launch's last, partial round of workgroups are split along K: each
 * earlier part leaves fp32 partial sums in the workspace and raises a ready
 * flag, and the last part adds them in part order before the epilogue. The
 * last part polls each flag at most `polls` times (default 2^24, about a
 * second) and, if it does not rise, stores NaN (bf16 / fp32 NaN; in
 * MXFP8 H the NaN codes and the e8m0 NaN scale 0xFF) for the outputs of
 * that tile instead of a partial sum, so a failed hand-off cannot pass for
 * a result; every workgroup still exits normally. polls = 0 makes every
 * split tile give up at once (for testing that path). The setting is
 * process-wide and the one piece of state the library keeps; it applies to
 * launches enqueued after the call. Returns the previous value, or
 * MOE_ERR_INVALID_ARG for polls < 0. */
int moe_set_split_wait(int polls);

/* Static text for a moe_status value (host pointer, never NULL). */
const char* moe_status_string(int status);

/* hipError_t of the calling thread's last MOE_ERR_HIP (0 if none). */
int moe_last_hip_error(void);

/* MOE_ABI_VERSION of the library. */
int moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
