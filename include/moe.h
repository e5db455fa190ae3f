/*
 * moe.h -- C ABI of libmoe: one Mixture-of-Experts FFN layer forward on an
 * AMD Instinct MI355X (gfx950).
 *
 * The layer is the pipeline of forward_prefill.rs (page 3,
 * MoeLayer::forward_prefill, doc comment "Pipeline"):
 *
 *   router GEMM -> gating + top-k -> sort by expert -> grouped gate/up GEMM
 *   with SiLU gating (SwiGLU) -> grouped down GEMM -> unpermute + weighted
 *   top-k reduce -> shared-expert blend
 *
 * out[t] = sum_j w[t,j] * E_{idx[t,j]}(x[t]) + S(x[t]),  with
 * E_e(x) = W2[e] . q( silu(W1[e] x) * (W3[e] x) ) and S the shared expert
 * (added with weight 1) when the plan has one.  q() rounds the SwiGLU output
 * to the down product's operand format (bf16, or fp8 per row per 128
 * columns).  The routing weight multiplies at the combine (page 3, step 7
 * moe_unpermute_reduce_indexed).
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned (hipMalloc'd or torch tensors); the
 *     library never allocates device memory and never synchronises the host.
 *   - All work is enqueued on the caller's stream (a hipStream_t passed as
 *     void*; NULL = the default stream).  Outputs are valid once that stream
 *     has completed.
 *   - Arguments are validated before anything is enqueued; on a validation
 *     error the return value is non-zero, nothing is enqueued and outputs are
 *     untouched.  A HIP error met while enqueueing (MOE_ERR_HIP) stops the
 *     call at that stage: the stages before it stay enqueued on the stream,
 *     and the outputs and the workspace are then undefined.
 *   - A zero-size launch is never made (page 3: a kernel with grid.x = 0 is
 *     an invalid launch, so the shared expert is skipped when absent);
 *     m == 0 returns MOE_OK with nothing enqueued.
 *   - No C++ exception crosses the ABI.  A plan is immutable after
 *     moe_plan() and may be used from several threads; a workspace must not
 *     be shared by calls that may run concurrently.
 *   - Two calls with the same inputs give bit-identical outputs (no
 *     floating-point atomics; every sum has a fixed order).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_plan_s *moe_plan_t;

/* Storage formats.  MOE_FP8_E4M3 is OCP e4m3fn (bias 7, max 448, no inf).
 * MOE_MXFP4 (expert weights only) is OCP Microscaling FP4: e2m1 elements
 * (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte along K (even element
 * in the low nibble), with one E8M0 scale byte 2^(e - 127) per 32 consecutive
 * elements of a row; scale bytes 0 and 255 are not supported.  The MX
 * elements are the "block-scaled" weight format of page 1 (its NVFP4 W4A4
 * MoE) on gfx950's own FP4 conversion; x, h and out stay bf16.  MOE_MXFP8
 * (expert weights only) is OCP Microscaling FP8: one e4m3fn byte per element
 * with the same E8M0 scale per 32 elements along K. */
typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3 = 2,
  MOE_MXFP4 = 3,
  MOE_MXFP8 = 4
} moe_dtype_t;

/* Gating (page 3, step 2 "Batched topK dispatch": softmax, sigmoid with a
 * correction bias, sqrtsoftplus with a correction bias, softmax with a
 * correction bias).  Experts are ranked by score + bias (bias = 0 when
 * router_bias is NULL; the bias selects only), ties -> lower index; the
 * weights use the unbiased scores:
 *  SOFTMAX:      score p = softmax(l) over all E;
 *  SIGMOID:      score s = 1 / (1 + e^-l);
 *  SQRTSOFTPLUS: score s = sqrt(ln(1 + e^l));
 *  w_j = score_j / sum_sel score (if renormalize) * routed_scale. */
typedef enum {
  MOE_GATE_SOFTMAX = 0,
  MOE_GATE_SIGMOID = 1,
  MOE_GATE_SQRTSOFTPLUS = 2
} moe_gating_t;

/* Expert-path choice.  AUTO: fp32 weights -> SIMPLE; bf16 weights: m <= 256
 * -> SMALL_M, else GROUPED; MXFP4 / MXFP8 weights: SMALL_M at every m; fp8
 * weights: GROUPED.  The others force a path (for testing; every path
 * computes the same layer). */
typedef enum {
  MOE_PATH_AUTO = 0,
  MOE_PATH_SIMPLE = 1,   /* fp32 VALU kernels, any dtype */
  MOE_PATH_GROUPED = 2,  /* MFMA grouped GEMM, bf16 / fp8 */
  MOE_PATH_SMALL_M = 3   /* weight-streaming path: bf16 m <= 256, MXFP4 / MXFP8 any m */
} moe_path_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misalignment       */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not supported by this build      */
  MOE_ERR_WORKSPACE = 3,    /* workspace too small                        */
  MOE_ERR_HIP = 4,          /* a HIP runtime call failed (see strerror)   */
  MOE_ERR_NO_MEMORY = 5     /* moe_plan could not allocate its host record */
} moe_status_t;

typedef struct {
  int32_t hidden;        /* H */
  int32_t num_experts;   /* E, 1..1024 */
  int32_t inter;         /* I of each routed expert */
  int32_t shared_inter;  /* I_s of the shared expert, 0 = none */
  int32_t topk;          /* k, 1..min(E, 32) */
  int32_t max_tokens;    /* largest m accepted by moe_forward */
  int32_t gating;        /* moe_gating_t */
  int32_t renormalize;   /* 1: divide the k selected weights by their sum */
  float routed_scale;    /* multiplier applied after renormalisation */
  int32_t weight_dtype;  /* moe_dtype_t.  F32 => x/out are fp32;
                            BF16, FP8_E4M3, MXFP4 or MXFP8 => x/out are bf16 */
  int32_t path;          /* moe_path_t */
} moe_config_t;

/* Shared expert weights (NULL pointer to this struct iff shared_inter == 0).
 * w13 [2*I_s, H]: rows [0, I_s) = w1 (gate), rows [I_s, 2*I_s) = w3 (up).
 * w2  [H, I_s].  fp8: w13_scale [2*I_s/128, H/128], w2_scale [H/128, I_s/128]
 * fp32 per 128x128 block (value = code * scale); MXFP4: w13 [2*I_s, H/2] and
 * w2 [H, I_s/2] bytes, w13_scale [2*I_s, H/32] and w2_scale [H, I_s/32] E8M0
 * bytes; MXFP8: w13 [2*I_s, H] and w2 [H, I_s] bytes with the same scales;
 * NULL otherwise.
 * gate [H] in the format of x (fp32 or bf16), or NULL: when set, the shared
 * row of token t is added with weight sigmoid(x[t] . gate) (fp32 dot product
 * of the unquantised input; page 3, step 8, the shared-expert blend),
 * otherwise with weight 1. */
typedef struct {
  const void *w13;
  const void *w2;
  const void *w13_scale;
  const void *w2_scale;
  const void *gate;
} moe_shared_t;

/* Stages of one forward, in launch order (page 3, MoeLayer::forward_prefill
 * steps 1-8). */
enum {
  MOE_STAGE_ROUTER = 0,   /* router logits                                  */
  MOE_STAGE_TOPK = 1,     /* gating + top-k                                 */
  MOE_STAGE_PERMUTE = 2,  /* sort by expert                                 */
  MOE_STAGE_QUANT = 3,    /* fp8 activation quantisation (empty otherwise)  */
  MOE_STAGE_GATEUP = 4,   /* gate/up GEMM + SwiGLU, routed and shared       */
  MOE_STAGE_DOWN = 5,     /* down GEMM, routed and shared                   */
  MOE_STAGE_COMBINE = 6,  /* unpermute + weighted reduce + shared blend     */
  MOE_NUM_STAGES = 7
};

/* Optional stage outputs of moe_forward_debug (any pointer may be NULL).
 * Sizes use te = m*k.  Rows of h and y are in sorted (by expert) order.
 * events[i] (a hipEvent_t, caller-created) is recorded on the stream just
 * before stage i is enqueued, events[MOE_NUM_STAGES] after the last one, so
 * hipEventElapsedTime(events[i], events[i+1]) times stage i (the timing hooks
 * of page 3's prof_step and page 4's BackendTimer, without a host sync). */
typedef struct {
  float *logits;          /* [m, E] fp32 router logits                     */
  int32_t *counts;        /* [E] tokens per expert                          */
  int32_t *offsets;       /* [E+1] exclusive prefix of counts               */
  int32_t *sorted_pair;   /* [te] pair p = t*k+j, grouped by expert, p asc. */
  int32_t *slot_of_pair;  /* [te] inverse of sorted_pair                    */
  uint8_t *xq;            /* [m, H] fp8 codes of x (FP8 weights only)       */
  float *sx;              /* [m, H/128] their scales (FP8 weights only)     */
  void *h;                /* [te, I] SwiGLU output in the down operand
                             format: fp32 (F32), bf16 (BF16), codes (FP8)   */
  float *h_scale;         /* [te, I/128] scales of h (FP8 weights only)     */
  void *events[MOE_NUM_STAGES + 1];
  void *h_shared;         /* [m, I_s] shared-expert SwiGLU output, as h     */
  float *h_shared_scale;  /* [m, I_s/128] its scales (FP8 weights only)     */
  float *y;               /* [te, H] routed down output, sorted rows, fp32  */
  float *y_shared;        /* [m, H] shared-expert down output, fp32         */
} moe_debug_t;

/* Validate cfg and create a plan (host memory only; no device work): the
 * layer's configuration, read once before the layer runs as forward.rs
 * (page 1, forward_rows) reads the model configuration's hidden size, top-k
 * experts, MoE intermediate size and number of experts.
 * Errors: MOE_ERR_NO_MEMORY if the plan's host record cannot be allocated;
 * MOE_ERR_INVALID_ARG for non-positive sizes, topk outside
 * [1, min(E,32)], E > 1024, unknown enums; MOE_ERR_UNSUPPORTED for fp8 with
 * H, I or I_s not multiples of 128, bf16/fp8 with H, I or I_s not multiples
 * of 32, MXFP4 (MXFP8) with H, I or I_s not multiples of 256 (128) or the
 * GROUPED path forced (the MX formats run on the weight-streaming path, or
 * the VALU path when forced), SMALL_M forced with fp8/fp32 weights, or
 * sizes whose operands
 * reach 2 GiB (max_tokens * topk * max(H, I, I_s) elements, or one expert's
 * 2 * max(I, I_s) * H weight elements, at 2 bytes per bf16/fp8 element and 4
 * per fp32: the expert kernels use 32-bit byte offsets). */
int moe_plan(const moe_config_t *cfg, moe_plan_t *plan_out);

/* Bytes of device workspace that moe_forward needs for any call of up to m
 * tokens (0 on a NULL plan): the caller-preallocated scratch of the pages'
 * layer (forward.rs, page 1, forward_rows: the decode arm's MoeDecodeScratch
 * of logits, expert ids, weights and quantised h buffers; forward_prefill.rs,
 * page 3, step 2: the top-k indices and weights in the shared scratch).  The
 * workspace holds logits, the permutation, the list of experts with rows and
 * their row-block prefix, quantised activations, the sorted intermediates,
 * the expert GEMMs' unit-queue counters (set by each call before use, so the
 * contents need not be initialised) and, for calls of <= 16 tokens, the
 * router's partial sums. */
size_t moe_workspace_bytes(moe_plan_t plan, int32_t m);

/* Forward of the layer for m tokens (page 2, MoeV41::forward: x, m and a
 * stream in; the bf16 [m, dim] output and the [m, topk] routing weights and
 * indices out).
 *   x          [m, H]     fp32 or bf16 (per weight_dtype), row-major.
 *   router_w   [E, H]     same format as x.  Logits are accumulated in fp32.
 *   experts_w13[E, 2I, H] rows [0,I) = w1 (gate), [I,2I) = w3 (up); weight
 *                         format (fp32 / bf16 / fp8 codes).
 *   experts_w2 [E, H, I]  weight format.
 *   shared_w   see moe_shared_t; NULL iff shared_inter == 0.
 *   topk       must equal the plan's k.
 *   out        [m, H]     fp32 (F32 weights) or bf16; overwritten.
 *   topk_idx   [m, k]     int32 expert ids, descending score, ties -> lower id.
 *   topk_w     [m, k]     fp32 gate weights in the same order.
 *   router_bias[E]        fp32 selection-only bias, or NULL (any gating).
 *   w13_scale  [E, 2I/128, H/128], w2_scale [E, H/128, I/128]: fp32 block
 *                         scales for FP8 weights; [E, 2I, H/32] and
 *                         [E, H, I/32] E8M0 bytes for MXFP4 / MXFP8
 *                         weights (then experts_w13 is [E, 2I, H/2] and
 *                         experts_w2 [E, H, I/2] bytes for MXFP4, [E, 2I, H]
 *                         and [E, H, I] bytes for MXFP8); NULL otherwise.
 *   workspace  device buffer of >= moe_workspace_bytes(plan, m) bytes,
 *              256-byte aligned; its contents need not be initialised.
 * Every pointer must be 16-byte aligned.  FP8: activations are quantised
 * inside the layer to e4m3 with one fp32 scale per token per 128 columns
 * (scale = amax/448), and the SwiGLU output likewise per row per 128
 * columns before the down product. */
int moe_forward(moe_plan_t plan, int32_t m, const void *x, const void *router_w,
                const void *experts_w13, const void *experts_w2,
                const moe_shared_t *shared_w, int32_t topk, void *out,
                int32_t *topk_idx, float *topk_w, const float *router_bias,
                const void *w13_scale, const void *w2_scale,
                void *workspace, size_t workspace_bytes, void *stream);

/* moe_forward with stage timing events, then copies of the intermediate
 * stages into dbg (stage-wise parity, after page 3's dump_gate_logits /
 * dump_expert_ids / dump_moe_out hooks).  Same arguments and errors; dbg
 * may be NULL. */
int moe_forward_debug(moe_plan_t plan, int32_t m, const void *x,
                      const void *router_w, const void *experts_w13,
                      const void *experts_w2, const moe_shared_t *shared_w,
                      int32_t topk, void *out, int32_t *topk_idx, float *topk_w,
                      const float *router_bias, const void *w13_scale,
                      const void *w2_scale, void *workspace,
                      size_t workspace_bytes, void *stream,
                      const moe_debug_t *dbg);

/* Bytes of the static device scratch behind moe_forward_noalloc (one copy
 * per GPU the library runs on, held until the process ends). */
#define MOE_NOALLOC_SCRATCH_BYTES (128u << 20)

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without the workspace, which comes from a static device
 * array of MOE_NOALLOC_SCRATCH_BYTES per GPU instead (its device address is
 * looked up once per device; no hipMalloc, hipFree or allocating library
 * call is made).  The caller still owns every input and output.  A call
 * whose workspace would exceed the scratch (moe_workspace_bytes(plan, m) >
 * MOE_NOALLOC_SCRATCH_BYTES, e.g. the 4096-token fp8 layer) returns
 * MOE_ERR_WORKSPACE before anything is enqueued, and moe_strerror names the
 * sizes.  Every call on one GPU shares that GPU's scratch and leaves its
 * contents behind (the layer needs none of them zeroed): calls that may
 * overlap on one GPU -- on different streams or threads -- race on it and
 * must be ordered by the caller.  Other errors as moe_forward. */
int moe_forward_noalloc(moe_plan_t plan, int32_t m, const void *x, const void *router_w,
                        const void *experts_w13, const void *experts_w2,
                        const moe_shared_t *shared_w, int32_t topk, void *out,
                        int32_t *topk_idx, float *topk_w, const float *router_bias,
                        const void *w13_scale, const void *w2_scale, void *stream);

/* Which expert path moe_forward takes for m tokens (a moe_path_t other than
 * AUTO), or -1 on a NULL plan. */
int moe_path_for(moe_plan_t plan, int32_t m);

/* Release a plan (NULL is ignored). */
void moe_plan_destroy(moe_plan_t plan);

/* Static text for a status code (library plumbing; the pages' layer code
 * returns each launch's error to its caller with the failing call's text,
 * forward.rs, page 1, forward_rows).  For MOE_ERR_HIP the text of the most
 * recent failing HIP call on this thread is appended; for MOE_ERR_WORKSPACE
 * the sizes of the most recent workspace error on this thread. */
const char *moe_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
