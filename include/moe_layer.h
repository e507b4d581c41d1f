/*
 * moe_layer.h -- C ABI of the MI355X (gfx950) DeepSeekMoE layer forward pass.
 *
 * The operation (DeepSeekMoE paper abstract; DeepSeekMoE blog post, sections
 * "Fine-Grained Expert Segmentation (Section 3.1)", "Shared Expert Isolation
 * (Section 3.2)" and "DeepSeekMoE 2B Model Example"; DeepSeek-V3 Technical
 * Report summary, section "2. Architecture"):
 *
 *   for every token u_t (row t of x):
 *     l_e   = u_t . Wg_e (+ logit_bias_e)                 fp32, e < n_routed
 *     s_e   = softmax_e(l) | sigmoid(l_e)
 *     key_e = s_e (+ select_bias_e)        bias used for choosing only
 *     [group limit: experts split into n_groups contiguous groups; a group's
 *      score is the sum of its two highest keys; only the topk_groups best
 *      groups stay eligible]
 *     sel   = the top_k largest keys (key descending, then index ascending)
 *     g_k   = s_{sel_k} [/ sum_k s_{sel_k} if norm_topk] * routed_scale
 *     out_t = u_t + sum_{s<n_shared} FFN^sh_s(u_t) + sum_k g_k FFN_{sel_k}(u_t)
 *   with every expert a SwiGLU FFN:  FFN(u) = W2 (silu(W1 u) * (W3 u)).
 *
 * No token is dropped (no capacity limit).  Shared experts are always active
 * with weight one.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (HIP), row-major, densely packed,
 *    unless stated otherwise.  The caller owns all memory; the library never
 *    allocates or frees device memory.  Its only state is the backward pass's
 *    side stream: one stream and three events per host thread and device,
 *    created on the first untraced bf16 backward with shared experts and
 *    destroyed when that host thread exits (moe_side_stream_count reports how
 *    many exist).  Calls on different streams may run concurrently (with
 *    distinct workspaces); backward calls made from one host thread on
 *    different streams share that thread's side stream, so their
 *    shared-expert branches run one after the other (results unaffected).
 *  - moe_layer_forward* are asynchronous: they enqueue kernels on `stream`
 *    (a hipStream_t, NULL = the null stream) and return without waiting.
 *    The forward enqueues, in order: the router, the dispatch scan, the row
 *    maps (in the scan's launch when T * top_k <= 8192), one grouped gate/up
 *    GEMM launch over the routed experts' tiles
 *    and the shared experts', one grouped down-projection launch (routed
 *    rows and the shared experts' sum), and the combine.
 *  - Validation errors are returned before anything is enqueued.  A failed
 *    kernel launch returns MOE_ERR_HIP.  An error left pending in the calling
 *    thread's HIP error state by an earlier, unrelated HIP call is cleared at
 *    entry (it is not this call's failure); a device fault stays sticky and
 *    fails the call.
 *  - Results are bitwise reproducible for identical inputs and shapes (no
 *    floating-point atomics; the expert-contiguous order is stable).
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* bad descriptor field or NULL required pointer */
  MOE_ERR_WORKSPACE = -2,   /* workspace NULL or smaller than required       */
  MOE_ERR_UNSUPPORTED = -3, /* valid layer, but a shape this build rejects   */
  MOE_ERR_ALIAS = -4,       /* out overlaps x                                 */
  MOE_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed     */
  MOE_ERR_SCRATCH = -6      /* moe_layer_forward_noalloc: the layer needs more
                               than MOE_NOALLOC_SCRATCH_BYTES of workspace    */
} moe_status_t;

/* Layer precision.  MOE_FP8: x and out bf16, router fp32 as for bf16; the
 * expert GEMMs take FP8 operands: weights given as OCP E4M3 codes with one
 * power-of-two scale per 128 x 128 block (see moe_ffn_weights_t), token rows
 * and SwiGLU activations quantised inside the call per 1 x 128 along the
 * reduction dimension (DeepSeek-V3 Technical Report summary, "3.3 FP8
 * Training" and "B.2 Discussion About Block-Wise Quantization"). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8 = 2 } moe_dtype_t;
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_t;

/* Shape and routing options of one MoE layer. */
typedef struct {
  int32_t T;            /* tokens (rows of x and out), >= 0                    */
  int32_t d;            /* hidden size, >= 1                                    */
  int32_t n_routed;     /* mN routed experts, 1..256                           */
  int32_t top_k;        /* mK kept per token, 1..min(n_routed, 32)             */
  int32_t inner;        /* routed expert SwiGLU inner size, >= 1               */
  int32_t n_shared;     /* K_s always-active shared experts, >= 0              */
  int32_t shared_inner; /* shared expert inner size (ignored if n_shared == 0) */
  int32_t n_groups;     /* expert groups for group-limited routing (1 = off);
                           must divide n_routed, <= 64                          */
  int32_t topk_groups;  /* groups kept per token, 1..n_groups, and
                           topk_groups * (n_routed / n_groups) >= top_k        */
  int32_t score;        /* moe_score_t                                          */
  int32_t norm_topk;    /* 1: kept gate weights renormalised to sum to 1       */
  float routed_scale;   /* factor on the routed gate weights (1.0 = none)      */
  int32_t dtype;        /* moe_dtype_t: of x, out and all expert weights for
                           F32 / BF16; MOE_FP8 see above                        */
} moe_layer_desc_t;

/* One set of expert weights, stacked over E experts (E = n_routed or
 * n_shared), in the output-major layout of a linear layer's weight:
 *   w1, w3 : [E][inner][d]   (gate and up projections, d -> inner)
 *   w2     : [E][d][inner]   (down projection, inner -> d)
 * Element type desc->dtype (F32, BF16) or one E4M3 byte (FP8).  FP8 only:
 *   s1, s3 : [E][inner / 128][d / 128] and s2 : [E][d / 128][inner / 128]
 *   scale bytes b of the 128 x 128 blocks (block value = code x 2^(b - 127));
 *   NULL for F32 / BF16.  moe_quantize_fp8_blocks produces this format. */
typedef struct {
  const void* w1;
  const void* w3;
  const void* w2;
  const uint8_t* s1;
  const uint8_t* s3;
  const uint8_t* s2;
} moe_ffn_weights_t;

/* Weight gradients of a group of experts (backward pass), fp32, written (not
 * accumulated): dw1, dw3 [E][inner][d] and dw2 [E][d][inner], the layout of
 * the weights. */
typedef struct {
  float* dw1;
  float* dw3;
  float* dw2;
} moe_ffn_grads_t;

/* Byte offsets of the intermediate buffers inside the workspace, for
 * inspection after a forward call has completed (-1 = not materialised).
 * Element types: *_i32 int32, *_f32 float, y as stated below, others
 * desc->dtype.  Rows of xp / h_routed / y are in expert-contiguous order
 * (expert ascending, token ascending); row r came from token row_src[r]. */
typedef struct {
  int64_t topk_idx_i32;     /* [T][top_k]; written only when topk_idx == NULL */
  int64_t topk_w_f32;       /* [T][top_k]; written only when topk_w == NULL   */
  int64_t counts_i32;       /* [n_routed] tokens per routed expert            */
  int64_t offsets_i32;      /* [n_routed + 1] exclusive prefix sum of counts  */
  int64_t slot_row_i32;     /* [T][top_k] row of token t's k-th expert        */
  int64_t row_src_i32;      /* [T * top_k] source token of each row           */
  int64_t xp;               /* [T * top_k][d] gathered token rows (-1: the
                               expert GEMM gathers rows of x directly)        */
  int64_t h_routed;         /* [T * top_k][inner] silu(W1 u) * (W3 u)         */
  int64_t h_shared;         /* [T][n_shared * shared_inner]                   */
  int64_t y;                /* [T * top_k][d] routed expert outputs: float for
                               fp32 layers; for bf16 layers IEEE half, each
                               64-column group of a row scaled by a power of
                               two (value = half * y_scale)                   */
  int64_t y_scale_f32;      /* [T * top_k][d / 64] those inverse scales (bf16
                               layers; -1 otherwise)                          */
  int64_t s_f32;            /* [T][d] x + sum of shared experts (fp32); -1
                               without shared experts                         */
  int64_t x_q;              /* FP8: [T][d] E4M3 token rows (-1 otherwise)     */
  int64_t x_scale;          /* FP8: [T][d / 128] their scale bytes            */
  int64_t h_routed_scale;   /* FP8: [T * top_k][inner / 128] scale bytes of
                               h_routed (E4M3 codes for FP8 layers)           */
  int64_t h_shared_scale;   /* FP8: [T][n_shared * shared_inner / 128]        */
  int64_t total_bytes;      /* = moe_layer_workspace_size                     */
} moe_workspace_layout_t;

/* Host-only check of a descriptor; no device call.  Returns MOE_OK,
 * MOE_ERR_INVALID_ARG (including desc == NULL) or MOE_ERR_UNSUPPORTED
 * (bf16 needs d, inner and shared_inner to be multiples of 64, FP8 multiples
 * of 128 with d, inner and n_shared * shared_inner at most 8192; fp32 needs
 * multiples of 4; row counts times widths must stay below 2^31). */
moe_status_t moe_layer_validate(const moe_layer_desc_t* desc);

/* Workspace bytes moe_layer_forward needs for `desc` (host-only).  `bytes`
 * must be non-NULL.  Validates desc first. */
moe_status_t moe_layer_workspace_size(const moe_layer_desc_t* desc,
                                      size_t* bytes);

/* Offsets of the intermediates inside the workspace (host-only). */
moe_status_t moe_layer_workspace_layout(const moe_layer_desc_t* desc,
                                        moe_workspace_layout_t* layout);

/* The layer forward pass.
 *   x            [T][d] dtype                        (required if T > 0)
 *   w_gate       [n_routed][d] float                 (required)
 *   logit_bias   [n_routed] float or NULL: added to the gate logits, so it
 *                changes both the choice and the weights
 *   select_bias  [n_routed] float or NULL: added to the scores for choosing
 *                experts only; weights use the unbiased scores
 *   routed       weights of the n_routed routed experts    (required)
 *   shared       weights of the n_shared shared experts (ignored if 0)
 *   out          [T][d] dtype, written; must not overlap x (MOE_ERR_ALIAS)
 *   topk_idx     [T][top_k] int32 or NULL: kept experts, key descending
 *   topk_w       [T][top_k] float or NULL: their gate weights g
 *   expert_counts [n_routed] int32 or NULL: tokens routed to each expert
 *   workspace    device scratch of >= moe_layer_workspace_size bytes,
 *                256-byte aligned; contents on entry are ignored
 *   stream       hipStream_t (NULL = null stream)
 * T == 0 is valid: it enqueues only a kernel that writes zeros to
 * expert_counts (nothing at all when expert_counts is NULL). */
moe_status_t moe_layer_forward(const moe_layer_desc_t* desc, const void* x,
                               const float* w_gate, const float* logit_bias,
                               const float* select_bias,
                               moe_ffn_weights_t routed,
                               moe_ffn_weights_t shared, void* out,
                               int32_t* topk_idx, float* topk_w,
                               int32_t* expert_counts, void* workspace,
                               size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc:
 * moe_layer_forward with the workspace taken from a fixed device buffer of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library, one per device (the library's
 * own static device array; each GPU the library runs on holds it until the
 * process ends; its address is resolved once per device, on the first call
 * there).  Arguments as for moe_layer_forward, without the workspace.  The
 * call allocates nothing and runs every stage in order on `stream` (no side
 * stream).  A layer whose moe_layer_workspace_size exceeds the buffer gets
 * MOE_ERR_SCRATCH before anything is enqueued (16B-shaped layer: up to 1168
 * tokens; V3-shaped: 272).  Every call on a device shares that
 * device's buffer, which keeps the last call's contents (the forward reads
 * nothing it has not written in the same call): calls that overlap in time on
 * one GPU -- concurrent streams or host threads -- race and must be ordered by
 * the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_layer_forward_noalloc(const moe_layer_desc_t* desc, const void* x,
                                       const float* w_gate, const float* logit_bias,
                                       const float* select_bias, moe_ffn_weights_t routed,
                                       moe_ffn_weights_t shared, void* out,
                                       int32_t* topk_idx, float* topk_w,
                                       int32_t* expert_counts, void* stream);

/* Side streams the library currently holds, over all host threads and
 * devices (each is destroyed when the host thread that created it exits).
 * Host-only; for leak checks. */
int32_t moe_side_stream_count(void);

/* Number of kernel stages moe_layer_forward_traced brackets with events,
 * and the name of stage i (NULL if out of range). */
int32_t moe_layer_trace_stage_count(void);
const char* moe_layer_trace_stage_name(int32_t i);

/* moe_layer_forward, with hipEvent_t events[i] recorded on `stream` before
 * stage i and events[n] after the last stage (n = stage count: router, scan,
 * permute, gemm_gateup, gemm_down, combine), so the caller can time every
 * stage (the permute stage is empty when the scan's launch writes the row
 * maps).  `events` holds n + 1 created events (MOE_ERR_INVALID_ARG if
 * n_events is smaller).  The same launches as the untraced call; the
 * results are bitwise equal.  Otherwise identical. */
moe_status_t moe_layer_forward_traced(
    const moe_layer_desc_t* desc, const void* x, const float* w_gate,
    const float* logit_bias, const float* select_bias,
    moe_ffn_weights_t routed, moe_ffn_weights_t shared, void* out,
    int32_t* topk_idx, float* topk_w, int32_t* expert_counts, void* workspace,
    size_t workspace_bytes, void* stream, void* const* events,
    int32_t n_events);

/* Backward pass of a bf16 layer.  The pages train these layers (DeepSeek-V3
 * Technical Report summary, "3.2.1 DualPipe": the chunks' backward for
 * inputs and backward for weights) and print no formula for it: this is the
 * gradient of the layer's forward function (moe_layer_forward with the same
 * desc and inputs) with the expert choice held fixed -- the top-K choice is
 * piecewise constant, and the selection bias is set by the load rule, not by
 * gradients.  For L = sum(dout * out):
 *   dx          [T][d] bf16: dL/dx (residual, shared and routed experts, and
 *               the gate through the scores)
 *   dw_gate     [n_routed][d] fp32: dL/dW_gate
 *   dlogit_bias [n_routed] fp32 or NULL: dL/d logit_bias
 *   d_routed, d_shared: the experts' weight gradients (moe_ffn_grads_t;
 *               d_shared ignored when n_shared = 0); experts that receive no
 *               token get zeros
 *   topk_idx    [T][top_k] int32 or NULL: receives the expert choice used
 *               (recomputed from the inputs; the forward's own choice, as the
 *               router is deterministic)
 * x, w_gate, logit_bias, select_bias, routed, shared: as in the forward;
 * dout [T][d] bf16.  Every product accumulates in fp32; the SwiGLU
 * pre-activations are recomputed rather than stored.  dx must not overlap x
 * or dout (MOE_ERR_ALIAS).  dtype must be MOE_BF16 (MOE_ERR_UNSUPPORTED
 * otherwise).  The workspace (moe_layer_backward_workspace_size bytes,
 * 256-byte aligned) is the caller's; nothing is allocated.  Asynchronous on
 * `stream`; bitwise reproducible. */
moe_status_t moe_layer_backward_workspace_size(const moe_layer_desc_t* desc, size_t* bytes);
moe_status_t moe_layer_backward(const moe_layer_desc_t* desc, const void* x,
                                const float* w_gate, const float* logit_bias,
                                const float* select_bias, moe_ffn_weights_t routed,
                                moe_ffn_weights_t shared, const void* dout, void* dx,
                                float* dw_gate, float* dlogit_bias, moe_ffn_grads_t d_routed,
                                moe_ffn_grads_t d_shared, int32_t* topk_idx, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Number of kernel stages moe_layer_backward_traced brackets with events,
 * and the name of stage i (NULL if out of range). */
int32_t moe_layer_backward_stage_count(void);
const char* moe_layer_backward_stage_name(int32_t i);

/* moe_layer_backward, with hipEvent_t events[i] recorded on `stream` before
 * stage i and events[n] after the last (n = backward stage count); `events`
 * holds n + 1 created events (MOE_ERR_INVALID_ARG if n_events is smaller).
 * Otherwise identical. */
moe_status_t moe_layer_backward_traced(
    const moe_layer_desc_t* desc, const void* x, const float* w_gate,
    const float* logit_bias, const float* select_bias, moe_ffn_weights_t routed,
    moe_ffn_weights_t shared, const void* dout, void* dx, float* dw_gate,
    float* dlogit_bias, moe_ffn_grads_t d_routed, moe_ffn_grads_t d_shared, int32_t* topk_idx,
    void* workspace, size_t workspace_bytes, void* stream, void* const* events,
    int32_t n_events);

/* Weights to the FP8 layer's format: `src` [batch][rows][cols] (src_dtype
 * MOE_F32 or MOE_BF16, device) to E4M3 `codes` (same shape, one byte each)
 * and `scales` [batch][rows / 128][cols / 128]: each 128 x 128 block gets the
 * smallest power of two 2^E with max|v| <= 448 * 2^E (byte E + 127, 127 for
 * an all-zero block) and each value the E4M3 code nearest to v * 2^-E, ties
 * to even.  rows and cols multiples of 128 (MOE_ERR_UNSUPPORTED otherwise);
 * asynchronous on `stream`; allocates nothing. */
moe_status_t moe_quantize_fp8_blocks(const void* src, int32_t src_dtype, int64_t batch,
                                     int32_t rows, int32_t cols, uint8_t* codes,
                                     uint8_t* scales, void* stream);

/* Auxiliary-loss-free load balancing, the step after a training forward pass
 * (DeepSeek-V3 Technical Report summary, "2. Architecture": the per-expert
 * selection bias is updated after each step by whether the expert was over-
 * or underloaded).  With total = sum of counts[0 .. n_routed) (= T * top_k for
 * a dropless forward) and count_e * n_routed compared with total exactly in
 * integers:
 *   select_bias[e] -= gamma  if count_e * n_routed > total  (overloaded)
 *   select_bias[e] += gamma  if count_e * n_routed < total  (underloaded)
 *   unchanged otherwise; each update is one fp32 addition.
 *   rel_load[e] = (float)(count_e * n_routed) / (float)total  (1 = balanced;
 *                 0 when total is 0)
 * counts      [n_routed] int32 device (e.g. the forward's expert_counts), read
 * select_bias [n_routed] float device, updated in place, or NULL
 * rel_load    [n_routed] float device, written, or NULL
 * 1 <= n_routed <= 256 (MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED otherwise),
 * counts non-NULL and gamma finite (MOE_ERR_INVALID_ARG).  Asynchronous on
 * `stream`; allocates nothing. */
moe_status_t moe_bias_update(const int32_t* counts, int32_t n_routed, float gamma,
                             float* select_bias, float* rel_load, void* stream);

/* Static description of a status code. */
const char* moe_strerror(moe_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LAYER_H */
