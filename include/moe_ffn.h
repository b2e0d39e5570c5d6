/*
 * moe_ffn -- sparse shared-expert MoE FFN for AMD Instinct MI355X (gfx950).
 *
 * One layer of the FFN described in "qwen35moe - Forward-Pass Design
 * (Pantheon port)", section "Shared-expert MoE FFN (every layer)":
 *
 *   moe_out = MoE(x; softmax router over 256 experts, top-8 used,
 *                 norm_topk_prob = true, SwiGLU experts)
 *   shexp   = SwiGLU(x; ffn_gate_shexp, ffn_up_shexp, ffn_down_shexp)
 *   sgate   = sigmoid(ffn_gate_inp_shexp . x)           (one scalar per token)
 *   y       = moe_out + sgate * shexp
 *
 * with expert(x) = down(silu(gate(x)) * up(x)) ("SSD Streaming Expert Layers
 * (streaming)", section "Math Contract") and routed expert weights in the
 * 4-bit affine layout of the same page, section "Quantized Layout".  Shapes are
 * those of the "Config" table of the qwen35moe page: n_embd 2048, 256 experts,
 * 8 used, expert FF 512, shared FF 512; quantisation group 64.
 *
 * Conventions of every entry point:
 *   - Plain C ABI; no exception crosses it.  Return 0 (MOE_FFN_OK) or a
 *     negative MOE_FFN_E* status; moe_ffn_status_string names it.
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned, row-major and contiguous.  bf16 values are passed as their
 *     uint16_t bit patterns.  The library never writes an input and never
 *     keeps a pointer after the call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  A call only
 *     enqueues work on it: no host synchronisation, no device allocation.
 *     Faults inside kernels surface as HIP errors at the caller's next
 *     synchronisation, as for any HIP launch.
 *   - Inputs must be finite; NaN and infinite inputs are outside the
 *     contract and are not checked.  Any finite x and weights are accepted:
 *     no intermediate is kept in a type narrower in range than fp32.  The
 *     decode path holds h = silu(gate) * up as two bf16 terms (16
 *     significant bits); the prefill path's fp16 MFMA operands (x, weights,
 *     h, the routed partials) each carry a power-of-two exponent per row
 *     (or row piece) that scales the row's largest magnitude into
 *     [2^14, 2^15) and is re-applied exactly in fp32.  A value far below its
 *     row's largest (under 2^-28 of it) keeps less than fp16 precision.  The
 *     result is only as finite as the fp32 arithmetic of the method: a
 *     logit, gate/up value, h or output beyond the fp32 range gives inf.
 *   - Calls that share a workspace must not overlap in time (same stream, or
 *     ordered by events).
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_FFN_OK 0
#define MOE_FFN_EINVAL (-1)       /* NULL required pointer, T < 0, bad path id, dims NULL */
#define MOE_FFN_EUNSUPPORTED (-2) /* dims differ from the compiled shape, or T too large */
#define MOE_FFN_EALIGN (-3)       /* a pointer is not 16-byte aligned */
#define MOE_FFN_EWORKSPACE (-4)   /* workspace NULL or smaller than moe_ffn_workspace_size */
#define MOE_FFN_EHIP (-5)         /* a kernel launch failed (hipGetLastError) */
#define MOE_FFN_ETOOBIG (-6)      /* T above MOE_FFN_NOALLOC_MAX_T in moe_ffn_forward_noalloc */

/* execution paths (moe_ffn_forward_path) */
/* Routing score (moe_ffn_router.gating). */
#define MOE_FFN_GATING_SOFTMAX 0       /* softmax over the experts, top-k renormalised (qwen35moe) */
#define MOE_FFN_GATING_SQRT_SOFTPLUS 1 /* score sqrt(softplus(logit)) (ds4.c study notes Part 3, MoE
                                          trace 3, router probabilities), top-k renormalised */

#define MOE_FFN_PATH_AUTO 0    /* decode for T <= MOE_FFN_DECODE_MAX_T, else prefill */
#define MOE_FFN_PATH_DECODE 1  /* small-T path: weight-streaming GEMV kernels */
#define MOE_FFN_PATH_PREFILL 2 /* large-T path: routing sort + grouped MFMA GEMMs */

#define MOE_FFN_DECODE_MAX_T 64
#define MOE_FFN_MAX_T (1 << 20)
/* The prefill path runs at most this many tokens per pass; a longer call runs
 * consecutive passes over token slices in the same workspace, so the
 * workspace stops growing at this size.  Tokens are independent and every
 * output row is accumulated in the same order whatever rows share its tile,
 * so the result is the one a single pass would give, bit for bit.  (The
 * qwen35moe page's batched prefill and the Lily engine page both process
 * long prompts in bounded slices.) */
#define MOE_FFN_PREFILL_CHUNK_T 32768

/* Layer shape.  The library is compiled for {2048, 256, 8, 512, 512, 64}
 * (d_model, n_experts, top_k, d_ff, d_ff_shared, group_size) and returns
 * MOE_FFN_EUNSUPPORTED for anything else. */
typedef struct {
    int32_t d_model, n_experts, top_k, d_ff, d_ff_shared, group_size;
} moe_ffn_dims;

/* A 4-bit affine tensor of E stacked matrices [out, in] ("Quantized Layout"):
 *   qweight u32  [E, out, in/8]: element 8j+k of a row is bits 4k..4k+3 of
 *                word j ("low first");
 *   scales  bf16 [E, out, in/64], biases bf16 [E, out, in/64];
 *   W[e, o, i] = scales[e, o, i/64] * q + biases[e, o, i/64]. */
typedef struct {
    const uint32_t *qweight;
    const uint16_t *scales;
    const uint16_t *biases;
} moe_q4_tensor;

/* ffn_{gate,up,down}_exps: gate and up are [E, d_ff, d_model] (out = d_ff),
 * down is [E, d_model, d_ff].
 *
 * gate_up_fused = 1 selects the fused gate/up layout of "SSD Streaming Expert
 * Layers" (section Quantized Layout and its fused-gate_up note): one tensor
 * [E, 2*d_ff, d_model] in `gate` (qweight [E, 2*d_ff, d_model/8], scales and
 * biases [E, 2*d_ff, d_model/64]) in which expert e holds its d_ff gate rows
 * and then its d_ff up rows (rows interleaved per expert, not all experts'
 * gate rows followed by all experts' up rows); `up` must then be all NULL.
 * gate_up_fused = 0 (the zero-initialised default): separate tensors.  Any
 * other value, or `up` pointers given with the fused layout, is
 * MOE_FFN_EINVAL.  Both layouts compute the same values bit for bit. */
typedef struct {
    moe_q4_tensor gate, up, down;
    int32_t gate_up_fused;
} moe_ffn_experts;

/* ffn_gate_inp: weight fp32 [E, d_model]; bias fp32 [E] or NULL, added to the
 * logits before the softmax (it moves both the selection and the weights).
 *
 * weights_scale: the expert_weights_scale of the routed MoE call
 * (qwen35moe Forward-Pass Design, "Shared-expert MoE FFN": gate = softmax,
 * norm_topk_prob, scale = expert_weights_scale): every renormalised routing
 * weight is multiplied by it before it weights its expert's output, and
 * topk_weight reports the product.  0 (the zero-initialised default) is
 * read as 1.  Negative, NaN or infinite values are MOE_FFN_EINVAL. */
typedef struct {
    const float *weight;
    const float *bias;
    float weights_scale;
    /* gating: MOE_FFN_GATING_SOFTMAX (0, the default) or
     * MOE_FFN_GATING_SQRT_SOFTPLUS: score_e = sqrt(softplus(logit_e)) with
     * softplus(z) = log(1 + e^z) computed stably.  Both select the top_k
     * experts by logit (the sqrt-softplus score rises strictly with the
     * logit, so the ranking is the same; ties to the lower index) and weight
     * them by their scores renormalised to sum 1 (for softmax: the selected
     * softmax probabilities), times weights_scale.  Other values are
     * MOE_FFN_EINVAL. */
    int32_t gating;
    /* Hash routing (ds4.c study notes Part 3, MoE trace 3, hash table
     * routing: selected[i] = table[i * n_vocab + token]).  tid2eid: int32
     * [top_k, n_vocab], or NULL (the zero-initialised default) for routing by
     * logit.  With a table, token t's experts are tid2eid[r * n_vocab +
     * token_ids[t]] for r = 0 .. top_k - 1, in that order (a repeated entry
     * is used once per rank), instead of the top_k by logit; their weights
     * are the gating's scores of those experts renormalised to sum 1, times
     * weights_scale (the router logits are still computed for them).
     * token_ids: int32 [T], the call's token ids, required with a table.
     * n_vocab >= 1 with a table.  Entries must lie in [0, n_experts) and ids
     * in [0, n_vocab); values outside are clamped into those ranges (never
     * read out of bounds) and give an unspecified choice of experts.  A
     * table without token ids, or n_vocab < 1, is MOE_FFN_EINVAL. */
    const int32_t *tid2eid;
    const int32_t *token_ids;
    int32_t n_vocab;
} moe_ffn_router;

/* Shared expert, bf16: gate, up [d_ff_shared, d_model]; down [d_model,
 * d_ff_shared]; gate_inp (ffn_gate_inp_shexp) [d_model] or NULL, in which case
 * sgate = 1. */
typedef struct {
    const uint16_t *gate_inp;
    const uint16_t *gate;
    const uint16_t *up;
    const uint16_t *down;
} moe_ffn_shared;

/* Bytes of device workspace a call with T tokens needs (0 for T == 0; 0 for
 * invalid dims or T); the same for every T >= MOE_FFN_PREFILL_CHUNK_T.  The
 * workspace holds the intermediates of the path's steps: routing results,
 * the sort's histograms, offsets and tile map, the gate/up activations and
 * the per-rank partials (the Lily engine page keeps routing on the GPU,
 * section "Palikti ekspertu marsrutizavima GPU", and bounds this
 * intermediate traffic, section "Sumazinti tarpini ir busenos srauta").  The
 * workspace needs no initialisation and carries no state from one call to
 * the next. */
size_t moe_ffn_workspace_size(const moe_ffn_dims *dims, int64_t T);

/* y[T, d_model] bf16 = the FFN above applied to x[T, d_model] bf16.
 *
 * router, experts: required.  shared: NULL means no shared expert (y =
 * moe_out).  topk_idx int32 [T, top_k] and topk_weight fp32 [T, top_k]:
 * optional outputs (NULL to skip): the selected experts in descending logit
 * order (ties to the lower index; table order with hash routing) and their
 * renormalised weights.
 * Routing uses fp32 logits.  y is rounded once, to nearest even.
 * T == 0 returns MOE_FFN_OK without launching anything. */
int moe_ffn_forward(const moe_ffn_dims *dims, int64_t T, const uint16_t *x, const moe_ffn_router *router,
                    const moe_ffn_experts *experts, const moe_ffn_shared *shared, uint16_t *y,
                    int32_t *topk_idx, float *topk_weight, void *workspace, size_t workspace_bytes,
                    void *stream);

/* moe_ffn_forward with the execution path forced (MOE_FFN_PATH_*).  Both
 * paths compute the same function; they differ in kernels and rounding
 * order.  The decode path accepts T <= MOE_FFN_DECODE_MAX_T only. */
int moe_ffn_forward_path(const moe_ffn_dims *dims, int64_t T, const uint16_t *x, const moe_ffn_router *router,
                         const moe_ffn_experts *experts, const moe_ffn_shared *shared, uint16_t *y,
                         int32_t *topk_idx, float *topk_weight, void *workspace, size_t workspace_bytes,
                         void *stream, int path);

/* Kernels a measurement tool can bracket with moe_ffn_forward_traced. */
#define MOE_FFN_KERNEL_ROUTER 1      /* router logits (+ top-8 where fused) */
#define MOE_FFN_KERNEL_EXPERT_GU 2   /* routed expert gate/up projections + SwiGLU */
#define MOE_FFN_KERNEL_EXPERT_DOWN 3 /* routed expert down projection */
#define MOE_FFN_KERNEL_COMBINE 4     /* shared-expert down + combine into y */

typedef struct {
    int32_t kernel; /* MOE_FFN_KERNEL_* */
    void *start;    /* hipEvent_t recorded on `stream` right before that kernel's launch */
    void *stop;     /* hipEvent_t recorded on `stream` right after it */
} moe_ffn_trace;

/* moe_ffn_forward_path that also records trace->start / trace->stop around
 * one kernel of the call, for timing it with hipEventElapsedTime.  The events
 * are caller-owned and created by the caller; trace may be NULL.  Measurement
 * use only: the two event records are the only difference from
 * moe_ffn_forward_path. */
int moe_ffn_forward_traced(const moe_ffn_dims *dims, int64_t T, const uint16_t *x, const moe_ffn_router *router,
                           const moe_ffn_experts *experts, const moe_ffn_shared *shared, uint16_t *y,
                           int32_t *topk_idx, float *topk_weight, void *workspace, size_t workspace_bytes,
                           void *stream, int path, const moe_ffn_trace *trace);

/* ---- The FFN sub-block of a layer, with its boundary steps.
 *
 * "qwen35moe - Forward-Pass Design", section "Block scaffold": every layer is
 * a pre-norm sandwich; the shared-MoE FFN reads the post-attention
 * RMS-normalised stream and its output is added back to the un-normalised
 * stream.  RMS normalisation as in "ds4.c study notes" Part 3, section 3,
 * trace 1: out[i] = x[i] / sqrt(mean(x^2) + eps) * weight[i].  So:
 *
 *   xn = bf16( h * (1 / sqrt(mean(h^2) + eps)) * norm_weight )   (per token)
 *   y  = bf16( h + FFN(xn) )                                     (one rounding)
 *
 * with FFN the function of moe_ffn_forward.  Readings taken where the pages
 * leave a step open: the sum of squares, the scale and each product are
 * computed in double (the pages accumulate in double); the normalised row is
 * rounded once to bf16, the FFN's input type; the FFN output is not rounded
 * before the residual is added.  eps is the
 * caller's (the pages name it but give no value); it must be finite and
 * >= 0.
 *
 * h bf16 [T, d_model]: the residual stream, read only.  norm_weight fp32
 * [d_model] (post_attention_norm), required.  y bf16 [T, d_model] may be h
 * itself (in-place update of the residual stream) but must not overlap it
 * otherwise.  Every other argument, status and the rules of the conventions
 * above are those of moe_ffn_forward_path / moe_ffn_forward_traced. */

/* Bytes of device workspace for moe_ffn_block_forward* with T tokens:
 * moe_ffn_workspace_size plus room for the normalised rows of one pass. */
size_t moe_ffn_block_workspace_size(const moe_ffn_dims *dims, int64_t T);

int moe_ffn_block_forward(const moe_ffn_dims *dims, int64_t T, const uint16_t *h, const float *norm_weight, float eps,
                          const moe_ffn_router *router, const moe_ffn_experts *experts, const moe_ffn_shared *shared,
                          uint16_t *y, int32_t *topk_idx, float *topk_weight, void *workspace, size_t workspace_bytes,
                          void *stream);

/* moe_ffn_block_forward with the execution path forced and an optional
 * trace (both as in moe_ffn_forward_traced). */
int moe_ffn_block_forward_traced(const moe_ffn_dims *dims, int64_t T, const uint16_t *h, const float *norm_weight,
                                 float eps, const moe_ffn_router *router, const moe_ffn_experts *experts,
                                 const moe_ffn_shared *shared, uint16_t *y, int32_t *topk_idx, float *topk_weight,
                                 void *workspace, size_t workspace_bytes, void *stream, int path,
                                 const moe_ffn_trace *trace);

/* ---- Entry point that allocates nothing.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * moe_ffn_forward for 1 <= T <= MOE_FFN_NOALLOC_MAX_T (always the decode
 * path) without a workspace argument: its scratch is a static device array of
 * MOE_FFN_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, which
 * each GPU the library runs on holds until the process ends.  The array's
 * device address is looked up once per device, on the first call made with
 * that device current; make every call with the stream's device current.
 * No call allocates or frees memory.
 *
 * T > MOE_FFN_NOALLOC_MAX_T returns MOE_FFN_ETOOBIG without launching; the
 * other statuses are moe_ffn_forward's (there is no MOE_FFN_EWORKSPACE).
 * Every call on one GPU uses that GPU's one scratch array: calls that may
 * overlap in time on the same GPU (other streams, or host threads without
 * ordering) race on it and must be ordered by the caller.  The scratch
 * needs no clearing: a call writes every scratch element before it reads it,
 * so what a previous call left there does not matter. */
#define MOE_FFN_NOALLOC_MAX_T 64
#define MOE_FFN_NOALLOC_SCRATCH_BYTES (8u << 20)

int moe_ffn_forward_noalloc(const moe_ffn_dims *dims, int64_t T, const uint16_t *x, const moe_ffn_router *router,
                            const moe_ffn_experts *experts, const moe_ffn_shared *shared, uint16_t *y,
                            int32_t *topk_idx, float *topk_weight, void *stream);

/* Static string for a status code.  (The pages define no error reporting;
 * these codes are this boundary's own.) */
const char *moe_ffn_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
