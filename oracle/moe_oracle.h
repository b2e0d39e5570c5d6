/*
 * fp64 CPU oracle of the sparse shared-expert MoE FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code with the GPU library: it has its own bf16 decoding, dequantisation,
 * router, top-k, SwiGLU and combine.
 *
 * What it computes (one token at a time, all in double unless noted):
 *   qwen35moe Forward-Pass Design (Pantheon port), "Shared-expert MoE FFN
 *   (every layer)":
 *     moe_out = MoE(x; softmax router over n_experts, top_k used,
 *                   norm_topk_prob = true; SwiGLU experts)
 *     shexp   = SwiGLU(x; shared gate/up/down)
 *     sgate   = sigmoid(ffn_gate_inp_shexp . x)
 *     out     = moe_out + sgate * shexp
 *   SSD Streaming Expert Layers (edge0), "Math Contract":
 *     expert(x) = down(silu(gate(x)) * up(x))
 *   SSD Streaming Expert Layers (edge0), "Quantized Layout":
 *     expert weights u32 [E, out, in/8], 4-bit affine, group along `in`,
 *     bf16 scales and biases [E, out, in/group].
 *   ds4.c study notes Part 3, section 4 (MoE), trace 3: top-k by strict
 *     ">" so an equal later score never displaces an earlier index.
 *
 * Readings where the pages leave a step open:
 *   - expert_weights_scale is 1.0;
 *   - the router may carry an optional fp32 per-expert offset added to the
 *     logits before softmax (NULL = none);
 *   - the shared-expert gate vector is optional (NULL => sgate = 1), and the
 *     whole shared expert is optional (sh_gate == NULL => no shared term);
 *   - nibble k of word j of a row is element 8j+k, at bits 4k..4k+3;
 *   - a dequantised weight is fp32(s*q + b) with s, b widened from bf16
 *     (s*q is exact in fp32, so exactly one rounding);
 *   - ties in the logits go to the lower expert index, for membership and
 *     order.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int64_t d_model;     /* D */
    int64_t n_experts;   /* E */
    int64_t top_k;       /* k */
    int64_t d_ff;        /* F, routed expert width */
    int64_t d_ff_shared; /* Fs, shared expert width */
    int64_t group_size;  /* g, quantisation group along the input axis */
} moe_oracle_dims;

typedef struct {
    const uint32_t *qweight; /* [E, out, in/8] */
    const uint16_t *scales;  /* bf16 bits [E, out, in/g] */
    const uint16_t *biases;  /* bf16 bits [E, out, in/g] */
} moe_oracle_q4;

typedef struct {
    const float *router_w;        /* [E, D] */
    const float *router_b;        /* [E] or NULL */
    moe_oracle_q4 gate, up;       /* out = F, in = D */
    moe_oracle_q4 down;           /* out = D, in = F */
    const uint16_t *sh_gate_inp;  /* bf16 [D] or NULL */
    const uint16_t *sh_gate;      /* bf16 [Fs, D]; NULL => no shared expert */
    const uint16_t *sh_up;        /* bf16 [Fs, D] */
    const uint16_t *sh_down;      /* bf16 [D, Fs] */
    double weights_scale;         /* expert_weights_scale; 0 is read as 1 */
    int32_t gating;               /* 0: softmax; 1: sqrt(softplus(logit)) scores */
    /* hash routing (ds4.c study notes Part 3, MoE trace 3, hash table
     * routing): when tid2eid != NULL, token t's experts are
     * tid2eid[r * n_vocab + token_ids[t]], r < top_k, in that order, instead
     * of the top_k by logit; the weights are the gating's scores of those
     * experts renormalised (reading: the same step as after a top-k).
     * Entries must lie in [0, n_experts) and ids in [0, n_vocab). */
    const int32_t *tid2eid;       /* [top_k, n_vocab] or NULL */
    int64_t n_vocab;
    const int32_t *token_ids;     /* [T], the call's token ids (with tid2eid) */
} moe_oracle_layer;

enum { MOE_ORACLE_OK = 0, MOE_ORACLE_EINVAL = -1, MOE_ORACLE_ENOMEM = -2 };

/* bf16 bit pattern -> fp32 (exact). */
float moe_oracle_bf16_to_f32(uint16_t bits);

/* Row `row` of matrix `expert` of a 4-bit tensor with shape [E, out_dim,
 * in_dim], dequantised to fp32 into dst[in_dim]. */
void moe_oracle_dequant_row(const moe_oracle_q4 *w, int64_t expert, int64_t out_dim, int64_t in_dim,
                            int64_t group, int64_t row, float *dst);

/* Router logits of one token: l[e] = sum_i Wr[e,i] x[i] (+ b[e]). */
void moe_oracle_router_logits(const moe_oracle_dims *d, const moe_oracle_layer *L, const uint16_t *x_row,
                              double *logits);

/* Top-k of E logits ordered by (logit desc, index asc); softmax over all E,
 * then the k selected probabilities renormalised to sum to 1.  margin =
 * logit of the k-th selected minus the best unselected (+inf if k == E). */
int moe_oracle_select(const double *logits, int64_t E, int64_t k, int32_t *sel, double *w, double *margin);

/* One routed expert on one token: out[D] = down(silu(gate x) * up x). */
void moe_oracle_expert(const moe_oracle_dims *d, const moe_oracle_layer *L, int64_t e, const double *xd,
                       double *out);

/* Shared expert on one token: out[D] = SwiGLU_shared(x), *sgate = gate or 1. */
void moe_oracle_shared(const moe_oracle_dims *d, const moe_oracle_layer *L, const double *xd, double *out,
                       double *sgate);

/* Whole FFN on the tokens listed in tokens[n_tok] (all T tokens, in order,
 * when tokens == NULL; then n_tok must equal T).  Outputs per listed token:
 * y[n_tok, D] (fp64, not rounded), idx[n_tok, k], w[n_tok, k],
 * margin[n_tok]; any output pointer except y may be NULL; logits[n_tok, E]
 * optional.  nthreads <= 0 means one thread. */
int moe_oracle_forward(const moe_oracle_dims *d, const moe_oracle_layer *L, int64_t T, const uint16_t *x,
                       const int64_t *tokens, int64_t n_tok, double *y, int32_t *idx, double *w, double *margin,
                       double *logits, int nthreads);

/* Routing only (logits, selection, weights, margin) for the listed tokens;
 * same conventions as moe_oracle_forward. */
int moe_oracle_route(const moe_oracle_dims *d, const moe_oracle_layer *L, int64_t T, const uint16_t *x,
                     const int64_t *tokens, int64_t n_tok, int32_t *idx, double *w, double *margin, double *logits,
                     int nthreads);

/* The FFN sub-block with its boundary steps.  qwen35moe page, "Block
 * scaffold": the FFN reads the RMS-normalised stream and its output is added
 * to the un-normalised input.  ds4.c study notes Part 3, section 3, trace 1:
 * out[i] = x[i] / sqrt(mean(x^2) + eps) * weight[i], squares summed in
 * double.  Readings: everything in double here, and the normalised row is
 * rounded once to bf16 (to nearest, ties to even), the FFN's input type.
 *
 * moe_oracle_rmsnorm_bf16: one row of n bf16 values -> n bf16 values. */
void moe_oracle_rmsnorm_bf16(const uint16_t *x_row, const float *weight, int64_t n, double eps, uint16_t *out_row);

/* y = h + FFN(xn) in double (not rounded) for the listed tokens, with xn the
 * rows of moe_oracle_rmsnorm_bf16(h); idx, w, margin, logits as in
 * moe_oracle_forward (of xn).  xn (optional, [T, D] bf16) receives every
 * normalised row. */
int moe_oracle_block_forward(const moe_oracle_dims *d, const moe_oracle_layer *L, int64_t T, const uint16_t *h,
                             const float *norm_w, double eps, const int64_t *tokens, int64_t n_tok, uint16_t *xn,
                             double *y, int32_t *idx, double *w, double *margin, double *logits, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
