/*
 * fp64 CPU oracle of the sparse shared-expert MoE FFN -- TEST INFRASTRUCTURE.
 * See moe_oracle.h for what is computed, the sources on the pages and the
 * readings taken where they are silent.  Deliberately plain: no blocking, no
 * fusion, no reordering; one token at a time.  Built with -ffp-contract=off
 * so every fp32 operation rounds as written.
 */
#include "moe_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

float moe_oracle_bf16_to_f32(uint16_t bits) {
    /* bf16 is the upper half of an fp32 bit pattern */
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* SSD Streaming Expert Layers (edge0), "Quantized Layout": packed u32
 * [E, out, in/8], 4-bit affine with one bf16 scale and bias per group of
 * `group` inputs.  W[i] = s * q[i] + b. */
void moe_oracle_dequant_row(const moe_oracle_q4 *w, int64_t expert, int64_t out_dim, int64_t in_dim,
                            int64_t group, int64_t row, float *dst) {
    const int64_t words = in_dim / 8, groups = in_dim / group;
    const uint32_t *q = w->qweight + (expert * out_dim + row) * words;
    const uint16_t *sc = w->scales + (expert * out_dim + row) * groups;
    const uint16_t *bi = w->biases + (expert * out_dim + row) * groups;
    for (int64_t i = 0; i < in_dim; i++) {
        uint32_t nib = (q[i / 8] >> (4 * (i % 8))) & 15u;
        float s = moe_oracle_bf16_to_f32(sc[i / group]);
        float b = moe_oracle_bf16_to_f32(bi[i / group]);
        dst[i] = s * (float)nib + b;
    }
}

/* qwen35moe Forward-Pass Design, "Shared-expert MoE FFN": the router is
 * ffn_gate_inp . x, one logit per expert. */
void moe_oracle_router_logits(const moe_oracle_dims *d, const moe_oracle_layer *L, const uint16_t *x_row,
                              double *logits) {
    for (int64_t e = 0; e < d->n_experts; e++) {
        double acc = 0.0;
        for (int64_t i = 0; i < d->d_model; i++)
            acc += (double)L->router_w[e * d->d_model + i] * (double)moe_oracle_bf16_to_f32(x_row[i]);
        if (L->router_b) acc += (double)L->router_b[e];
        logits[e] = acc;
    }
}

/* Selection: gate = SOFTMAX over all experts, top_k used, norm_topk_prob =
 * TRUE (qwen35moe Forward-Pass Design, "Shared-expert MoE FFN" and
 * "Correctness watch-list").  Ranking by strict ">" scanning indices upwards,
 * so the lower index wins a tie (ds4.c notes Part 3, MoE trace 3, top-k). */
int moe_oracle_select(const double *logits, int64_t E, int64_t k, int32_t *sel, double *w, double *margin) {
    if (E <= 0 || k <= 0 || k > E) return MOE_ORACLE_EINVAL;
    unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
    if (!taken) return MOE_ORACLE_ENOMEM;
    for (int64_t r = 0; r < k; r++) {
        int64_t best = -1;
        for (int64_t e = 0; e < E; e++)
            if (!taken[e] && (best < 0 || logits[e] > logits[best])) best = e;
        taken[best] = 1;
        sel[r] = (int32_t)best;
    }
    if (margin) {
        int64_t next = -1;
        for (int64_t e = 0; e < E; e++)
            if (!taken[e] && (next < 0 || logits[e] > logits[next])) next = e;
        *margin = next < 0 ? INFINITY : logits[sel[k - 1]] - logits[next];
    }
    free(taken);
    /* softmax over all E experts */
    double mx = logits[0];
    for (int64_t e = 1; e < E; e++)
        if (logits[e] > mx) mx = logits[e];
    double z = 0.0;
    for (int64_t e = 0; e < E; e++) z += exp(logits[e] - mx);
    /* renormalise the selected probabilities */
    double ps = 0.0;
    for (int64_t r = 0; r < k; r++) ps += exp(logits[sel[r]] - mx) / z;
    for (int64_t r = 0; r < k; r++) w[r] = (exp(logits[sel[r]] - mx) / z) / ps;
    return MOE_ORACLE_OK;
}

/* The routed MoE call scales the renormalised weights by
 * expert_weights_scale (qwen35moe Forward-Pass Design, "Shared-expert MoE
 * FFN"); 0 stands for the unscaled default 1. */
static double weights_scale(const moe_oracle_layer *L) { return L->weights_scale == 0.0 ? 1.0 : L->weights_scale; }

/* log(softplus(z)), softplus(z) = log(1 + e^z) written as max(z, 0) +
 * log1p(e^-|z|) (the same value, no overflow).  Below z = -30, softplus(z)
 * = e^z (1 - e^z / 2 + O(e^2z)), so its log is z + log1p(-e^z / 2) to
 * double precision, with no underflow however negative z is. */
static double log_softplus(double z) {
    if (z > -30.0) return log(fmax(z, 0.0) + log1p(exp(-fabs(z))));
    return z + log1p(-0.5 * exp(z));
}

/* sqrt-softplus gating (ds4.c notes Part 3, MoE trace 3, router
 * probabilities): score = sqrt(softplus(logit)).  The score rises strictly
 * with the logit, so the experts chosen by logit are the experts chosen by
 * score; their scores are renormalised to sum 1 (the weight step is not
 * printed for this router: the reading taken is the renormalisation used
 * with the softmax gate).  The ratio score_r / sum(score) is formed from
 * log scores, 0.5 log softplus(z), relative to the largest: the same value,
 * and defined where every score underflows (logits below about -1500). */
static void sqrt_softplus_weights(const double *logits, const int32_t *sel, int64_t k, double *w) {
    double mx = -INFINITY;
    for (int64_t r = 0; r < k; r++) {
        w[r] = 0.5 * log_softplus(logits[sel[r]]);
        if (w[r] > mx) mx = w[r];
    }
    double s = 0.0;
    for (int64_t r = 0; r < k; r++) {
        w[r] = exp(w[r] - mx);
        s += w[r];
    }
    for (int64_t r = 0; r < k; r++) w[r] /= s;
}

/* Softmax over all E logits, then the probabilities of the k listed
 * experts renormalised to sum 1 (norm_topk_prob): the weights of experts
 * chosen by a table rather than by their logits. */
static void softmax_weights(const double *logits, int64_t E, const int32_t *sel, int64_t k, double *w) {
    double top = logits[0];
    for (int64_t e = 1; e < E; e++)
        if (logits[e] > top) top = logits[e];
    double norm = 0.0;
    for (int64_t e = 0; e < E; e++) norm += exp(logits[e] - top);
    double chosen = 0.0;
    for (int64_t r = 0; r < k; r++) chosen += exp(logits[sel[r]] - top) / norm;
    for (int64_t r = 0; r < k; r++) w[r] = (exp(logits[sel[r]] - top) / norm) / chosen;
}

/* The routing of token t from its logits: the experts (by logit, or by the
 * hash table: ds4.c notes Part 3, MoE trace 3 looks them up as
 * table[r * n_vocab + token]), their renormalised weights under the layer's
 * gating, times expert_weights_scale; margin as moe_oracle_select's (+inf
 * for table routing, whose choice does not depend on the logits). */
static int route_token(const moe_oracle_dims *d, const moe_oracle_layer *L, int64_t t, const double *lg, int32_t *sel,
                       double *ww, double *mg) {
    const int64_t E = d->n_experts, k = d->top_k;
    int st = MOE_ORACLE_OK;
    if (L->tid2eid) {
        for (int64_t r = 0; r < k; r++) sel[r] = L->tid2eid[r * L->n_vocab + L->token_ids[t]];
        softmax_weights(lg, E, sel, k, ww);
        *mg = INFINITY;
    } else {
        st = moe_oracle_select(lg, E, k, sel, ww, mg);
    }
    if (L->gating == 1) sqrt_softplus_weights(lg, sel, k, ww);
    for (int64_t r = 0; r < k; r++) ww[r] *= weights_scale(L);
    return st;
}

/* silu(z) = z * sigmoid(z) (ds4.c notes Part 3, MoE trace 1). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* SSD Streaming Expert Layers (edge0), "Math Contract":
 * expert(x) = down(silu(gate(x)) * up(x)). */
void moe_oracle_expert(const moe_oracle_dims *d, const moe_oracle_layer *L, int64_t e, const double *xd,
                       double *out) {
    const int64_t D = d->d_model, F = d->d_ff, g = d->group_size;
    float *row = (float *)malloc(sizeof(float) * (size_t)(D > F ? D : F));
    double *h = (double *)malloc(sizeof(double) * (size_t)F);
    for (int64_t j = 0; j < F; j++) {
        double gj = 0.0, uj = 0.0;
        moe_oracle_dequant_row(&L->gate, e, F, D, g, j, row);
        for (int64_t i = 0; i < D; i++) gj += (double)row[i] * xd[i];
        moe_oracle_dequant_row(&L->up, e, F, D, g, j, row);
        for (int64_t i = 0; i < D; i++) uj += (double)row[i] * xd[i];
        h[j] = silu(gj) * uj;
    }
    for (int64_t o = 0; o < D; o++) {
        double acc = 0.0;
        moe_oracle_dequant_row(&L->down, e, D, F, g, o, row);
        for (int64_t j = 0; j < F; j++) acc += (double)row[j] * h[j];
        out[o] = acc;
    }
    free(h);
    free(row);
}

/* qwen35moe Forward-Pass Design, "Shared-expert MoE FFN":
 * shexp = SwiGLU(x, ffn_gate_shexp, ffn_up_shexp, ffn_down_shexp),
 * sgate = sigmoid(ffn_gate_inp_shexp . x).  Weights are bf16, widened
 * exactly. */
void moe_oracle_shared(const moe_oracle_dims *d, const moe_oracle_layer *L, const double *xd, double *out,
                       double *sgate) {
    const int64_t D = d->d_model, Fs = d->d_ff_shared;
    double *h = (double *)malloc(sizeof(double) * (size_t)Fs);
    for (int64_t j = 0; j < Fs; j++) {
        double gj = 0.0, uj = 0.0;
        for (int64_t i = 0; i < D; i++) {
            gj += (double)moe_oracle_bf16_to_f32(L->sh_gate[j * D + i]) * xd[i];
            uj += (double)moe_oracle_bf16_to_f32(L->sh_up[j * D + i]) * xd[i];
        }
        h[j] = silu(gj) * uj;
    }
    for (int64_t o = 0; o < D; o++) {
        double acc = 0.0;
        for (int64_t j = 0; j < Fs; j++) acc += (double)moe_oracle_bf16_to_f32(L->sh_down[o * Fs + j]) * h[j];
        out[o] = acc;
    }
    if (L->sh_gate_inp) {
        double z = 0.0;
        for (int64_t i = 0; i < D; i++) z += (double)moe_oracle_bf16_to_f32(L->sh_gate_inp[i]) * xd[i];
        *sgate = 1.0 / (1.0 + exp(-z));
    } else {
        *sgate = 1.0;
    }
    free(h);
}

/* A hash table with its token ids, every entry an expert and every id a
 * column of the table (or no table). */
static int hash_table_ok(const moe_oracle_dims *d, const moe_oracle_layer *L, int64_t T) {
    if (!L->tid2eid) return 1;
    if (!L->token_ids || L->n_vocab < 1) return 0;
    for (int64_t i = 0; i < d->top_k * L->n_vocab; i++)
        if (L->tid2eid[i] < 0 || L->tid2eid[i] >= d->n_experts) return 0;
    for (int64_t t = 0; t < T; t++)
        if (L->token_ids[t] < 0 || L->token_ids[t] >= L->n_vocab) return 0;
    return 1;
}

/* ------------------------------------------------------------- forward */
typedef struct {
    const moe_oracle_dims *d;
    const moe_oracle_layer *L;
    const uint16_t *x;
    const int64_t *tokens;
    double *y, *w, *margin, *logits;
    int32_t *idx;
    int64_t lo, hi;
    int status;
} fwd_job;

static int forward_one(const fwd_job *j, int64_t n) {
    const moe_oracle_dims *d = j->d;
    const int64_t D = d->d_model, E = d->n_experts, k = d->top_k;
    const int64_t t = j->tokens ? j->tokens[n] : n;
    const uint16_t *xr = j->x + t * D;
    double *xd = (double *)malloc(sizeof(double) * (size_t)D);
    double *lg = (double *)malloc(sizeof(double) * (size_t)E);
    double *eo = (double *)malloc(sizeof(double) * (size_t)D);
    double *ww = (double *)malloc(sizeof(double) * (size_t)k);
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    double mg = 0.0, sg = 1.0;
    int st = (xd && lg && eo && ww && sel) ? MOE_ORACLE_OK : MOE_ORACLE_ENOMEM;
    if (st == MOE_ORACLE_OK) {
        for (int64_t i = 0; i < D; i++) xd[i] = (double)moe_oracle_bf16_to_f32(xr[i]);
        moe_oracle_router_logits(d, j->L, xr, lg);
        st = route_token(d, j->L, t, lg, sel, ww, &mg);
    }
    if (st == MOE_ORACLE_OK) {
        double *yr = j->y + n * D;
        for (int64_t o = 0; o < D; o++) yr[o] = 0.0;
        /* moe_out = sum over the selected experts, in rank order, of
         * weight * expert(x) */
        for (int64_t r = 0; r < k; r++) {
            moe_oracle_expert(d, j->L, sel[r], xd, eo);
            for (int64_t o = 0; o < D; o++) yr[o] += ww[r] * eo[o];
        }
        /* out = moe_out + sgate * shexp */
        if (j->L->sh_gate) {
            moe_oracle_shared(d, j->L, xd, eo, &sg);
            for (int64_t o = 0; o < D; o++) yr[o] += sg * eo[o];
        }
        if (j->idx)
            for (int64_t r = 0; r < k; r++) j->idx[n * k + r] = sel[r];
        if (j->w)
            for (int64_t r = 0; r < k; r++) j->w[n * k + r] = ww[r];
        if (j->margin) j->margin[n] = mg;
        if (j->logits)
            for (int64_t e = 0; e < E; e++) j->logits[n * E + e] = lg[e];
    }
    free(xd); free(lg); free(eo); free(ww); free(sel);
    return st;
}

static void *forward_range(void *p) {
    fwd_job *j = (fwd_job *)p;
    for (int64_t n = j->lo; n < j->hi && j->status == MOE_ORACLE_OK; n++) j->status = forward_one(j, n);
    return NULL;
}

int moe_oracle_forward(const moe_oracle_dims *d, const moe_oracle_layer *L, int64_t T, const uint16_t *x,
                       const int64_t *tokens, int64_t n_tok, double *y, int32_t *idx, double *w, double *margin,
                       double *logits, int nthreads) {
    if (!d || !L || !y || (!x && n_tok > 0) || T < 0 || n_tok < 0) return MOE_ORACLE_EINVAL;
    if (d->d_model <= 0 || d->n_experts <= 0 || d->top_k <= 0 || d->top_k > d->n_experts || d->d_ff <= 0 ||
        d->group_size <= 0 || d->group_size % 8 != 0 || d->d_model % d->group_size != 0 ||
        d->d_ff % d->group_size != 0)
        return MOE_ORACLE_EINVAL;
    if (!L->router_w || !L->gate.qweight || !L->up.qweight || !L->down.qweight) return MOE_ORACLE_EINVAL;
    if (L->sh_gate && (!L->sh_up || !L->sh_down || d->d_ff_shared <= 0)) return MOE_ORACLE_EINVAL;
    if (!tokens && n_tok != T) return MOE_ORACLE_EINVAL;
    if (tokens)
        for (int64_t n = 0; n < n_tok; n++)
            if (tokens[n] < 0 || tokens[n] >= T) return MOE_ORACLE_EINVAL;
    if (!hash_table_ok(d, L, T)) return MOE_ORACLE_EINVAL;
    if (n_tok == 0) return MOE_ORACLE_OK;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > n_tok) nthreads = (int)n_tok;
    fwd_job jobs[256];
    pthread_t th[256];
    int joinable[256];
    int64_t chunk = (n_tok + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; t++) {
        int64_t lo = t * chunk, hi = lo + chunk < n_tok ? lo + chunk : n_tok;
        jobs[t] = (fwd_job){d, L, x, tokens, y, w, margin, logits, idx, lo, hi < lo ? lo : hi, MOE_ORACLE_OK};
        joinable[t] = 0;
        if (nthreads > 1 && pthread_create(&th[t], NULL, forward_range, &jobs[t]) == 0) joinable[t] = 1;
        else forward_range(&jobs[t]);
    }
    int st = MOE_ORACLE_OK;
    for (int t = 0; t < nthreads; t++) {
        if (joinable[t]) pthread_join(th[t], NULL);
        if (jobs[t].status != MOE_ORACLE_OK) st = jobs[t].status;
    }
    return st;
}

/* ------------------------------------------------------------- routing only */
typedef struct {
    const moe_oracle_dims *d;
    const moe_oracle_layer *L;
    const uint16_t *x;
    const int64_t *tokens;
    int32_t *idx;
    double *w, *margin, *logits;
    int64_t lo, hi;
    int status;
} route_job;

static void *route_range(void *p) {
    route_job *j = (route_job *)p;
    const int64_t D = j->d->d_model, E = j->d->n_experts, k = j->d->top_k;
    double *lg = (double *)malloc(sizeof(double) * (size_t)E);
    double *ww = (double *)malloc(sizeof(double) * (size_t)k);
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    if (!lg || !ww || !sel) j->status = MOE_ORACLE_ENOMEM;
    for (int64_t n = j->lo; n < j->hi && j->status == MOE_ORACLE_OK; n++) {
        const int64_t t = j->tokens ? j->tokens[n] : n;
        double mg = 0.0;
        moe_oracle_router_logits(j->d, j->L, j->x + t * D, lg);
        j->status = route_token(j->d, j->L, t, lg, sel, ww, &mg);
        if (j->idx) for (int64_t r = 0; r < k; r++) j->idx[n * k + r] = sel[r];
        if (j->w) for (int64_t r = 0; r < k; r++) j->w[n * k + r] = ww[r];
        if (j->margin) j->margin[n] = mg;
        if (j->logits) for (int64_t e = 0; e < E; e++) j->logits[n * E + e] = lg[e];
    }
    free(lg); free(ww); free(sel);
    return NULL;
}

int moe_oracle_route(const moe_oracle_dims *d, const moe_oracle_layer *L, int64_t T, const uint16_t *x,
                     const int64_t *tokens, int64_t n_tok, int32_t *idx, double *w, double *margin, double *logits,
                     int nthreads) {
    if (!d || !L || !L->router_w || (!x && n_tok > 0) || T < 0 || n_tok < 0) return MOE_ORACLE_EINVAL;
    if (d->n_experts <= 0 || d->top_k <= 0 || d->top_k > d->n_experts || d->d_model <= 0) return MOE_ORACLE_EINVAL;
    if (!tokens && n_tok != T) return MOE_ORACLE_EINVAL;
    if (tokens)
        for (int64_t n = 0; n < n_tok; n++)
            if (tokens[n] < 0 || tokens[n] >= T) return MOE_ORACLE_EINVAL;
    if (!hash_table_ok(d, L, T)) return MOE_ORACLE_EINVAL;
    if (n_tok == 0) return MOE_ORACLE_OK;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > n_tok) nthreads = (int)n_tok;
    route_job jobs[256];
    pthread_t th[256];
    int joinable[256];
    int64_t chunk = (n_tok + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; t++) {
        int64_t lo = t * chunk, hi = lo + chunk < n_tok ? lo + chunk : n_tok;
        jobs[t] = (route_job){d, L, x, tokens, idx, w, margin, logits, lo, hi < lo ? lo : hi, MOE_ORACLE_OK};
        joinable[t] = 0;
        if (nthreads > 1 && pthread_create(&th[t], NULL, route_range, &jobs[t]) == 0) joinable[t] = 1;
        else route_range(&jobs[t]);
    }
    int st = MOE_ORACLE_OK;
    for (int t = 0; t < nthreads; t++) {
        if (joinable[t]) pthread_join(th[t], NULL);
        if (jobs[t].status != MOE_ORACLE_OK) st = jobs[t].status;
    }
    return st;
}

/* ------------------------------------------------------- block boundary */
/* Nearest bf16 of a double, ties to even; bf16 keeps 8 significant bits and
 * the fp32 exponent range (subnormals down to 2^-133). */
static uint16_t f64_to_bf16(double v) {
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    const double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a) || isnan(a)) return isnan(a) ? 0x7fc0u : (uint16_t)(sign | 0x7f80u);
    double r;
    if (a < ldexp(1.0, -126)) {
        r = ldexp(rint(ldexp(a, 133)), -133); /* subnormal step 2^-133 */
    } else {
        int e;
        const double m = frexp(a, &e);        /* a = m * 2^e, m in [0.5, 1) */
        r = ldexp(rint(ldexp(m, 8)), e - 8);  /* 8 significant bits; rint: ties to even */
    }
    if (r > ldexp(2.0 - ldexp(1.0, -7), 127)) return (uint16_t)(sign | 0x7f80u); /* past the largest bf16 */
    const float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

void moe_oracle_rmsnorm_bf16(const uint16_t *x_row, const float *weight, int64_t n, double eps, uint16_t *out_row) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; i++) {
        const double v = (double)moe_oracle_bf16_to_f32(x_row[i]);
        ss += v * v;
    }
    const double scale = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; i++)
        out_row[i] = f64_to_bf16((double)moe_oracle_bf16_to_f32(x_row[i]) * scale * (double)weight[i]);
}

int moe_oracle_block_forward(const moe_oracle_dims *d, const moe_oracle_layer *L, int64_t T, const uint16_t *h,
                             const float *norm_w, double eps, const int64_t *tokens, int64_t n_tok, uint16_t *xn,
                             double *y, int32_t *idx, double *w, double *margin, double *logits, int nthreads) {
    if (!d || !norm_w || (!h && T > 0) || T < 0 || !(eps >= 0.0)) return MOE_ORACLE_EINVAL;
    const int64_t D = d->d_model;
    uint16_t *xr = xn ? xn : (uint16_t *)calloc((size_t)(T > 0 ? T * D : 1), sizeof(uint16_t));
    if (!xr) return MOE_ORACLE_EINVAL;
    for (int64_t t = 0; t < T; t++) moe_oracle_rmsnorm_bf16(h + t * D, norm_w, D, eps, xr + t * D);
    int st = moe_oracle_forward(d, L, T, xr, tokens, n_tok, y, idx, w, margin, logits, nthreads);
    if (st == MOE_ORACLE_OK)
        for (int64_t n = 0; n < n_tok; n++) {
            const int64_t t = tokens ? tokens[n] : n;
            for (int64_t o = 0; o < D; o++) y[n * D + o] += (double)moe_oracle_bf16_to_f32(h[t * D + o]);
        }
    if (!xn) free(xr);
    return st;
}
