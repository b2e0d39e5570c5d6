/*
 * Seeded synthetic inputs for the sparse shared-expert MoE FFN.
 *
 * This module only draws and encodes inputs.  It computes nothing the FFN
 * computes: no router logits, no dequantisation, no SwiGLU.  Both the fp64
 * oracle and the GPU library consume the bytes it writes.
 *
 * Random numbers: splitmix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; the 64-bit finaliser as
 * published by Vigna) used as a counter-based generator.  The n-th draw of
 * stream `key` is mix64(key + (n + 1) * GOLDEN), i.e. the n-th output of a
 * splitmix64 whose state starts at `key`.  Because every element has its own
 * counter, any slice can be generated independently and in parallel.
 *
 * Normals: Box-Muller in fp32 on two 24-bit uniforms taken from one 64-bit
 * draw (bits 40..63 and 8..31); draw p yields elements 2p (cosine branch) and
 * 2p+1 (sine branch).
 *
 * 4-bit affine encoding, group g along the input axis (the layout of the
 * edge0 streaming page, "Quantized Layout": u32 [.., out, in/8], bf16 scales
 * and biases [.., out, in/g]):
 *   s = bf16_rne((max - min) / 15)   (the division in fp32)
 *   b = bf16_rne(min)
 *   q = clamp(round_half_even((w - b) / s), 0, 15), q = 0 when s == 0
 *   element 8*j + k of a row sits in bits 4k..4k+3 of word j ("low first").
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Stream key for (seed, tensor id, sub-stream). */
uint64_t synth_key(uint64_t seed, uint32_t tensor, uint32_t stream) {
    uint64_t k = mix64(seed + GOLDEN);
    k = mix64(k ^ ((uint64_t)tensor * 0xD1B54A32D192ED03ULL));
    k = mix64(k ^ ((uint64_t)stream * 0x8CB92BA72F3D8DD7ULL));
    return k;
}

uint64_t synth_draw(uint64_t key, uint64_t n) { return mix64(key + (n + 1) * GOLDEN); }

/* Standard normals for elements [start, start+n) of stream `key`, scaled by
 * sd and rounded to fp32.  Both branches of a Box-Muller pair are used. */
static void fill_normal(uint64_t key, uint64_t start, int64_t n, double sd, float *out) {
    uint64_t end = start + (uint64_t)n;
    for (uint64_t p = start >> 1; 2 * p < end; p++) {
        uint64_t d = synth_draw(key, p);
        /* uniforms in (0,1) with 24-bit resolution, never 0 */
        float u1 = ((float)(uint32_t)(d >> 40) + 0.5f) * (1.0f / 16777216.0f);
        float u2 = ((float)(uint32_t)((d >> 8) & 0xffffffu) + 0.5f) * (1.0f / 16777216.0f);
        float r = (float)sd * sqrtf(-2.0f * logf(u1)), sn, cs;
        sincosf(6.2831853f * u2, &sn, &cs);
        uint64_t i0 = 2 * p, i1 = 2 * p + 1;
        if (i0 >= start) out[i0 - start] = r * cs;
        if (i1 >= start && i1 < end) out[i1 - start] = r * sn;
    }
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40); /* quiet NaN */
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t synth_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

/* ---- generic parallel-for over [0, n) in contiguous chunks ---- */
typedef void (*range_fn)(void *ctx, int64_t lo, int64_t hi);
typedef struct { range_fn fn; void *ctx; int64_t lo, hi; } range_job;
static void *range_thread(void *p) {
    range_job *j = (range_job *)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}
static void parallel_for(int64_t n, int nthreads, range_fn fn, void *ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > n) nthreads = (int)(n > 0 ? n : 1);
    if (nthreads == 1) { fn(ctx, 0, n); return; }
    pthread_t th[256];
    int joinable[256];
    range_job jobs[256];
    int64_t chunk = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; t++) {
        int64_t lo = t * chunk, hi = lo + chunk < n ? lo + chunk : n;
        joinable[t] = 0;
        if (lo >= hi) continue;
        jobs[t] = (range_job){fn, ctx, lo, hi};
        if (pthread_create(&th[t], NULL, range_thread, &jobs[t]) == 0) joinable[t] = 1;
        else fn(ctx, lo, hi);
    }
    for (int t = 0; t < nthreads; t++)
        if (joinable[t]) pthread_join(th[t], NULL);
}

/* ---- plain normal tensors ---- */
typedef struct { uint64_t key, start; double sd; uint16_t *bf; float *f32; } normal_ctx;
static void normal_range(void *p, int64_t lo, int64_t hi) {
    normal_ctx *c = (normal_ctx *)p;
    enum { CH = 4096 };
    float buf[CH];
    for (int64_t i = lo; i < hi; i += CH) {
        int64_t m = hi - i < CH ? hi - i : CH;
        fill_normal(c->key, c->start + (uint64_t)i, m, c->sd, buf);
        for (int64_t j = 0; j < m; j++) {
            if (c->bf) c->bf[i + j] = f32_to_bf16_rne(buf[j]);
            else c->f32[i + j] = buf[j];
        }
    }
}

/* out[i] = bf16_rne(float(sd * N(element start+i))) */
void synth_normal_bf16(uint64_t seed, uint32_t tensor, uint32_t stream, uint64_t start, int64_t n,
                       double sd, uint16_t *out, int nthreads) {
    normal_ctx c = {synth_key(seed, tensor, stream), start, sd, out, NULL};
    parallel_for(n, nthreads, normal_range, &c);
}

/* out[i] = float(sd * N(element start+i)) */
void synth_normal_f32(uint64_t seed, uint32_t tensor, uint32_t stream, uint64_t start, int64_t n,
                      double sd, float *out, int nthreads) {
    normal_ctx c = {synth_key(seed, tensor, stream), start, sd, NULL, out};
    parallel_for(n, nthreads, normal_range, &c);
}

/* ---- activations with per-row redraw counters ----
 * Row t of x uses sub-stream redraw[t] (0 when redraw is NULL) and element
 * counters t*D + c, so a row can be redrawn without touching the others. */
typedef struct { uint64_t seed; uint32_t tensor; int64_t D; const uint32_t *redraw; double sd; uint16_t *x; } xrows_ctx;
static void xrows_range(void *p, int64_t lo, int64_t hi) {
    xrows_ctx *c = (xrows_ctx *)p;
    for (int64_t t = lo; t < hi; t++) {
        uint32_t r = c->redraw ? c->redraw[t] : 0;
        uint64_t key = synth_key(c->seed, c->tensor, r);
        float *buf = (float *)malloc(sizeof(float) * (size_t)c->D);
        fill_normal(key, (uint64_t)(t * c->D), c->D, c->sd, buf);
        for (int64_t j = 0; j < c->D; j++) c->x[t * c->D + j] = f32_to_bf16_rne(buf[j]);
        free(buf);
    }
}
void synth_x_rows(uint64_t seed, uint32_t tensor, int64_t T, int64_t D, const uint32_t *redraw, double sd,
                  uint16_t *x, int nthreads) {
    xrows_ctx c = {seed, tensor, D, redraw, sd, x};
    parallel_for(T, nthreads, xrows_range, &c);
}

/* ---- 4-bit affine matrices ----
 * nmat stacked matrices of rows x cols; fp32 weights sd*N(element), element
 * index (m*rows + r)*cols + c of stream 0, then encoded per row and group. */
typedef struct {
    uint64_t key; int64_t rows_total, cols, group; double sd;
    uint32_t *qw; uint16_t *sc, *bi;
} q4_ctx;
static void q4_range(void *p, int64_t lo, int64_t hi) {
    q4_ctx *c = (q4_ctx *)p;
    float *w = (float *)malloc(sizeof(float) * (size_t)c->cols);
    int64_t ng = c->cols / c->group;
    for (int64_t r = lo; r < hi; r++) {
        fill_normal(c->key, (uint64_t)(r * c->cols), c->cols, c->sd, w);
        uint32_t *qrow = c->qw + r * (c->cols / 8);
        memset(qrow, 0, sizeof(uint32_t) * (size_t)(c->cols / 8));
        for (int64_t g = 0; g < ng; g++) {
            const float *wg = w + g * c->group;
            float mn = wg[0], mx = wg[0];
            for (int64_t j = 1; j < c->group; j++) {
                if (wg[j] < mn) mn = wg[j];
                if (wg[j] > mx) mx = wg[j];
            }
            uint16_t sbits = f32_to_bf16_rne((mx - mn) / 15.0f);
            uint16_t bbits = f32_to_bf16_rne(mn);
            c->sc[r * ng + g] = sbits;
            c->bi[r * ng + g] = bbits;
            double s = (double)bf16_to_f32(sbits), b = (double)bf16_to_f32(bbits);
            for (int64_t j = 0; j < c->group; j++) {
                int q = 0;
                if (s != 0.0) {
                    double v = nearbyint(((double)wg[j] - b) / s);
                    q = v < 0.0 ? 0 : (v > 15.0 ? 15 : (int)v);
                }
                int64_t col = g * c->group + j;
                qrow[col >> 3] |= (uint32_t)q << (4 * (col & 7));
            }
        }
    }
    free(w);
}
void synth_q4_matrix(uint64_t seed, uint32_t tensor, int64_t nmat, int64_t rows, int64_t cols, int64_t group,
                     double sd, uint32_t *qw, uint16_t *scales, uint16_t *biases, int nthreads) {
    q4_ctx c = {synth_key(seed, tensor, 0), nmat * rows, cols, group, sd, qw, scales, biases};
    parallel_for(nmat * rows, nthreads, q4_range, &c);
}

/* ---- per-expert router logit offsets with Zipf-ranked experts ----
 * Ranks 1..E are assigned to experts by a seeded Fisher-Yates shuffle, and
 * bias_e = c * ln(rank_e^-s / H_s), H_s = sum_{r=1..E} r^-s. */
void synth_zipf_bias(uint64_t seed, uint32_t tensor, int64_t E, double s, double coef, float *bias) {
    uint64_t key = synth_key(seed, tensor, 0);
    int64_t *perm = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    for (int64_t i = 0; i < E; i++) perm[i] = i;
    for (int64_t i = E - 1; i >= 1; i--) {
        uint64_t d = synth_draw(key, (uint64_t)i);
        int64_t j = (int64_t)(((unsigned __int128)d * (unsigned __int128)(uint64_t)(i + 1)) >> 64);
        int64_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
    double H = 0.0;
    for (int64_t r = 1; r <= E; r++) H += pow((double)r, -s);
    for (int64_t i = 0; i < E; i++) {
        double rank = (double)(i + 1);
        bias[perm[i]] = (float)(coef * (-s * log(rank) - log(H)));
    }
    free(perm);
}
