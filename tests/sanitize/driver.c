/* Host driver for the sanitizer build of the fp64 oracle and the input
 * generator (both plain C, CPU only): it generates a small layer and
 * activations with the generator and runs every oracle entry point over them,
 * threaded and unthreaded, with and without the optional tensors, so that
 * AddressSanitizer and UndefinedBehaviorSanitizer see every code path.  It
 * prints a checksum and exits 0; a sanitizer finding aborts it. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../oracle/moe_oracle.h"

void synth_normal_bf16(uint64_t, uint32_t, uint32_t, uint64_t, int64_t, double, uint16_t *, int);
void synth_normal_f32(uint64_t, uint32_t, uint32_t, uint64_t, int64_t, double, float *, int);
void synth_x_rows(uint64_t, uint32_t, int64_t, int64_t, const uint32_t *, double, uint16_t *, int);
void synth_q4_matrix(uint64_t, uint32_t, int64_t, int64_t, int64_t, int64_t, double, uint32_t *, uint16_t *,
                     uint16_t *, int);
void synth_zipf_bias(uint64_t, uint32_t, int64_t, double, double, float *);

static void *xmalloc(size_t n) {
    void *p = malloc(n);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static moe_oracle_q4 q4(int64_t E, int64_t out, int64_t in, int64_t g, uint32_t tensor) {
    uint32_t *qw = xmalloc(sizeof(uint32_t) * E * out * in / 8);
    uint16_t *sc = xmalloc(sizeof(uint16_t) * E * out * in / g);
    uint16_t *bi = xmalloc(sizeof(uint16_t) * E * out * in / g);
    synth_q4_matrix(7, tensor, E, out, in, g, 0.05, qw, sc, bi, 3);
    moe_oracle_q4 t = {qw, sc, bi};
    return t;
}

int main(void) {
    const moe_oracle_dims d = {128, 16, 4, 64, 64, 64};
    const int64_t D = d.d_model, E = d.n_experts, k = d.top_k, F = d.d_ff, Fs = d.d_ff_shared, g = d.group_size;
    const int64_t T = 9;
    float *rw = xmalloc(sizeof(float) * E * D), *rb = xmalloc(sizeof(float) * E), *nw = xmalloc(sizeof(float) * D);
    synth_normal_f32(7, 2, 0, 0, E * D, 0.05, rw, 2);
    synth_zipf_bias(7, 3, E, 1.2, 1.2, rb);
    for (int64_t i = 0; i < D; i++) nw[i] = 1.0f + 0.01f * (float)(i % 7);
    uint16_t *sg = xmalloc(2 * Fs * D), *su = xmalloc(2 * Fs * D), *sd = xmalloc(2 * D * Fs), *sgi = xmalloc(2 * D);
    synth_normal_bf16(7, 7, 0, 0, Fs * D, 0.05, sg, 2);
    synth_normal_bf16(7, 8, 0, 0, Fs * D, 0.05, su, 2);
    synth_normal_bf16(7, 9, 0, 0, D * Fs, 0.05, sd, 1);
    synth_normal_bf16(7, 10, 0, 0, D, 0.05, sgi, 1);
    uint16_t *x = xmalloc(2 * T * D), *xn = xmalloc(2 * T * D);
    uint32_t redraw[9] = {0, 1, 0, 2, 0, 0, 3, 0, 1};
    synth_x_rows(7, 1, T, D, redraw, 1.0, x, 3);

    moe_oracle_layer L = {rw, rb, q4(E, F, D, g, 4), q4(E, F, D, g, 5), q4(E, D, F, g, 6), sgi, sg, su, sd, 0.0, 0};
    double *y = xmalloc(sizeof(double) * T * D), *w = xmalloc(sizeof(double) * T * k);
    double *margin = xmalloc(sizeof(double) * T), *logits = xmalloc(sizeof(double) * T * E);
    int32_t *idx = xmalloc(sizeof(int32_t) * T * k);
    const int64_t tokens[3] = {8, 0, 4};
    double sum = 0.0;
    for (int variant = 0; variant < 4; variant++) {
        L.gating = variant & 1;
        L.weights_scale = variant == 2 ? 2.5 : 0.0;
        L.router_b = variant == 3 ? NULL : rb;
        L.sh_gate_inp = variant == 1 ? NULL : sgi;
        L.sh_gate = variant == 3 ? NULL : sg;
        for (int nt = 1; nt <= 4; nt += 3) {
            if (moe_oracle_forward(&d, &L, T, x, NULL, T, y, idx, w, margin, logits, nt) != MOE_ORACLE_OK) return 3;
            for (int64_t i = 0; i < T * D; i++) sum += y[i];
            if (moe_oracle_forward(&d, &L, T, x, tokens, 3, y, NULL, NULL, NULL, NULL, nt) != MOE_ORACLE_OK) return 3;
            for (int64_t i = 0; i < 3 * D; i++) sum += y[i];
            if (moe_oracle_route(&d, &L, T, x, tokens, 3, idx, w, margin, logits, nt) != MOE_ORACLE_OK) return 3;
            for (int64_t i = 0; i < 3 * k; i++) sum += w[i] + idx[i];
            if (moe_oracle_block_forward(&d, &L, T, x, nw, 1e-6, NULL, T, xn, y, idx, w, margin, NULL, nt) !=
                MOE_ORACLE_OK)
                return 3;
            for (int64_t i = 0; i < T * D; i++) sum += y[i];
        }
    }
    printf("checksum %.17g\n", sum);
    const moe_oracle_q4 *qs[3] = {&L.gate, &L.up, &L.down};
    for (int i = 0; i < 3; i++) {
        free((void *)qs[i]->qweight);
        free((void *)qs[i]->scales);
        free((void *)qs[i]->biases);
    }
    void *bufs[] = {rw, rb, nw, sg, su, sd, sgi, x, xn, y, w, margin, logits, idx};
    for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); i++) free(bufs[i]);
    return isfinite(sum) ? 0 : 4;
}
