// Decode-path kernel arguments and the per-token routing helpers shared by
// the decode kernels (k_decode.hip: T > TINY_T tokens; k_decode_tiny.hip: T <= TINY_T).
#pragma once

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

// Up to this many tokens the vector-ALU kernels (one block per routed pair,
// no distinct-expert lists) beat the MFMA path: 29.5 against 43.5 us at 5
// tokens, 41.7 against 46.9 us at 8; they cost about 4 us more per token,
// the MFMA path about 1 us.
constexpr int TINY_T = 8;

struct DecodeArgs {
    const uint16_t* x;
    int T;
    const float* wr;
    const float* rbias;
    float wscale;    // factor on the renormalised routing weights
    int gating;      // MOE_FFN_GATING_*
    const int32_t* tid2eid;    // hash routing table [K, n_vocab] or nullptr
    const int32_t* token_ids;  // [T] with the table
    int n_vocab;
    const uint16_t *sgi, *sg, *su, *sd;  // shared expert (sg == nullptr: none)
    const uint32_t *gq, *uq, *dq;
    const uint16_t *gs, *gb, *us, *ub, *ds, *db;
    int gu_rows;     // rows per expert in the gate/up arrays (F, or 2F fused)
    float* logits;   // [T, E]
    uint16_t* xp;    // bf16 [T, D], perm8
    float* xsum;     // [T, D/32] sums of x over 32-element chunks (T <= TINY_T)
    float* hs;       // [T, FS] shared SwiGLU output
    float* ys;       // [T, D] shared down output
    uint16_t* h;     // bf16 [8T, F] (pair-major), perm8: h rounded to nearest
    uint16_t* hl;    // bf16 [8T, F]: the rounded remainder h - hi (hi + lo: 16 significant bits)
    float* part;     // [8T, D] routed down outputs per pair (T > TINY_T)
    float* pa;       // T > TINY_T: stage A's K-slice partials [8][T][E + 2 FS] (in part's space)
    int32_t* idx;
    float* w;
    float* sgate;
    const uint16_t* resid;  // bf16 [T, D] added to y before its rounding, or nullptr
    const float* nw;        // T <= TINY_T: RMSNorm weights (x un-normalised), or nullptr
    float eps;
    uint16_t* xn;           // T <= TINY_T with nw: the normalised rows, bf16 [T, D]
    uint16_t* y;
};

// The experts of token t (top 8 by logit, or looked up in the hash table)
// with their logits (one wave, result wave-uniform); the top-8 form stops
// after the first `ranks` of them.
template <bool HASH>
__device__ __forceinline__ void token_select(const DecodeArgs& a, int t, int lane, float* sel_v, int* sel_i,
                                             int ranks = K) {
    select_experts<HASH>(a.logits + (size_t)t * E, a.tid2eid, a.n_vocab, HASH ? a.token_ids[t] : 0, lane, sel_v,
                         sel_i, ranks);
}

// One wave: write token t's routing, the expert ids and renormalised weights
// (the selected scores over their sum; for softmax the full normaliser
// cancels under norm_topk_prob: the softmax of the eight selected logits).
template <bool HASH>
__device__ inline void write_token_route(const DecodeArgs& a, int t, int lane, const float* sel_v, const int* sel_i,
                                         int* sidx) {
    float p[K], s = 0.0f;
    const float vmax = selected_max<HASH>(sel_v);
#pragma unroll
    for (int r = 0; r < K; r++) {
        p[r] = route_score(sel_v[r], vmax, a.gating);
        s += p[r];
    }
    const float inv = a.wscale / s;  // expert_weights_scale folded into the normaliser
    if (lane < K) {
        float wv = 0.f;
        int iv = 0;
#pragma unroll
        for (int r = 0; r < K; r++)
            if (r == lane) {
                wv = p[r] * inv;
                iv = sel_i[r];
            }
        a.idx[t * K + lane] = iv;
        a.w[t * K + lane] = wv;
        if (sidx) sidx[t * K + lane] = iv;
    }
}


hipError_t launch_decode_tiny(const DecodeArgs& a, const Tracer& tr, hipStream_t s);

}  // namespace moe
