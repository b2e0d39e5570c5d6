// Router (subsystem 1): fp32 logits, softmax, top-8 with lower-index
// tie-break, renormalised weights; and the shared-expert gate sigmoid.
//
// qwen35moe forward-pass page, "Shared-expert MoE FFN (every layer)": gate =
// SOFTMAX over 256 experts, 8 used, norm_topk_prob = TRUE ("Correctness
// watch-list": renormalise the top-8 weights); sgate = sigmoid(
// ffn_gate_inp_shexp . x).
//
// Large T: the logits are a [T, 2048] x [2048, 256] GEMM on fp16 MFMA (the
// grouped-GEMM kernel's router mode).  x is exact in fp16 within the fp16
// range; each fp32 router weight is split into two fp16 planes hi + lo with
// |w - hi - lo| <= max(2^-22 |w|, 2^-25) (hi = fp16(w), lo = fp16(w - hi),
// w - hi exact in fp32; the absolute term is fp16's subnormal spacing), so a
// logit over 2048 inputs of unit size is off by ~1e-6 at most: far below the
// 1e-4 top-8/top-9 margin the index-exactness bar is stated for.
#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe_ffn.h"

namespace moe {

// Wr fp32 [E, D] -> Wr2 fp16 [2, E, D] (hi, lo), K in the perm8 order.  One
// thread per 8-element block.
__global__ void __launch_bounds__(256) k_split_router(const float* __restrict__ wr, uint16_t* __restrict__ wr2) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= E * D / 8) return;
    const f32x4 a = ((const f32x4*)wr)[2 * i], b = ((const f32x4*)wr)[2 * i + 1];
    const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    u32x4 hi, lo;
#pragma unroll
    for (int j = 0; j < 4; j++) {  // perm8: pair j holds elements j and j + 4
        const f16 h0 = (f16)v[j], h1 = (f16)v[j + 4];
        const f16 l0 = (f16)(v[j] - (float)h0), l1 = (f16)(v[j + 4] - (float)h1);
        hi[j] = __builtin_bit_cast(uint32_t, f16x2{h0, h1});
        lo[j] = __builtin_bit_cast(uint32_t, f16x2{l0, l1});
    }
    ((u32x4*)wr2)[i] = hi;
    ((u32x4*)wr2)[E * D / 8 + i] = lo;
}

// One wave per token: top-8 of the 256 logits, renormalised softmax weights,
// and sgate.  Lane l holds experts l, l+64, l+128, l+192.
__global__ void __launch_bounds__(256) k_topk(const float* __restrict__ logits, const uint16_t* __restrict__ x,
                                              const uint16_t* __restrict__ gate_inp, int32_t* __restrict__ idx_out,
                                              float* __restrict__ w_out, float* __restrict__ sgate_out, float wscale,
                                              int gating, int T) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; c++) v[c] = logits[(size_t)t * E + lane + 64 * c];
    float sel_v[K];
    int sel_i[K];
    wave_top8(v, lane, sel_v, sel_i);
    // norm_topk_prob: the eight selected scores renormalised (for softmax
    // the full normaliser cancels: the softmax over the selected logits)
    float p[K], s = 0.0f;
#pragma unroll
    for (int r = 0; r < K; r++) {
        p[r] = route_score(sel_v[r], sel_v[0], gating);
        s += p[r];
    }
    const float inv = wscale / s;  // expert_weights_scale folded into the normaliser
    if (lane < K) {
        float wv = 0.0f;
        int iv = 0;
#pragma unroll
        for (int r = 0; r < K; r++)
            if (r == lane) {
                wv = p[r] * inv;
                iv = sel_i[r];
            }
        idx_out[(size_t)t * K + lane] = iv;
        w_out[(size_t)t * K + lane] = wv;
    }
    // sgate = sigmoid(gate_inp . x); lane l covers inputs [32l, 32l+32)
    if (sgate_out) {
        float z = 0.0f;
        if (gate_inp) {
            const u32x4* xp = (const u32x4*)(x + (size_t)t * D + 32 * lane);
            const u32x4* gp = (const u32x4*)(gate_inp + 32 * lane);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                u32x4 xv = xp[q], gv = gp[q];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    z += __uint_as_float(xv[j] << 16) * __uint_as_float(gv[j] << 16);
                    z += __uint_as_float(xv[j] & 0xffff0000u) * __uint_as_float(gv[j] & 0xffff0000u);
                }
            }
            z = wave_sum(z);
        }
        if (lane == 0) sgate_out[t] = gate_inp ? 1.0f / (1.0f + __expf(-z)) : 1.0f;
    }
}

hipError_t launch_split_router(const float* wr, uint16_t* wr2, hipStream_t s) {
    hipLaunchKernelGGL(k_split_router, dim3((E * D / 8 + 255) / 256), dim3(256), 0, s, wr, wr2);
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const uint16_t* x, const uint16_t* gate_inp, int32_t* idx, float* w,
                       float* sgate, float wscale, int gating, int T, hipStream_t s) {
    hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, x, gate_inp, idx, w, sgate, wscale, gating,
                       T);
    return hipGetLastError();
}

}  // namespace moe
