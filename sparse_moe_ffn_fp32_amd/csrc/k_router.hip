// Router (subsystem 1): fp32 logits, softmax, top-8 with lower-index
// tie-break, renormalised weights; and the shared-expert gate sigmoid.
//
// qwen35moe forward-pass page, "Shared-expert MoE FFN (every layer)": gate =
// SOFTMAX over 256 experts, 8 used, norm_topk_prob = TRUE ("Correctness
// watch-list": renormalise the top-8 weights); sgate = sigmoid(
// ffn_gate_inp_shexp . x).
//
// Large T: the logits are a [T, 2048] x [2048, 256] GEMM on bf16 MFMA.  x is
// bf16 already; each fp32 router weight is split exactly into three bf16
// terms hi + mid + lo (8 significant bits each), so every MFMA product is
// exact and the logits carry fp32 accumulation error only.
#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe_ffn.h"

namespace moe {

// Wr fp32 [E, D] -> Wr3 bf16 [3, E, D] with Wr = hi + mid + lo exactly.
__global__ void __launch_bounds__(256) k_split_router(const float* __restrict__ wr, uint16_t* __restrict__ wr3) {
    const int i = blockIdx.x * 256 + threadIdx.x;  // one element per thread
    if (i >= E * D) return;
    const uint32_t u = __float_as_uint(wr[i]);
    const uint32_t hi = u & 0xffff0000u;                       // truncate to 8 significant bits
    const float r1 = __uint_as_float(u) - __uint_as_float(hi);  // exact, <= 16 significant bits
    const uint32_t mid = __float_as_uint(r1) & 0xffff0000u;
    const float r2 = r1 - __uint_as_float(mid);                 // exact, <= 8 significant bits
    wr3[i] = (uint16_t)(hi >> 16);
    wr3[E * D + i] = (uint16_t)(mid >> 16);
    wr3[2 * E * D + i] = (uint16_t)(__float_as_uint(r2) >> 16);  // exact in bf16
}

// logits[T, E] = x . Wr^T (+ bias).  Block: 32 tokens x 256 experts, 4 waves;
// wave w owns experts [64w, 64w+64) as four 16-wide tiles; two 16-token
// tiles.  v_mfma_f32_16x16x32_bf16 operand layout: lane l holds
// A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16]; the accumulator lane l
// holds C[4*(l/16) + v][l%16], v = 0..3.
__global__ void __launch_bounds__(256) k_router_logits(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr3,
                                                       const float* __restrict__ bias, float* __restrict__ logits,
                                                       int T) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * 32;
    const int li = lane & 15, lk = lane >> 4;
    f32x4 acc[2][4];
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
        for (int n = 0; n < 4; n++) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t* xa[2];
    bool va[2];
#pragma unroll
    for (int m = 0; m < 2; m++) {
        int t = t0 + m * 16 + li;
        va[m] = t < T;
        xa[m] = x + (size_t)(va[m] ? t : 0) * D + 8 * lk;
    }
    const uint16_t* wb = wr3 + (size_t)(wave * 64 + li) * D + 8 * lk;

    for (int k0 = 0; k0 < D; k0 += 32) {
        bf16x8 a[2];
#pragma unroll
        for (int m = 0; m < 2; m++) {
            u32x4 v = va[m] ? *(const u32x4*)(xa[m] + k0) : u32x4{0u, 0u, 0u, 0u};
            a[m] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int n = 0; n < 4; n++) {
#pragma unroll
            for (int s = 2; s >= 0; s--) {
                u32x4 v = *(const u32x4*)(wb + (size_t)s * E * D + (size_t)n * 16 * D + k0);
                bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
                for (int m = 0; m < 2; m++) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m], b, acc[m][n], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int n = 0; n < 4; n++) {
        const int e = wave * 64 + n * 16 + li;
        const float b = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int m = 0; m < 2; m++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                int t = t0 + m * 16 + 4 * lk + v;
                if (t < T) logits[(size_t)t * E + e] = acc[m][n][v] + b;
            }
    }
}

// One wave per token: top-8 of the 256 logits, renormalised softmax weights,
// and sgate.  Lane l holds experts l, l+64, l+128, l+192.
__global__ void __launch_bounds__(256) k_topk(const float* __restrict__ logits, const uint16_t* __restrict__ x,
                                              const uint16_t* __restrict__ gate_inp, int32_t* __restrict__ idx_out,
                                              float* __restrict__ w_out, float* __restrict__ sgate_out, int T) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; c++) v[c] = logits[(size_t)t * E + lane + 64 * c];
    float sel_v[K];
    int sel_i[K];
    wave_top8(v, lane, sel_v, sel_i);
    // norm_topk_prob: the full-softmax normaliser cancels, so the weights are
    // the softmax over the eight selected logits.
    float p[K], s = 0.0f;
#pragma unroll
    for (int r = 0; r < K; r++) {
        p[r] = __expf(sel_v[r] - sel_v[0]);
        s += p[r];
    }
    const float inv = 1.0f / s;
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
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
        }
        if (lane == 0) sgate_out[t] = gate_inp ? 1.0f / (1.0f + __expf(-z)) : 1.0f;
    }
}

hipError_t launch_split_router(const float* wr, uint16_t* wr3, hipStream_t s) {
    hipLaunchKernelGGL(k_split_router, dim3((E * D + 255) / 256), dim3(256), 0, s, wr, wr3);
    return hipGetLastError();
}

hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr3, const float* bias, float* logits, int T,
                                const Tracer& tr, hipStream_t s) {
    tr.launch(MOE_FFN_KERNEL_ROUTER, k_router_logits, dim3((T + 31) / 32), dim3(256), 0, s, x, wr3, bias, logits, T);
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const uint16_t* x, const uint16_t* gate_inp, int32_t* idx, float* w,
                       float* sgate, int T, hipStream_t s) {
    hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, x, gate_inp, idx, w, sgate, T);
    return hipGetLastError();
}

}  // namespace moe
