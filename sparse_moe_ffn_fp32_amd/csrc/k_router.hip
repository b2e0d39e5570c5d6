// Router (subsystem 1): fp32 logits, softmax, top-8 with lower-index
// tie-break, renormalised weights; and the shared-expert gate sigmoid.
//
// qwen35moe forward-pass page, "Shared-expert MoE FFN (every layer)": gate =
// SOFTMAX over 256 experts, 8 used, norm_topk_prob = TRUE ("Correctness
// watch-list": renormalise the top-8 weights); sgate = sigmoid(
// ffn_gate_inp_shexp . x).
//
// Large T: the logits are a [T, 2048] x [2048, 256] GEMM on fp16 MFMA (the
// grouped-GEMM kernel's router mode).  Each x row and each router row is
// scaled by its own power of two into the fp16 range (x exactly, bf16 having
// fewer significant bits than fp16), each fp32 router weight split into two
// fp16 planes hi + lo with |w' - hi - lo| <= 2^-22 |w'|, and the exponents
// are re-applied exactly to the fp32 sums, so a logit over 2048 inputs of
// unit size is off by ~1e-6 at most whatever the magnitudes: far below the
// 1e-4 top-8/top-9 margin the index-exactness bar is stated for.
#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe_ffn.h"

namespace moe {

// The fp16 operands of the prefill GEMMs that come from weight matrices
// given in other types, one wave per row, each row with its power-of-two
// exponent (row_exp: the row's largest magnitude scaled into [2^14, 2^15)):
//   rows [0, E):  router fp32 [E, D] -> wr2 fp16 [2, E, D], hi = fp16(w'),
//                 lo = fp16(w' - hi) for w' = w 2^-e (w' - hi is exact in
//                 fp32), so |w' - hi - lo| <= 2^-22 |w'| (or 2^-25 absolute
//                 in the subnormals, under 2^-39 of the row's largest
//                 value); er[row] = e;
//   rows [E, E + 2 FS + D): the shared expert's gate, up (K = D) and down
//                 (K = FS) rows, bf16 -> fp16 (exact within the scaled
//                 range) in shw = [gate FS x D | up FS x D | down D x FS];
//                 es[row - E] = e.
// K is in the perm8 order everywhere.
__device__ __forceinline__ void prep_weight_row(const float* __restrict__ wr, uint16_t* __restrict__ wr2,
                                                int32_t* __restrict__ er, const uint16_t* __restrict__ sg,
                                                const uint16_t* __restrict__ su, const uint16_t* __restrict__ sd,
                                                uint16_t* __restrict__ shw, int32_t* __restrict__ es, int row,
                                                int lane) {
    if (row < E) {
        // 256 pieces of 8 weights: lane takes pieces lane + 64 i
        const f32x4* src = (const f32x4*)(wr + (size_t)row * D);
        float v[4][8];
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const f32x4 a = src[2 * (lane + 64 * i)], b = src[2 * (lane + 64 * i) + 1];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                v[i][j] = a[j];
                v[i][4 + j] = b[j];
            }
#pragma unroll
            for (int j = 0; j < 8; j++) m = __builtin_fmaxf(m, __builtin_fabsf(v[i][j]));
        }
        m = __builtin_bit_cast(float, wave_max(__builtin_bit_cast(int, m)));
        const int e = row_exp(m);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            u32x4 hi, lo;
#pragma unroll
            for (int j = 0; j < 4; j++) {  // perm8: pair j holds elements j and j + 4
                const float w0 = __builtin_ldexpf(v[i][j], -e), w1 = __builtin_ldexpf(v[i][j + 4], -e);
                const f16 h0 = (f16)w0, h1 = (f16)w1;
                const f16 l0 = (f16)(w0 - (float)h0), l1 = (f16)(w1 - (float)h1);
                hi[j] = __builtin_bit_cast(uint32_t, f16x2{h0, h1});
                lo[j] = __builtin_bit_cast(uint32_t, f16x2{l0, l1});
            }
            u32x4* dst = (u32x4*)(wr2 + (size_t)row * D) + lane + 64 * i;
            dst[0] = hi;
            dst[E * D / 8] = lo;
        }
        if (lane == 0) er[row] = e;
        return;
    }
    const int r = row - E;
    const bool down = r >= 2 * FS;
    const int kdim = down ? FS : D;
    const uint16_t* src = r < FS ? sg + (size_t)r * D : r < 2 * FS ? su + (size_t)(r - FS) * D : sd + (size_t)(r - 2 * FS) * FS;
    uint16_t* dst = shw + (size_t)(down ? 2 * FS * D + (r - 2 * FS) * FS : r * D);
    const int npc = kdim / 8 / 64;  // pieces of 8 per lane: 4 (K = D) or 1 (K = FS)
    u32x4 d[4];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (i < npc) {
            d[i] = ((const u32x4*)src)[lane + 64 * i];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t w = d[i][j];
                m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(__uint_as_float(w << 16)),
                                                       __builtin_fabsf(__uint_as_float(w & 0xffff0000u))));
            }
        }
    }
    m = __builtin_bit_cast(float, wave_max(__builtin_bit_cast(int, m)));
    const int e = row_exp(m);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        if (i < npc) {
            float f[8];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t w = d[i][j];
                f[2 * j] = __uint_as_float(w << 16);
                f[2 * j + 1] = __uint_as_float(w & 0xffff0000u);
            }
            ((u32x4*)dst)[lane + 64 * i] = f32x8_to_f16x8_perm_scaled(f, e);
        }
    }
    if (lane == 0) es[r] = e;
}

// x bf16 [T, D] -> fp16 [T, D] in perm8 order, each row times 2^-ex[t] with
// its exponent (row_exp of its largest |x|); exact where the scaled value is
// an fp16 normal.  With the row at hand, also the shared-expert gate
// (qwen35moe page, "Shared-expert MoE FFN"): sgate[t] = sigmoid(gate_inp . x)
// (1 when the layer has no gate vector).  One wave per row, lane pieces
// lane + 64 i.
__device__ __forceinline__ void prep_x_row(const uint16_t* __restrict__ x, uint16_t* __restrict__ xh,
                                           int32_t* __restrict__ ex, const uint16_t* __restrict__ gate_inp,
                                           float* __restrict__ sgate, int t, int lane) {
    const u32x4* src = (const u32x4*)(x + (size_t)t * D);
    u32x4 d[4], gv[4];
    float m = 0.0f, z = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        d[i] = src[lane + 64 * i];
        gv[i] = gate_inp ? ((const u32x4*)gate_inp)[lane + 64 * i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t w = d[i][j], gw = gv[i][j];
            z += __uint_as_float(w << 16) * __uint_as_float(gw << 16);
            z += __uint_as_float(w & 0xffff0000u) * __uint_as_float(gw & 0xffff0000u);
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t w = d[i][j];
            m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(__uint_as_float(w << 16)),
                                                   __builtin_fabsf(__uint_as_float(w & 0xffff0000u))));
        }
    }
    m = __builtin_bit_cast(float, wave_max(__builtin_bit_cast(int, m)));
    z = wave_sum(z);
    if (lane == 0) sgate[t] = gate_inp ? 1.0f / (1.0f + __expf(-z)) : 1.0f;
    const int e = row_exp(m);
    u32x4* dst = (u32x4*)(xh + (size_t)t * D);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        float f[8];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t w = d[i][j];
            f[2 * j] = __uint_as_float(w << 16);
            f[2 * j + 1] = __uint_as_float(w & 0xffff0000u);
        }
        dst[lane + 64 * i] = f32x8_to_f16x8_perm_scaled(f, e);
    }
    if (lane == 0) ex[t] = e;
}


// Both preparations in one launch, one wave per row: blocks [0, nb_w) take
// the n_rows weight rows, the next nb_x blocks the T rows of x, and the last
// ones zero the sort's per-chunk expert counts (n_cnt ints), which the top-k
// launch then accumulates (a fill kernel of its own would be one more
// launch; no memset node either, so the sequence can be captured in a graph).
__global__ void __launch_bounds__(256) k_prep(const float* __restrict__ wr, uint16_t* __restrict__ wr2,
                                              int32_t* __restrict__ er, const uint16_t* __restrict__ sg,
                                              const uint16_t* __restrict__ su, const uint16_t* __restrict__ sd,
                                              uint16_t* __restrict__ shw, int32_t* __restrict__ es, int n_rows,
                                              int nb_w, const uint16_t* __restrict__ x, uint16_t* __restrict__ xh,
                                              int32_t* __restrict__ ex, const uint16_t* __restrict__ gate_inp,
                                              float* __restrict__ sgate, int T, int nb_x, int32_t* __restrict__ cnt,
                                              int n_cnt) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if ((int)blockIdx.x < nb_w) {
        const int row = blockIdx.x * 4 + wave;
        if (row < n_rows) prep_weight_row(wr, wr2, er, sg, su, sd, shw, es, row, lane);
    } else if ((int)blockIdx.x < nb_w + nb_x) {
        const int t = (blockIdx.x - nb_w) * 4 + wave;
        if (t < T) prep_x_row(x, xh, ex, gate_inp, sgate, t, lane);
    } else {
        const int i = ((int)blockIdx.x - nb_w - nb_x) * 256 + threadIdx.x;
        if (i < n_cnt) cnt[i] = 0;
    }
}

// One wave per token: top-8 of the 256 logits (or the hash table's
// experts) and their renormalised weights.  Lane l holds experts l, l+64,
// l+128, l+192.
template <bool HASH>
__global__ void __launch_bounds__(256) k_topk(const float* __restrict__ logits, int32_t* __restrict__ idx_out,
                                              float* __restrict__ w_out, float wscale,
                                              int gating, const int32_t* __restrict__ tid2eid,
                                              const int32_t* __restrict__ token_ids, int n_vocab, int T,
                                              int32_t* __restrict__ cnt, int chunk) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float sel_v[K];
    int sel_i[K];
    select_experts<HASH>(logits + (size_t)t * E, tid2eid, n_vocab, HASH ? token_ids[t] : 0, lane, sel_v, sel_i);
    // norm_topk_prob: the eight selected scores renormalised (for softmax
    // the full normaliser cancels: the softmax over the selected logits)
    float p[K], s = 0.0f;
    const float vmax = selected_max<HASH>(sel_v);
#pragma unroll
    for (int r = 0; r < K; r++) {
        p[r] = route_score(sel_v[r], vmax, gating);
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
        // the sort's expert counts of this assignment's chunk (integer
        // atomics: the totals do not depend on their order)
        atomicAdd(&cnt[(size_t)((t * K + lane) / chunk) * E + (iv & (E - 1))], 1);
    }
}

hipError_t launch_prep(const float* wr, uint16_t* wr2, int32_t* er, const uint16_t* sg, const uint16_t* su,
                       const uint16_t* sd, uint16_t* shw, int32_t* es, const uint16_t* x, uint16_t* xh, int32_t* ex,
                       const uint16_t* gate_inp, float* sgate, int T, int32_t* cnt, int n_cnt, hipStream_t s) {
    const int n_rows = E + (sg ? 2 * FS + D : 0);
    const int nb_w = (n_rows + 3) / 4, nb_x = (T + 3) / 4;
    hipLaunchKernelGGL(k_prep, dim3(nb_w + nb_x + (n_cnt + 255) / 256), dim3(256), 0, s, wr, wr2, er, sg, su, sd,
                       shw, es, n_rows, nb_w, x, xh, ex, gate_inp, sgate, T, nb_x, cnt, n_cnt);
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int32_t* idx, float* w, float wscale, int gating, const int32_t* tid2eid,
                       const int32_t* token_ids, int n_vocab, int T, int32_t* cnt, int chunk, hipStream_t s) {
    if (tid2eid)
        hipLaunchKernelGGL(k_topk<true>, dim3((T + 3) / 4), dim3(256), 0, s, logits, idx, w, wscale, gating, tid2eid,
                           token_ids, n_vocab, T, cnt, chunk);
    else
        hipLaunchKernelGGL(k_topk<false>, dim3((T + 3) / 4), dim3(256), 0, s, logits, idx, w, wscale, gating, tid2eid,
                           token_ids, n_vocab, T, cnt, chunk);
    return hipGetLastError();
}

}  // namespace moe
