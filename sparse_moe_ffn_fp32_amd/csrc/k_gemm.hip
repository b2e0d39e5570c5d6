// Grouped expert GEMMs on fp16 MFMA with dequantisation fused into the tile
// load (subsystems 3-6 of the prefill path).
//
// Lily engine page, "Dekvantuoti svorius matricos daugybos metu" (dequantise
// weights during the matmul): the 4-bit codes are expanded one small tile at
// a time into on-chip memory, used at once by the MFMAs, and the full
// dequantised matrix never exists; accumulation is fp32.
//
// Block tile: 128 activation rows (tokens) x 256 weight rows (output
// features); 4 waves as 2 x 2, each 64 x 128 = 2 x 4 tiles of
// v_mfma_f32_32x32x16_f16.  MFMA layout: lane l holds A[l%32][8*(l/32) .. +8]
// and B[8*(l/32) .. +8][l%32]; accumulator lane l holds C[i][l%32] for
// i = 8*(v/4) + 4*(l/32) + v%4, v = 0..15.  K advances in steps of 64, one
// quantisation group.  Both operands are fp16 with K inside every 8-block in
// the perm8 order (see moe_common.h); a dequantised weight is fp16(s*q + b)
// rounded once, x is converted from bf16 exactly (within the fp16 range), h is
// rounded once to fp16.
//
//   A (activations) goes from global memory straight into registers in MFMA
//     layout.  Inside a K step the lane half kq = l/32 owns K in
//     [32kq, 32kq + 32) and MFMA sub-step kk uses [32kq + 8kk, +8), so a
//     lane's slice of one row is one contiguous 64-byte load.  The same K
//     mapping is applied to B, so every product pairs equal K.
//   B (weights), one row per thread: the row's codes (or bf16 values) and the
//     group's scale and bias are loaded two steps ahead, expanded in registers
//     and written to a double-buffered LDS tile [256][64 + 8]; the MFMAs read
//     their B fragments from there.
//   One barrier per K step: step k multiplies from LDS buffer k%2 while the
//     threads expand step k+1 into the other buffer.
//
// Modes:
//   GU     routed gate/up over the expert-sorted rows; epilogue SwiGLU
//          h = silu(gate) * up -> fp16 (fused chain (i) of the Lily page,
//          "Sumazinti tarpini ir busenos srauta");
//   DOWN   routed down over h; epilogue * routing weight -> fp16 partials
//          (one per assignment, scaled by 2^6, summed in fp32 by the combine);
//   SGU    shared gate/up over all tokens (bf16 weights converted to fp16);
//   SDOWN  shared down; epilogue = the combine: y = sum_{r=0..7} partial_r
//          + sgate * shexp, fixed order, one bf16 rounding, no atomics
//          (fused chain (ii)).
#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe_ffn.h"

namespace moe {

enum { MODE_GU = 0, MODE_DOWN = 1, MODE_SGU = 2, MODE_SDOWN = 3 };

constexpr int GEMM_BM = 128;          // activation rows per block
constexpr int GEMM_BN = 256;          // weight rows per block
constexpr int BK = 64;
constexpr int LDSB = BK + 8;          // fp16 per LDS row (16-byte pad)
// Partials are stored as fp16(2^6 * w * out): the power of two moves the
// typical magnitudes (1e-6 .. 1) clear of the fp16 subnormal range and is
// removed exactly in the combine; |w * out| must stay below 1023.
constexpr float PARTIAL_SCALE = 64.0f;

template <int MODE>
struct GemmCfg {
    static constexpr bool GATED = (MODE == MODE_GU || MODE == MODE_SGU);
    static constexpr bool Q4 = (MODE == MODE_GU || MODE == MODE_DOWN);
    static constexpr int KTOT = GATED ? D : (MODE == MODE_DOWN ? F : FS);
    static constexpr int NK = KTOT / BK;  // even for every mode
    static constexpr int BW = Q4 ? 2 : 8; // 16-byte words of B source per row per step
};

struct GemmArgs {
    // activations
    const uint16_t* xh;      // fp16 [T, D] (perm8)
    const uint16_t* h;       // fp16 [N_assign, F] (perm8), expert-sorted rows
    const uint16_t* hs;      // fp16 [T, FS] (perm8)
    // routing
    const int32_t* perm;     // sorted position -> assignment
    const int32_t* pos_of;   // assignment -> sorted position
    const int32_t* offs;     // [E+1] expert segment starts
    const int32_t* tiles;    // [2*i] expert, [2*i+1] first row
    const int32_t* tile_count;
    const float* wflat;      // [T*K] routing weights by assignment
    const float* sgate;      // [T]
    // weights
    const uint32_t* q[2];    // GU: gate, up; DOWN: down
    const uint16_t* sc[2];
    const uint16_t* bi[2];
    const uint16_t* sw[2];   // SGU: shared gate, up; SDOWN: shared down
    // outputs
    uint16_t* h_out;         // GU
    uint16_t* p_out;         // DOWN: fp16 partials [N_assign, D]
    uint16_t* hs_out;        // SGU
    uint16_t* y;             // SDOWN: bf16 [T, D]
    const uint16_t* p_in;    // SDOWN: fp16 partials
    int T;
};

// One step of one thread's B row, as loaded from global memory.
template <int BW>
struct BStage {
    u32x4 c[BW];
    uint16_t s, b;  // Q4: the group's bf16 scale and bias
};

template <int MODE>
__global__ void __launch_bounds__(256) k_gemm(GemmArgs g) {
    using C = GemmCfg<MODE>;
    __shared__ __attribute__((aligned(16))) f16 sB[2][GEMM_BN * LDSB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, kq = lane >> 5;

    // ---- which rows this block owns
    int e = 0, m0 = 0, rows = 0, seg = 0;
    if constexpr (MODE == MODE_GU || MODE == MODE_DOWN) {
        const int tile = blockIdx.x;
        if (tile >= g.tile_count[0]) return;
        e = g.tiles[2 * tile];
        m0 = g.tiles[2 * tile + 1];
        seg = g.offs[e];
        rows = min(GEMM_BM, g.offs[e + 1] - seg - m0);  // >= 1 for a listed tile
    } else {
        m0 = blockIdx.x * GEMM_BM;
        rows = min(GEMM_BM, g.T - m0);                  // >= 1 inside the grid
    }

    // ---- this lane's two A rows; rows past the end repeat the last valid row
    // (their products are computed and dropped)
    const uint16_t* arow[2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
        const int r = min(wm * 64 + mt * 32 + l32, rows - 1);
        const uint16_t* p;
        if constexpr (MODE == MODE_GU) p = g.xh + (size_t)(g.perm[seg + m0 + r] / K) * D;
        else if constexpr (MODE == MODE_DOWN) p = g.h + (size_t)(seg + m0 + r) * F;
        else if constexpr (MODE == MODE_SGU) p = g.xh + (size_t)(m0 + r) * D;
        else p = g.hs + (size_t)(m0 + r) * FS;
        arow[mt] = p + 32 * kq;
    }

    // ---- this thread's B row: LDS row tid.  Gated modes: inside each wave
    // column's 128 rows, 32-row tile nt holds gate (nt even) or up (nt odd)
    // rows of features fbase + (nt/2)*32 + 0..31, so one lane's accumulators
    // for tiles 2h and 2h+1 hold the gate and up value of the same feature.
    const u32x4* bsrc;
    const uint16_t *bsc = nullptr, *bbi = nullptr;
    if constexpr (C::GATED) {
        const int j = tid & 127, nt = j >> 5, mat = nt & 1;
        const int feat = blockIdx.y * 128 + (tid >> 7) * 64 + (nt >> 1) * 32 + (j & 31);
        if constexpr (C::Q4) {
            const size_t row = (size_t)e * F + feat;
            bsrc = (const u32x4*)(g.q[mat] + row * (D / 8));
            bsc = g.sc[mat] + row * (D / G);
            bbi = g.bi[mat] + row * (D / G);
        } else {
            bsrc = (const u32x4*)(g.sw[mat] + (size_t)feat * D);
        }
    } else {
        const int o = blockIdx.y * GEMM_BN + tid;
        if constexpr (C::Q4) {
            const size_t row = (size_t)e * D + o;
            bsrc = (const u32x4*)(g.q[0] + row * (F / 8));
            bsc = g.sc[0] + row * (F / G);
            bbi = g.bi[0] + row * (F / G);
        } else {
            bsrc = (const u32x4*)(g.sw[0] + (size_t)o * FS);
        }
    }

    auto load_a = [&](int k, u32x4 (&a)[2][4]) {
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int i = 0; i < 4; i++) a[mt][i] = *(const u32x4*)(arow[mt] + k * BK + 8 * i);
    };
    auto load_b = [&](int k, BStage<C::BW>& b) {
#pragma unroll
        for (int i = 0; i < C::BW; i++) b.c[i] = bsrc[k * C::BW + i];
        if constexpr (C::Q4) {
            b.s = bsc[k];
            b.b = bbi[k];
        }
    };
    // expand one step of this thread's row into LDS buffer `buf`
    auto store_b = [&](const BStage<C::BW>& b, int buf) {
        f16* dst = &sB[buf][tid * LDSB];
        if constexpr (C::Q4) {
            const f16 s = (f16)bf16_to_f32(b.s), bb = (f16)bf16_to_f32(b.b);
            const f16x2 s2 = {s, s}, b2 = {bb, bb};
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int w = 0; w < 4; w++) *(u32x4*)(dst + 8 * (4 * i + w)) = q4_word_to_f16x8(b.c[i][w], s2, b2);
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++) *(u32x4*)(dst + 8 * i) = bf16x8_to_f16x8_perm(b.c[i]);
        }
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nt = 0; nt < 4; nt++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[mt][nt][v] = 0.0f;

    auto mfma_step = [&](int buf, const u32x4 (&a)[2][4]) {
        const f16* bb = &sB[buf][(wn * 128 + l32) * LDSB + 32 * kq];
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            f16x8 bf[4];
#pragma unroll
            for (int nt = 0; nt < 4; nt++) bf[nt] = *(const f16x8*)(bb + nt * 32 * LDSB + 8 * kk);
#pragma unroll
            for (int mt = 0; mt < 2; mt++) {
                const f16x8 af = __builtin_bit_cast(f16x8, a[mt][kk]);
#pragma unroll
                for (int nt = 0; nt < 4; nt++)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf[nt], acc[mt][nt], 0, 0, 0);
            }
        }
    };

    // ---- pipeline.  Global loads run three steps ahead of the MFMAs (A into
    // a ring of four register sets, B codes into a ring of four stages); the
    // B tile of step k+1 is expanded into LDS while step k multiplies.  The
    // loop body covers four steps so every ring index and LDS buffer is a
    // compile-time constant; loads past the last step re-read the last step
    // (in bounds, unused) so the body has no branches.
    u32x4 ar[4][2][4];
    BStage<C::BW> br[4];
#pragma unroll
    for (int j = 0; j < 3; j++) {
        load_a(j, ar[j]);
        load_b(j, br[j]);
    }
    store_b(br[0], 0);
    __syncthreads();
    static_assert(C::NK % 4 == 0, "K steps must be a multiple of four");
#pragma unroll 1
    for (int k = 0; k < C::NK; k += 4) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int kn = min(k + j + 3, C::NK - 1);
            load_a(kn, ar[(j + 3) & 3]);
            load_b(kn, br[(j + 3) & 3]);
            // keep the loads here: the scheduler would otherwise sink them
            // towards their first use and undo the prefetch
            __builtin_amdgcn_sched_barrier(0);
            mfma_step(j & 1, ar[j]);
            store_b(br[(j + 1) & 3], (j + 1) & 1);  // past the end: rewrites an unused buffer
            __syncthreads();
        }
    }

    // ---- epilogues
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int r = wm * 64 + mt * 32 + 8 * (v >> 2) + 4 * kq + (v & 3);
            if (r >= rows) continue;
            if constexpr (C::GATED) {
#pragma unroll
                for (int hf = 0; hf < 2; hf++) {
                    const int feat = blockIdx.y * 128 + wn * 64 + hf * 32 + l32;
                    const float hv = silu_f32(acc[mt][2 * hf][v]) * acc[mt][2 * hf + 1][v];
                    const int pc = (feat & ~7) | perm8_pos(feat & 7);
                    const uint16_t hb = __builtin_bit_cast(uint16_t, (f16)hv);
                    if constexpr (MODE == MODE_GU) g.h_out[(size_t)(seg + m0 + r) * F + pc] = hb;
                    else g.hs_out[(size_t)(m0 + r) * FS + pc] = hb;
                }
            } else if constexpr (MODE == MODE_DOWN) {
                const int s = seg + m0 + r;
                const float wt = g.wflat[g.perm[s]] * PARTIAL_SCALE;
#pragma unroll
                for (int nt = 0; nt < 4; nt++) {
                    const int o = blockIdx.y * GEMM_BN + wn * 128 + nt * 32 + l32;
                    g.p_out[(size_t)s * D + o] = __builtin_bit_cast(uint16_t, (f16)(wt * acc[mt][nt][v]));  // wt carries 2^6
                }
            } else {
                const int t = m0 + r;
                const float sg = g.sgate[t];
#pragma unroll
                for (int nt = 0; nt < 4; nt++) {
                    const int o = blockIdx.y * GEMM_BN + wn * 128 + nt * 32 + l32;
                    float sum = 0.0f;
#pragma unroll
                    for (int rr = 0; rr < K; rr++) sum += (float)__builtin_bit_cast(f16, g.p_in[(size_t)g.pos_of[t * K + rr] * D + o]);
                    sum = sum * (1.0f / PARTIAL_SCALE) + sg * acc[mt][nt][v];
                    g.y[(size_t)t * D + o] = f32_to_bf16_rne(sum);
                }
            }
        }
    }
}

// y = sum_r partial_r, for layers without a shared expert.
__global__ void __launch_bounds__(256) k_combine_routed(const uint16_t* __restrict__ p, const int32_t* __restrict__ pos_of,
                                                        uint16_t* __restrict__ y, int T) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= T * D) return;
    const int t = i / D, o = i % D;
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < K; r++) sum += (float)__builtin_bit_cast(f16, p[(size_t)pos_of[t * K + r] * D + o]);
    y[i] = f32_to_bf16_rne(sum * (1.0f / PARTIAL_SCALE));
}

// x bf16 [T, D] -> fp16 [T, D] in perm8 order.
__global__ void __launch_bounds__(256) k_prep_x(const uint16_t* __restrict__ x, uint16_t* __restrict__ xh, int n8) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    ((u32x4*)xh)[i] = bf16x8_to_f16x8_perm(((const u32x4*)x)[i]);
}

int gemm_bm() { return GEMM_BM; }

hipError_t launch_prep_x(const uint16_t* x, uint16_t* xh, int T, hipStream_t s) {
    const int n8 = T * D / 8;
    hipLaunchKernelGGL(k_prep_x, dim3((n8 + 255) / 256), dim3(256), 0, s, x, xh, n8);
    return hipGetLastError();
}

hipError_t launch_prefill_gemms(const PrefillGemmParams& p, const Tracer& tr, hipStream_t s) {
    GemmArgs g = {};
    g.xh = p.xh; g.h = p.h; g.hs = p.hs;
    g.perm = p.perm; g.pos_of = p.pos_of; g.offs = p.offs; g.tiles = p.tiles; g.tile_count = p.tile_count;
    g.wflat = p.wflat; g.sgate = p.sgate;
    g.T = p.T;
    const int max_tiles = (p.T * K + GEMM_BM - 1) / GEMM_BM + E;
    const int mt = (p.T + GEMM_BM - 1) / GEMM_BM;
    // routed gate/up: 128 features (256 gate + up rows) per block
    g.q[0] = p.gate_q; g.sc[0] = p.gate_s; g.bi[0] = p.gate_b;
    g.q[1] = p.up_q; g.sc[1] = p.up_s; g.bi[1] = p.up_b;
    g.h_out = p.h;
    tr.launch(MOE_FFN_KERNEL_EXPERT_GU, k_gemm<MODE_GU>, dim3(max_tiles, F / 128), dim3(256), 0, s, g);
    // shared gate/up
    if (p.sh_gate) {
        g.sw[0] = p.sh_gate; g.sw[1] = p.sh_up; g.hs_out = p.hs;
        hipLaunchKernelGGL(k_gemm<MODE_SGU>, dim3(mt, FS / 128), dim3(256), 0, s, g);
    }
    // routed down
    g.q[0] = p.down_q; g.sc[0] = p.down_s; g.bi[0] = p.down_b;
    g.p_out = p.partial;
    tr.launch(MOE_FFN_KERNEL_EXPERT_DOWN, k_gemm<MODE_DOWN>, dim3(max_tiles, D / GEMM_BN), dim3(256), 0, s, g);
    // combine
    if (p.sh_gate) {
        g.sw[0] = p.sh_down; g.p_in = p.partial; g.y = p.y;
        tr.launch(MOE_FFN_KERNEL_COMBINE, k_gemm<MODE_SDOWN>, dim3(mt, D / GEMM_BN), dim3(256), 0, s, g);
    } else {
        tr.launch(MOE_FFN_KERNEL_COMBINE, k_combine_routed, dim3((p.T * D + 255) / 256), dim3(256), 0, s,
                  (const uint16_t*)p.partial, (const int32_t*)p.pos_of, p.y, p.T);
    }
    return hipGetLastError();
}

}  // namespace moe
