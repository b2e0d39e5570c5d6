// Grouped expert GEMMs on fp16 MFMA with dequantisation fused into the tile
// load (subsystems 3-6 of the prefill path).
//
// Lily engine page, "Dekvantuoti svorius matricos daugybos metu" (dequantise
// weights during the matmul): the 4-bit codes are expanded one small tile at
// a time into on-chip memory, used at once by the MFMAs, and the full
// dequantised matrix never exists; accumulation is fp32.
//
// Operands.  A = activation rows (tokens), B = weight rows (output features),
// both fp16 in LDS with K inside every 8-block in the perm8 order (see
// moe_common.h).  A dequantised weight is fp16(s*q + b) rounded once; x is
// converted from bf16 exactly (within the fp16 range); h is rounded once to
// fp16.  MFMA v_mfma_f32_32x32x16_f16: lane l holds A[l%32][8*(l/32) .. +8]
// and B[8*(l/32) .. +8][l%32]; accumulator lane l holds C[i][l%32] for
// i = 8*(v/4) + 4*(l/32) + v%4, v = 0..15.
//
// Modes:
//   GU     routed gate/up over the expert-sorted rows; epilogue SwiGLU
//          h = silu(gate) * up -> fp16 (fused chain (i) of the Lily page,
//          "Sumazinti tarpini ir busenos srauta");
//   DOWN   routed down over h; epilogue * routing weight -> fp32 partials;
//   SGU    shared gate/up over all tokens (bf16 weights converted to fp16);
//   SDOWN  shared down; epilogue = the combine: y = sum_{r=0..7} partial_r
//          + sgate * shexp, fixed order, one bf16 rounding, no atomics
//          (fused chain (ii)).
#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe_ffn.h"

namespace moe {

enum { MODE_GU = 0, MODE_DOWN = 1, MODE_SGU = 2, MODE_SDOWN = 3 };

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // fp16 elements per LDS row (16 B pad)

template <int MODE, int BM>
struct GemmCfg {
    static constexpr int BN = 128;
    static constexpr bool GATED = (MODE == MODE_GU || MODE == MODE_SGU);
    static constexpr bool Q4 = (MODE == MODE_GU || MODE == MODE_DOWN);
    static constexpr int KTOT = GATED ? D : (MODE == MODE_DOWN ? F : FS);
    static constexpr int MT = BM / 64;   // 32-row MFMA tiles per wave (2x2 waves)
    static constexpr int NT = 2;         // 32-col MFMA tiles per wave
    static constexpr int A_CHUNKS = BM * (BK / 8) / 256;  // 16-byte chunks per thread
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
    float* p_out;            // DOWN: fp32 partials [N_assign, D]
    uint16_t* hs_out;        // SGU
    uint16_t* y;             // SDOWN: bf16 [T, D]
    const float* p_in;       // SDOWN: partials
    int T;
};

template <int MODE, int BM>
__global__ void __launch_bounds__(256) k_gemm(GemmArgs g) {
    using C = GemmCfg<MODE, BM>;
    constexpr int BN = C::BN;
    __shared__ __attribute__((aligned(16))) f16 sA[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) f16 sB[BN * LDS_STRIDE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- which rows this block owns
    int e = 0, m0 = 0, rows = 0, seg = 0;
    if constexpr (MODE == MODE_GU || MODE == MODE_DOWN) {
        const int tile = blockIdx.x;
        if (tile >= g.tile_count[0]) return;
        e = g.tiles[2 * tile];
        m0 = g.tiles[2 * tile + 1];
        seg = g.offs[e];
        rows = min(BM, g.offs[e + 1] - seg - m0);
    } else {
        m0 = blockIdx.x * BM;
        rows = min(BM, g.T - m0);
    }

    // ---- A row pointers of this thread's chunks (fixed over K)
    const uint16_t* arow[C::A_CHUNKS];
    const int acol = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; i++) {
        const int r = (tid >> 3) + 32 * i;
        const uint16_t* p = nullptr;
        if (r < rows) {
            if constexpr (MODE == MODE_GU) p = g.xh + (size_t)(g.perm[seg + m0 + r] / K) * D;
            else if constexpr (MODE == MODE_DOWN) p = g.h + (size_t)(seg + m0 + r) * F;
            else if constexpr (MODE == MODE_SGU) p = g.xh + (size_t)(m0 + r) * D;
            else p = g.hs + (size_t)(m0 + r) * FS;
        }
        arow[i] = p;
    }

    // ---- B row of this thread: row n = tid/2, half = tid%2 (32 K each)
    const int bn = tid >> 1, bhalf = tid & 1;
    const uint32_t* bq = nullptr;
    const uint16_t *bsc = nullptr, *bbi = nullptr, *bw = nullptr;
    if constexpr (C::GATED) {
        const int blk = bn >> 5, mat = blk & 1;
        const int feat = blockIdx.y * 64 + (blk >> 1) * 32 + (bn & 31);
        if constexpr (C::Q4) {
            const size_t row = (size_t)e * F + feat;
            bq = g.q[mat] + row * (D / 8) + 4 * bhalf;
            bsc = g.sc[mat] + row * (D / G);
            bbi = g.bi[mat] + row * (D / G);
        } else {
            bw = g.sw[mat] + (size_t)feat * D + 32 * bhalf;
        }
    } else {
        const int o = blockIdx.y * BN + bn;
        if constexpr (C::Q4) {
            const size_t row = (size_t)e * D + o;
            bq = g.q[0] + row * (F / 8) + 4 * bhalf;
            bsc = g.sc[0] + row * (F / G);
            bbi = g.bi[0] + row * (F / G);
        } else {
            bw = g.sw[0] + (size_t)o * FS + 32 * bhalf;
        }
    }

    f32x16 acc[C::MT][C::NT];
#pragma unroll
    for (int m = 0; m < C::MT; m++)
#pragma unroll
        for (int n = 0; n < C::NT; n++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[m][n][v] = 0.0f;

    for (int k0 = 0; k0 < C::KTOT; k0 += BK) {
        // global -> registers
        u32x4 av[C::A_CHUNKS];
#pragma unroll
        for (int i = 0; i < C::A_CHUNKS; i++)
            av[i] = arow[i] ? *(const u32x4*)(arow[i] + k0 + acol) : u32x4{0u, 0u, 0u, 0u};
        u32x4 bv[4];
        if constexpr (C::Q4) {
            const u32x4 wq = *(const u32x4*)(bq + k0 / 8);
            const float s = bf16_to_f32(bsc[k0 / G]);
            const float b = bf16_to_f32(bbi[k0 / G]);
            const f16x2 s2 = {(f16)s, (f16)s}, b2 = {(f16)b, (f16)b};
#pragma unroll
            for (int j = 0; j < 4; j++) bv[j] = q4_word_to_f16x8(wq[j], s2, b2);
        } else {
#pragma unroll
            for (int j = 0; j < 4; j++) bv[j] = bf16x8_to_f16x8_perm(*(const u32x4*)(bw + k0 + 8 * j));
        }
        __syncthreads();  // previous step's MFMAs are done with LDS
#pragma unroll
        for (int i = 0; i < C::A_CHUNKS; i++)
            *(u32x4*)(sA + ((tid >> 3) + 32 * i) * LDS_STRIDE + acol) = av[i];
#pragma unroll
        for (int j = 0; j < 4; j++) *(u32x4*)(sB + bn * LDS_STRIDE + 32 * bhalf + 8 * j) = bv[j];
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK / 16; kk++) {
            f16x8 a[C::MT], b[C::NT];
#pragma unroll
            for (int m = 0; m < C::MT; m++)
                a[m] = *(const f16x8*)(sA + (wm * (BM / 2) + m * 32 + (lane & 31)) * LDS_STRIDE + kk * 16 +
                                       8 * (lane >> 5));
#pragma unroll
            for (int n = 0; n < C::NT; n++)
                b[n] = *(const f16x8*)(sB + (wn * (BN / 2) + n * 32 + (lane & 31)) * LDS_STRIDE + kk * 16 +
                                       8 * (lane >> 5));
#pragma unroll
            for (int m = 0; m < C::MT; m++)
#pragma unroll
                for (int n = 0; n < C::NT; n++)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m], b[n], acc[m][n], 0, 0, 0);
        }
    }

    // ---- epilogues
    const int col = lane & 31;
#pragma unroll
    for (int m = 0; m < C::MT; m++) {
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int r = wm * (BM / 2) + m * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (r >= rows) continue;
            if constexpr (C::GATED) {
                const int feat = blockIdx.y * 64 + wn * 32 + col;
                const float hv = silu_f32(acc[m][0][v]) * acc[m][1][v];
                const int pc = (feat & ~7) | perm8_pos(feat & 7);
                const f16 hh = (f16)hv;
                if constexpr (MODE == MODE_GU)
                    g.h_out[(size_t)(seg + m0 + r) * F + pc] = __builtin_bit_cast(uint16_t, hh);
                else
                    g.hs_out[(size_t)(m0 + r) * FS + pc] = __builtin_bit_cast(uint16_t, hh);
            } else if constexpr (MODE == MODE_DOWN) {
                const int s = seg + m0 + r;
                const float wt = g.wflat[g.perm[s]];
#pragma unroll
                for (int n = 0; n < C::NT; n++) {
                    const int o = blockIdx.y * BN + wn * 64 + n * 32 + col;
                    g.p_out[(size_t)s * D + o] = wt * acc[m][n][v];
                }
            } else {
                const int t = m0 + r;
                const float sg = g.sgate[t];
#pragma unroll
                for (int n = 0; n < C::NT; n++) {
                    const int o = blockIdx.y * BN + wn * 64 + n * 32 + col;
                    float sum = 0.0f;
#pragma unroll
                    for (int rr = 0; rr < K; rr++) sum += g.p_in[(size_t)g.pos_of[t * K + rr] * D + o];
                    sum += sg * acc[m][n][v];
                    g.y[(size_t)t * D + o] = f32_to_bf16_rne(sum);
                }
            }
        }
    }
}

// y = sum_r partial_r, for layers without a shared expert.
__global__ void __launch_bounds__(256) k_combine_routed(const float* __restrict__ p, const int32_t* __restrict__ pos_of,
                                                        uint16_t* __restrict__ y, int T) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= T * D) return;
    const int t = i / D, o = i % D;
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < K; r++) sum += p[(size_t)pos_of[t * K + r] * D + o];
    y[i] = f32_to_bf16_rne(sum);
}

// x bf16 [T, D] -> fp16 [T, D] in perm8 order.
__global__ void __launch_bounds__(256) k_prep_x(const uint16_t* __restrict__ x, uint16_t* __restrict__ xh, int n8) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    ((u32x4*)xh)[i] = bf16x8_to_f16x8_perm(((const u32x4*)x)[i]);
}

constexpr int GEMM_BM = 64;

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
    // routed gate/up
    g.q[0] = p.gate_q; g.sc[0] = p.gate_s; g.bi[0] = p.gate_b;
    g.q[1] = p.up_q; g.sc[1] = p.up_s; g.bi[1] = p.up_b;
    g.h_out = p.h;
    tr.launch(MOE_FFN_KERNEL_EXPERT_GU, k_gemm<MODE_GU, GEMM_BM>, dim3(max_tiles, F / 64), dim3(256), 0, s, g);
    // shared gate/up
    if (p.sh_gate) {
        g.sw[0] = p.sh_gate; g.sw[1] = p.sh_up; g.hs_out = p.hs;
        hipLaunchKernelGGL((k_gemm<MODE_SGU, GEMM_BM>), dim3(mt, FS / 64), dim3(256), 0, s, g);
    }
    // routed down
    g.q[0] = p.down_q; g.sc[0] = p.down_s; g.bi[0] = p.down_b;
    g.p_out = p.partial;
    tr.launch(MOE_FFN_KERNEL_EXPERT_DOWN, k_gemm<MODE_DOWN, GEMM_BM>, dim3(max_tiles, D / 128), dim3(256), 0, s, g);
    // combine
    if (p.sh_gate) {
        g.sw[0] = p.sh_down; g.p_in = p.partial; g.y = p.y;
        tr.launch(MOE_FFN_KERNEL_COMBINE, k_gemm<MODE_SDOWN, GEMM_BM>, dim3(mt, D / 128), dim3(256), 0, s, g);
    } else {
        tr.launch(MOE_FFN_KERNEL_COMBINE, k_combine_routed, dim3((p.T * D + 255) / 256), dim3(256), 0, s,
                  (const float*)p.partial, (const int32_t*)p.pos_of, p.y, p.T);
    }
    return hipGetLastError();
}

}  // namespace moe
