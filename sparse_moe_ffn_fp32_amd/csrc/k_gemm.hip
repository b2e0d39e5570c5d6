// Grouped expert GEMMs on fp16 MFMA with dequantisation fused into the tile
// load (subsystems 3-6 of the prefill path).
//
// Lily engine page, "Dekvantuoti svorius matricos daugybos metu" (dequantise
// weights during the matmul): the 4-bit codes are expanded one small tile at
// a time into on-chip memory, used at once by the MFMAs, and the full
// dequantised matrix never exists; accumulation is fp32.
//
// Block tile: 128 activation rows (tokens) x 256 weight rows (output
// features); 8 waves (two per SIMD), wave (m, n) = (w / 4, w % 4) computing
// activation rows [64m, 64m + 64) against weight rows [64n, 64n + 64) as
// 2 x 2 tiles of v_mfma_f32_32x32x16_f16.  The 4-bit modes on 128-row tiles
// run 8 waves on 512 weight rows, each wave all 128 rows against its 64:
// gemm_block_gu_wide, gemm_block_down_wide.  MFMA layout:
// lane l holds A[l%32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l%32];
// accumulator lane l holds C[i][l%32] for i = 8*(v/4) + 4*(l/32) + v%4,
// v = 0..15.  K advances in steps of 64, one quantisation group.  Both
// operands are fp16 with K inside every 8-block in the perm8 order (see
// moe_common.h).  Every operand row carries a power-of-two exponent that
// puts its largest magnitude in [2^14, 2^15) (row_exp), so no finite input
// or intermediate overflows fp16 or sinks into its subnormals: x rows
// (converted from bf16 exactly), router and shared-expert rows (prepared per
// call), routed weight rows (the group scales and biases of the row scaled
// before s*q + b is formed, one fp16 rounding), h per (row, 256 features),
// the shared h per (row, 128 features) and the partials per (row, 512
// outputs).  The exponents are re-applied to the fp32 results exactly
// (ldexp).  Inside a K step, MFMA sub-step kk and lane half kq = l/32 use K
// in [32kq + 8kk, +8) for both operands.
//
// Per K step the operands go global -> registers in coalesced pieces:
//   A (activations): eight lanes per row, 16 bytes each, so one load
//     instruction covers eight whole 128-byte rows of the step, then LDS;
//     the MFMAs read their fragments from LDS;
//   4-bit weights: each wave loads the raw codes of its own 64 rows (two
//     lanes per row, 16 bytes = 32 weights each, a quarter of the fp16
//     bytes) straight into registers in the MFMA operand layout and expands
//     them there, fp16 s*q + b with the group's scale and bias (staged in
//     LDS once at the block's start), in the step that uses them (the other
//     wave of the SIMD covering it);
//   16-bit weights (shared expert, router planes): fp16 rows prepared per
//     call (k_prep), staged in LDS and read back as fragments.
// Global loads run ahead in a ring of register stages (three steps for 4-bit
// weights, one otherwise); activation tiles are double-buffered; one barrier
// per step.  Epilogues stage the output tile in LDS so global stores are
// 16-byte row pieces.
//
// Modes:
//   GU     routed gate/up over the expert-sorted rows; epilogue SwiGLU
//          h = silu(gate) * up in fp32 -> fp16 with its row exponent (fused
//          chain (i) of the Lily page, "Sumazinti tarpini ir busenos
//          srauta");
//   DOWN   routed down over h; epilogue * routing weight -> fp16 partials
//          (one per assignment, with an exponent per 512 outputs, summed in
//          fp32 by the combine);
//   SGU    shared gate/up over all tokens;
//   SDOWN  shared down; epilogue = the combine: y = sum_{r=0..7} partial_r
//          + sgate * shexp, fixed order, one bf16 rounding, no atomics
//          (fused chain (ii));
//   ROUTER router logits over all tokens: B = the fp32 router weights as two
//          fp16 planes hi + lo (|w' - hi - lo| <= 2^-22 |w'|), paired like
//          gate and up so one lane adds the two planes of an expert;
//          epilogue + router bias -> fp32 logits.
#include <type_traits>

#include "moe_common.h"
#include "moe_kernels.h"
#include "../../include/moe_ffn.h"

namespace moe {

enum { MODE_GU = 0, MODE_DOWN = 1, MODE_SGU = 2, MODE_SDOWN = 3, MODE_ROUTER = 4 };

constexpr int GEMM_BM = 128;          // activation rows per block
constexpr int GEMM_BN = 256;          // weight rows per block
constexpr int BK = 64;
constexpr int LDSB = BK + 8;          // fp16 per LDS operand row (16-byte pad)
// A partial w * down(h) of assignment row r and output column o is stored
// as fp16(w * acc * 2^(ew[o] - ew_max - E_w - PART_BOUND)), acc being the
// fp32 sum over the row-normalised operands (|acc| < 512 * 2^30 = 2^39),
// w < 2^E_w, ew[o] <= ew_max the down rows' exponents: the stored value is
// below 2^15 whatever the magnitudes, typically about 2^5.  Its exponent
// eh_max + ew_max + E_w + PART_BOUND is kept per (row, 512 outputs).
constexpr int PART_BOUND = 24;

// A kernel-argument pointer pinned in scalar registers.  Without this the
// compiler reloads the argument inside every predicated store of an epilogue
// and waits for it there, serialising one scalar round trip per store.
template <typename P>
__device__ __forceinline__ P pinned(P p) {
    asm volatile("" : "+s"(p));
    return p;
}

template <int MODE>
struct GemmCfg {
    static constexpr bool GATED = (MODE == MODE_GU || MODE == MODE_SGU);
    static constexpr bool PAIRED = GATED || MODE == MODE_ROUTER;  // B rows in pairs of 32-row tiles
    static constexpr bool Q4 = (MODE == MODE_GU || MODE == MODE_DOWN);
    static constexpr bool F16SRC = !Q4;                              // B already fp16 in perm8 order
    static constexpr bool ROUTED = (MODE == MODE_GU || MODE == MODE_DOWN);
    static constexpr int KTOT = (GATED || MODE == MODE_ROUTER) ? D : (MODE == MODE_DOWN ? F : FS);
    static constexpr int NK = KTOT / BK;
    static constexpr int NG = KTOT / G;      // quantisation groups per weight row
    static constexpr int SROW = NG + 4;      // u32 per staged scale row (pad)
    static constexpr int BW = Q4 ? 1 : 4;    // 16-byte B words per (row, lane half) per step
    static constexpr int R = Q4 ? 4 : 2;     // register ring stages (loads run R-1 steps ahead)
    static constexpr int NB = MODE == MODE_ROUTER ? E / 128
                            : GATED ? (MODE == MODE_GU ? F : FS) / 128 : D / GEMM_BN;  // column blocks
    static constexpr int NB_XCD = MODE == MODE_SGU ? 2 : NB;  // column blocks per XCD (16-bit modes)
    static_assert(NB % NB_XCD == 0 && 8 % (NB / NB_XCD) == 0, "column groups divide the XCDs");
};

// Blocks of a 16-bit-mode launch over n_tiles row tiles (the mapping of
// gemm_block: every XCD gets slots for its rectangle).
template <int MODE>
__host__ __device__ constexpr int dense_grid(int n_tiles) {
    constexpr int GRP = GemmCfg<MODE>::NB / GemmCfg<MODE>::NB_XCD, PARTS = 8 / GRP;
    return 8 * ((n_tiles + PARTS - 1) / PARTS) * GemmCfg<MODE>::NB_XCD;
}

struct GemmArgs {
    // activations, fp16 rows each with its power-of-two exponent
    const uint16_t* xh;      // fp16 [T, D] (perm8)
    const int32_t* ex;       // [T]
    const uint16_t* h;       // fp16 [N_assign, F] (perm8), expert-sorted rows
    int32_t* eh;             // [N_assign, 2]: per 256 features (GU writes, DOWN reads)
    const uint16_t* hs;      // fp16 [T, FS] (perm8)
    int32_t* ehs;            // [T, 4]: per 128 features (SGU writes, SDOWN reads)
    int32_t* ep;             // [N_assign, 4]: partials per 512 outputs (DOWN writes, combine reads)
    // routing
    const int32_t* perm;     // sorted position -> assignment
    const int32_t* pos_of;   // assignment -> sorted position
    const int32_t* offs;     // [E+1] expert segment starts
    const int32_t* tiles;    // [4i..4i+3] expert, first row, segment start, rows; longest first
    const int32_t* tiles_e;  // the same records in expert order
    const int32_t* tile_count;
    const float* wsort;      // [T*K] routing weights by expert-sorted position
    const float* sgate;      // [T]
    int gu_rows;             // GU: rows per expert in the gate/up arrays (F, or 2F fused)
    // weights
    const uint32_t* q[2];    // GU: gate, up; DOWN: down
    const uint16_t* sc[2];
    const uint16_t* bi[2];
    const uint16_t* shw;     // SGU, SDOWN: shared fp16 [gate FS x D | up FS x D | down D x FS] (perm8)
    const int32_t* es;       // their row exponents [2 FS + D]
    // outputs
    uint16_t* h_out;         // GU
    uint16_t* p_out;         // DOWN: fp16 partials [N_assign, D]
    int stream_nt;           // GU, DOWN: store h and the partials non-temporal (long passes)
    uint16_t* hs_out;        // SGU
    uint16_t* y;             // SDOWN: bf16 [T, D]
    const uint16_t* resid;   // SDOWN: bf16 [T, D] added before the rounding of y, or null
    const uint16_t* p_in;    // SDOWN: fp16 partials
    const uint16_t* wr2;     // ROUTER: fp16 [2, E, D] (hi, lo planes; perm8)
    const int32_t* er;       // ROUTER: row exponents [E]
    const float* rbias;      // ROUTER: fp32 [E] or null
    float* logits;           // ROUTER: fp32 [T, E]
    int T;
};

// LDS room the 4-bit kernels keep beside their tiles for the epilogues'
// output staging (sized as four 512-row code buffers of 48-byte rows)
constexpr int BQS = 12;
constexpr int QBUF = 4;

// LDS of one block of the 16-bit modes: double-buffered activation tiles and
// a double-buffered fp16 weight tile.  The epilogues reuse the operand tiles
// (a, then b).
template <int MODE>
struct GemmSmem {
    f16 a[2][GEMM_BM * LDSB];
    f16 b[2][GEMM_BN * LDSB];
    // SDOWN: with a and b, room for the combine's fp32 shared tile [128][260]
    float yx[MODE == MODE_SDOWN ? GEMM_BM * (GEMM_BN + 4) - (2 * (GEMM_BM + GEMM_BN) * LDSB) / 2 : 1];
    int32_t ea[GEMM_BM];                                // the activation rows' exponents
    uint32_t fac[MODE == MODE_SDOWN ? GEMM_BM : 1][4];  // SDOWN: fp16 2^(ehs - ehs_max) per 128 features, both halves
    int32_t pos[MODE == MODE_SDOWN ? GEMM_BM * K : 4];  // SDOWN: each row's partial positions
    int32_t epp[MODE == MODE_SDOWN ? GEMM_BM * K : 4];  // SDOWN: and those partials' exponents
};

// One block's work; `bid` is the block's index within its mode's grid
// (a multiple-of-8 offset from blockIdx.x, so bid % 8 is still the XCD).
//
// 8 waves, two per SIMD (GEMM_THREADS): wave w = (wm, wn) = (w / 4, w % 4)
// computes activation rows [64wm, 64wm + 64) against LDS weight rows
// [64wn, 64wn + 64): 32-row tiles acc[mt][nt] for activation rows
// 64wm + 32mt and weight rows 64wn + 32nt.  Paired modes map LDS row
// 64wn + 32nt + j to gate (nt = 0) or up (nt = 1) of feature 32wn + j of the
// block (ROUTER: the hi or lo plane of expert 32wn + j), so one lane holds
// both values of a feature.  (With four waves, one per SIMD, each wave
// computing all 128 rows, every LDS wait and barrier left the matrix pipe
// idle: about 48 us per block against 16 us of MFMAs.)
constexpr int GEMM_THREADS = 512;
template <int MODE>
__device__ __forceinline__ void gemm_block(const GemmArgs& g, GemmSmem<MODE>& sm, int bid) {
    using C = GemmCfg<MODE>;
    static_assert(!C::Q4, "the 4-bit modes run in gemm_block_gu_wide / gemm_block_down_wide");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    const int l32 = lane & 31, kq = lane >> 5;

    // ---- which (row tile, column block) this block owns.  Workgroups are
    // dealt to the 8 XCDs round-robin by id (XCD bid % 8).  Each XCD owns a
    // rectangle of the (tile, column block) grid, small enough in columns
    // that its weights stay in the XCD's 4 MB L2 (router 2 MB, shared down
    // 2 MB: every column block; shared gate/up 4 MB: two of its four
    // blocks), and runs it tile by tile, column block fastest, so the blocks
    // sharing a tile's activations meet in that L2 too.
    constexpr int NB = C::NB;
    constexpr int NGX = C::NB_XCD, GRP = NB / NGX, PARTS = 8 / GRP;
    const int n_tiles = (g.T + GEMM_BM - 1) / GEMM_BM;
    const int tpp = (n_tiles + PARTS - 1) / PARTS;  // tiles per XCD
    const int x = bid & 7, slot = bid >> 3;
    const int tile = (x / GRP) * tpp + slot / NGX, nblk = (x % GRP) * NGX + slot % NGX;
    if (slot >= tpp * NGX || tile >= n_tiles) return;
    const int m0 = tile * GEMM_BM;
    const int rows = min(GEMM_BM, g.T - m0);  // >= 1 for tile < n_tiles

    // ---- A: this thread loads 16 bytes (chunk ac) of rows ar0 + 64i, i < 2;
    // rows past the end repeat the last valid row (their results are dropped)
    const int ac = tid & 7, ar0 = tid >> 3;
    const uint16_t* apt[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int r = min(ar0 + 64 * i, rows - 1);
        const uint16_t* p;
        if constexpr (MODE == MODE_SGU || MODE == MODE_ROUTER) p = g.xh + (size_t)(m0 + r) * D;
        else p = g.hs + (size_t)(m0 + r) * FS;
        apt[i] = p + 8 * ac;
    }

    // ---- B: this thread covers lane half bh (K [32bh, 32bh+32) of a step) of
    // LDS weight row br0, an fp16 row of the prepared arrays
    const int bh = tid & 1, br0 = tid >> 1;
    auto wrow = [&](int n) -> const uint16_t* {  // global fp16 weight row of LDS row n
        if constexpr (C::PAIRED) {
            const int mat = (n >> 5) & 1;
            const int feat = nblk * 128 + 32 * (n >> 6) + (n & 31);
            if constexpr (MODE == MODE_ROUTER) return g.wr2 + ((size_t)mat * E + feat) * D;  // plane, expert
            else return g.shw + ((size_t)mat * FS + feat) * D;                               // gate / up
        } else {
            return g.shw + 2 * (size_t)FS * D + (size_t)(nblk * GEMM_BN + n) * FS;           // shared down
        }
    };
    const u32x4* bpt = (const u32x4*)wrow(br0) + 4 * bh;

    // ---- the activation rows' exponents; SDOWN: the shared h rows come in
    // four 128-feature pieces with exponents of their own, brought to the
    // row's largest one when staged (factor 2^(e_piece - e_max) <= 1), and the
    // combine's partial rows with their exponents, read long before the
    // epilogue needs them (rows past the end repeat the last valid row)
    if (tid < GEMM_BM) {
        const int t = m0 + min(tid, rows - 1);
        if constexpr (MODE == MODE_SDOWN) {
            const int4 e4 = *(const int4*)&g.ehs[(size_t)t * 4];
            const int em = max(max(e4.x, e4.y), max(e4.z, e4.w));
            sm.ea[tid] = em;
            const int ev[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const f16 f = pow2_f16(ev[b] - em);
                sm.fac[tid][b] = __builtin_bit_cast(uint32_t, f16x2{f, f});
            }
        } else {
            sm.ea[tid] = g.ex[t];
        }
    }
    // SDOWN: the exponents of this lane's two shared-down weight rows, loaded
    // here so the epilogue's staging waits for no global load (the partial
    // loads issued before it would be drained with it)
    int ew_sd[2] = {0, 0};
    if constexpr (MODE == MODE_SDOWN) {
#pragma unroll
        for (int nt = 0; nt < 2; nt++) ew_sd[nt] = g.es[2 * FS + nblk * GEMM_BN + 64 * wn + 32 * nt + l32];
    }
    if constexpr (MODE == MODE_SDOWN) {
        const int pblk = (nblk * GEMM_BN) / 512;  // the partials' 512-column exponent block
#pragma unroll
        for (int i = 0; i < GEMM_BM * K / GEMM_THREADS; i++) {
            const int q = tid + GEMM_THREADS * i;
            const int pos = g.pos_of[(size_t)(m0 + min(q / K, rows - 1)) * K + q % K];
            sm.pos[q] = pos;
            sm.epp[q] = g.ep[(size_t)pos * 4 + pblk];
        }
    }
    __syncthreads();  // exponents and factors before the first A store

    f32x16 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nt = 0; nt < 2; nt++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[mt][nt][v] = 0.0f;

    // Four MFMAs per sub-step kk against the activation tile in LDS buffer
    // abuf; the fragments of sub-step kk + 1 are read before the MFMAs of kk.
    auto mfma_step = [&](int abuf, const f16x8 (&bf)[2][4]) {
        const f16* ab = &sm.a[abuf][(64 * wm + l32) * LDSB + 32 * kq];
        f16x8 af[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; mt++) af[0][mt] = *(const f16x8*)(ab + mt * 32 * LDSB);
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            if (kk < 3)
#pragma unroll
                for (int mt = 0; mt < 2; mt++) af[(kk + 1) & 1][mt] = *(const f16x8*)(ab + mt * 32 * LDSB + 8 * (kk + 1));
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int nt = 0; nt < 2; nt++)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[kk & 1][mt], bf[nt][kk], acc[mt][nt], 0, 0, 0);
        }
    };

    // ---- operands: global -> registers R - 1 steps ahead -> LDS
    constexpr int R = 2;
    static_assert(C::NK % R == 0, "K steps must be a multiple of the ring size");
    struct Stage { u32x4 a[2]; u32x4 b[4]; };
    auto load = [&](int k, Stage& st) {
#pragma unroll
        for (int i = 0; i < 2; i++) st.a[i] = *(const u32x4*)(apt[i] + k * BK);
#pragma unroll
        for (int w = 0; w < 4; w++) st.b[w] = bpt[8 * k + w];
    };
    auto store = [&](const Stage& st, int k, int buf) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            u32x4 v = st.a[i];
            if constexpr (MODE == MODE_SDOWN) {  // this 128-feature piece to the row's exponent
                const f16x2 f = __builtin_bit_cast(f16x2, sm.fac[ar0 + 64 * i][k >> 1]);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t vj = v[j];
                    v[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, vj) * f);
                }
            }
            *(u32x4*)&sm.a[buf][(ar0 + 64 * i) * LDSB + 8 * ac] = v;
        }
        f16* dst = &sm.b[buf][br0 * LDSB + 32 * bh];
#pragma unroll
        for (int w = 0; w < 4; w++) *(u32x4*)(dst + 8 * w) = st.b[w];
    };
    auto read_b = [&](int buf, f16x8 (&bf)[2][4]) {
#pragma unroll
        for (int nt = 0; nt < 2; nt++) {
            const f16* bb = &sm.b[buf][(64 * wn + 32 * nt + l32) * LDSB + 32 * kq];
#pragma unroll
            for (int kk = 0; kk < 4; kk++) bf[nt][kk] = *(const f16x8*)(bb + 8 * kk);
        }
    };
    Stage ring[R];
#pragma unroll
    for (int k = 0; k < R - 1; k++) load(k, ring[k]);
    store(ring[0], 0, 0);
    __syncthreads();
#pragma unroll 1
    for (int k0 = 0; k0 < C::NK; k0 += R) {
#pragma unroll
        for (int j = 0; j < R; j++) {
            const int k = k0 + j;
            load(min(k + R - 1, C::NK - 1), ring[(j + R - 1) % R]);
            __builtin_amdgcn_sched_barrier(0);
            f16x8 bf[2][4];
            read_b(j & 1, bf);
            mfma_step(j & 1, bf);
            store(ring[(j + 1) % R], min(k + 1, C::NK - 1), (j + 1) & 1);
            __syncthreads();
        }
    }

    // ---- epilogues (the loop ended with a barrier: the operand tiles are
    // free).  Accumulator element v of acc[mt][nt] is activation row
    // r = 32mt + 8(v/4) + 4kq + v%4 and LDS weight row 64w + 32nt + l32.
    auto acc_row = [&](int mt, int v) { return 64 * wm + mt * 32 + 8 * (v >> 2) + 4 * kq + (v & 3); };
    if constexpr (MODE == MODE_ROUTER) {
        const int ex = nblk * 128 + 32 * wn + l32;
        const float b = g.rbias ? g.rbias[ex] : 0.0f;
        const int ew = g.er[ex];
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int r = acc_row(mt, v);
                if (r < rows)
                    g.logits[(size_t)(m0 + r) * E + ex] = __builtin_ldexpf(acc[mt][0][v] + acc[mt][1][v], sm.ea[r] + ew) + b;
            }
    } else if constexpr (C::GATED) {
        // h tile [128 rows][128 features] fp32 in LDS; then per row piece of
        // 8 features: the row's largest |h| over the block's 128 features
        // (16 lanes), its exponent, fp16 in perm8 order, 16-byte stores
        constexpr int HS = 128 + 4;
        static_assert(GEMM_BM * HS * sizeof(float) <= offsetof(GemmSmem<MODE>, ea), "h tile must fit a, b");
        float* hb = (float*)&sm.a[0][0];
        const int f = 32 * wn + l32;  // feature inside the block
        const int eg = g.es[nblk * 128 + f], eu = g.es[FS + nblk * 128 + f];
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int r = acc_row(mt, v);
                const float gv = __builtin_ldexpf(acc[mt][0][v], sm.ea[r] + eg);
                const float uv = __builtin_ldexpf(acc[mt][1][v], sm.ea[r] + eu);
                hb[r * HS + f] = silu_f32(gv) * uv;
            }
        // buffer stores: a flat store also counts as an LDS access, so the
        // LDS reads of the next rows would wait for it
        const __amdgpu_buffer_rsrc_t rhs = buffer_rsrc(g.hs_out), rehs = buffer_rsrc(g.ehs);
        __syncthreads();
        // 128 rows x 16 pieces: thread tid takes rows tid/16 + 32i, piece tid%16
        const int c = tid & 15, rb = tid >> 4;
#pragma unroll
        for (int i = 0; i < GEMM_BM * 16 / GEMM_THREADS; i++) {
            const int r = rb + 32 * i;
            const f32x4 p0 = *(const f32x4*)&hb[r * HS + 8 * c], p1 = *(const f32x4*)&hb[r * HS + 8 * c + 4];
            const float v[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j++) m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
            const int e = row_exp(row16_max(m));
            const u32x4 o = f32x8_to_f16x8_perm_scaled(v, e);
            if (r < rows) {
                __builtin_amdgcn_raw_buffer_store_b128(o, rhs, ((uint32_t)(m0 + r) * FS + nblk * 128 + 8 * c) * 2, 0, 0);
                if (c == 0) __builtin_amdgcn_raw_buffer_store_b32((uint32_t)e, rehs, ((uint32_t)(m0 + r) * 4 + nblk) * 4, 0, 0);
            }
        }
    } else {
        // combine: y = sum_r partial_r * 2^ep_r + sgate * shexp.  The fp32
        // shared tile of all 256 columns goes to LDS once; then 128 rows x 32
        // pieces of 8 outputs, thread tid taking pieces tid + 512 i (row
        // (tid + 512 i) / 32, piece tid % 32), CB at a time, the loads of the
        // next CB pieces (8 partials, residual, gate each) issued before the
        // current ones are summed; the first are issued before the tile is
        // staged.  Rows past the end load the last valid row and store nothing.
        constexpr int YS = GEMM_BN + 4;
        static_assert(GEMM_BM * YS * sizeof(float) <= offsetof(GemmSmem<MODE>, ea), "shared tile must fit a, b, y");
        float* yb = (float*)&sm.a[0][0];  // 128 x 260 fp32 = 133 KB
        constexpr int CB = 2, NPIECE = GEMM_BM * (GEMM_BN / 8) / GEMM_THREADS, NBATCH = NPIECE / CB;
        static_assert(NPIECE % CB == 0, "whole batches");
        // buffer loads and stores: vector-memory only (a flat access also
        // counts as an LDS access, so every LDS read of the next batch's
        // positions would wait for the partials in flight); without a
        // residual its resource has no records and reads as zeros
        const __amdgpu_buffer_rsrc_t rp = buffer_rsrc(g.p_in), ry = buffer_rsrc(g.y);
        const __amdgpu_buffer_rsrc_t rres = g.resid ? buffer_rsrc(g.resid) : empty_rsrc(g.y);
        const int c = tid & 31;
        const int o = nblk * GEMM_BN + 8 * c;  // this thread's first output column
        u32x4 pv[2][CB][K], rv[2][CB];
        float sg[2][CB];
        auto issue = [&](int bi, int buf) {
#pragma unroll
            for (int u = 0; u < CB; u++) {
                const int r = min((tid + GEMM_THREADS * (CB * bi + u)) >> 5, rows - 1);
                const int t = m0 + r;
#pragma unroll
                for (int rr = 0; rr < K; rr++)
                    pv[buf][u][rr] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, ((uint32_t)sm.pos[r * K + rr] * D + o) * 2, 0, 0));
                rv[buf][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rres, ((uint32_t)t * D + o) * 2, 0, 0));
                sg[buf][u] = g.sgate[t];
            }
        };
        auto finish = [&](int bi, int buf) {
#pragma unroll
            for (int u = 0; u < CB; u++) {
                const int r = (tid + GEMM_THREADS * (CB * bi + u)) >> 5;
                const int rl = min(r, rows - 1);
                float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int rr = 0; rr < K; rr++) {
                    const int ep = sm.epp[rl * K + rr];
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        // copy the element to a scalar first: a bit cast of the
                        // vector-element expression itself is miscompiled by
                        // clang 22 (it reads element 0 for every j)
                        const uint32_t pw = pv[buf][u][rr][j];
                        const f16x2 h2 = __builtin_bit_cast(f16x2, pw);
                        sum[2 * j] += __builtin_ldexpf((float)h2[0], ep);
                        sum[2 * j + 1] += __builtin_ldexpf((float)h2[1], ep);
                    }
                }
                // the residual (added last, before the one rounding)
                u32x4 out;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t rj = rv[buf][u][j];
                    const float y0 = sum[2 * j] + sg[buf][u] * yb[rl * YS + 8 * c + 2 * j] + bf16_to_f32(rj & 0xffffu);
                    const float y1 =
                        sum[2 * j + 1] + sg[buf][u] * yb[rl * YS + 8 * c + 2 * j + 1] + bf16_to_f32(rj >> 16);
                    out[j] = (uint32_t)f32_to_bf16_rne(y0) | ((uint32_t)f32_to_bf16_rne(y1) << 16);
                }
                if (r < rows) __builtin_amdgcn_raw_buffer_store_b128(out, ry, ((uint32_t)(m0 + r) * D + o) * 2, 0, 0);
            }
        };
        issue(0, 0);
#pragma unroll
        for (int nt = 0; nt < 2; nt++) {
            const int col = 64 * wn + 32 * nt + l32;
            const int ew = ew_sd[nt];
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int v = 0; v < 16; v++) {
                    const int r = acc_row(mt, v);
                    yb[r * YS + col] = __builtin_ldexpf(acc[mt][nt][v], sm.ea[r] + ew);
                }
        }
        __syncthreads();
#pragma unroll
        for (int bi = 0; bi < NBATCH; bi++) {
            if (bi + 1 < NBATCH) issue(bi + 1, (bi + 1) & 1);
            finish(bi, bi & 1);
        }
    }
}

// The (tile, column block) item of routed block `bid`.  Workgroups are dealt
// to the 8 XCDs in turn by id (XCD bid % 8) and started in id order as
// compute units free up.  The tile map lists the longest tiles first; pairs
// of consecutive tiles (TPAIR) are dealt to the XCDs in turn, and each XCD
// runs all NB column blocks of a tile back to back: the tile's activation
// rows and, within a pair, an expert's weights meet in one L2, and every XCD
// works through the list from its longest tiles to its shortest.  Ids that
// map past the last tile return false.
constexpr int TPAIR = 2;
template <int NB>
__device__ __forceinline__ bool tile_of_block(int bid, int n_tiles, int& tile, int& nblk) {
    const int xcd = bid & 7, slot = bid >> 3;
    const int k = slot / NB;  // the XCD's k-th tile
    nblk = slot % NB;
    tile = (k / TPAIR) * (8 * TPAIR) + xcd * TPAIR + k % TPAIR;
    return tile < n_tiles;
}
// Blocks of a routed launch: every XCD gets slots for its share of max_tiles.
template <int NB>
__host__ __device__ constexpr int routed_grid(int max_tiles) {
    return 8 * ((max_tiles + 8 * TPAIR - 1) / (8 * TPAIR)) * TPAIR * NB;
}

// ---------------------------------------------------------------- wide down
// The routed down projection on 128-row tiles with 512 output columns per
// block: 8 waves, wave w computing all 128 rows against weight rows
// [64w, 64w + 64) over the whole K (K = F: 8 steps).  Against two 256-column
// blocks the tile's h rows are read once instead of twice and the block's
// fixed costs (tile record, routing weights, prologue loads, epilogue) are
// paid once; the 16-byte code rows, the ring and the epilogue are those of
// gemm_block.
constexpr int WBN = 512;  // output columns per wide block
struct WideSmem {
    f16 a[2][GEMM_BM * LDSB];
    uint32_t pad[QBUF][WBN * BQS];   // unused in the loop: with a, room for the epilogue's partial tile
    uint32_t sb[WBN * (F / G + 4)];  // (bias' << 16) | scale', fp16 bits (row-scaled)
    float rw[GEMM_BM];               // routing weight * 2^-(E_w + PART_BOUND) per row
    int32_t eprow[GEMM_BM];          // eh_max + E_w + PART_BOUND per row
    uint32_t fac[GEMM_BM];           // fp16 2^(eh_half - eh_max) for halves 0 (low) and 1 (high)
    int32_t ew[WBN];                 // the down rows' exponents
    int32_t red[8];
};

// A row's group scales and biases (bf16) -> the row exponent and the scaled
// pairs (bias' << 16) | scale' in fp16 (exact: bf16 has fewer significant
// bits), so that every dequantised weight s' q + b' of the row lies below
// 2^15 (the affine map is monotone in q, so its extremes are b and 15 s + b).
template <int NG>
__device__ __forceinline__ int scale_row_params(const uint32_t (&sw)[NG / 2], const uint32_t (&bw)[NG / 2],
                                                uint32_t (&out)[NG]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < NG; i++) {
        const float sv = (i & 1) ? __uint_as_float(sw[i >> 1] & 0xffff0000u) : __uint_as_float(sw[i >> 1] << 16);
        const float bv = (i & 1) ? __uint_as_float(bw[i >> 1] & 0xffff0000u) : __uint_as_float(bw[i >> 1] << 16);
        m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(bv), __builtin_fabsf(__builtin_fmaf(15.0f, sv, bv))));
    }
    const int e = row_exp(m);
#pragma unroll
    for (int i = 0; i < NG; i++) {
        const float sv = (i & 1) ? __uint_as_float(sw[i >> 1] & 0xffff0000u) : __uint_as_float(sw[i >> 1] << 16);
        const float bv = (i & 1) ? __uint_as_float(bw[i >> 1] & 0xffff0000u) : __uint_as_float(bw[i >> 1] << 16);
        const f16x2 p = {(f16)__builtin_ldexpf(sv, -e), (f16)__builtin_ldexpf(bv, -e)};
        out[i] = __builtin_bit_cast(uint32_t, p);
    }
    return e;
}

// Group g's fp16 scale and bias from a staged pair, each in both halves.
__device__ __forceinline__ void group_sb(uint32_t sbw, f16x2& s2, f16x2& b2) {
    s2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sbw, sbw, 0x01000100u));
    b2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(sbw, sbw, 0x03020302u));
}

__device__ __forceinline__ void gemm_block_down_wide(const GemmArgs& g, WideSmem& sm, int bid) {
    using C = GemmCfg<MODE_DOWN>;
    constexpr int SROW = C::NG + 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, kq = lane >> 5;

    // (tile, column block) item: the tiles in expert order, XCD p % 8 taking
    // one contiguous run of items, column block fastest: the blocks sharing
    // a tile's h rows, and the tiles sharing an expert's weights (590 KB, the
    // larger operand here), meet in one L2
    constexpr int NB = D / WBN;
    const int n_tiles = g.tile_count[0];
    const int live = n_tiles * NB, per_xcd = (live + 7) >> 3;
    const int slot = bid >> 3, item = (bid & 7) * per_xcd + slot;
    if (slot >= per_xcd || item >= live) return;
    const int tile = item / NB, nblk = item % NB;
    const int4 rec = *(const int4*)&g.tiles_e[4 * tile];  // one dependent load
    const int e = rec.x, m0 = rec.y, seg = rec.z, rows = rec.w;  // rows: 1 .. GEMM_BM

    // ---- A (h rows): thread loads 16 bytes (chunk ac) of rows ar0 + 64i
    const int ac = tid & 7, ar0 = tid >> 3;
    const uint16_t* apt[2];
#pragma unroll
    for (int i = 0; i < 2; i++) apt[i] = g.h + (size_t)(seg + m0 + min(ar0 + 64 * i, rows - 1)) * F + 8 * ac;
    // ---- B: each wave loads the codes of its own rows 64 w + 32 nt + l32
    // straight into registers in the layout its MFMAs take (lane half kq:
    // 16 bytes = 32 weights of the step)
    const u32x4* bpt[2];
#pragma unroll
    for (int nt = 0; nt < 2; nt++)
        bpt[nt] = (const u32x4*)(g.q[0] + ((size_t)e * D + nblk * WBN + 64 * wave + 32 * nt + l32) * (F / 8)) + kq;
    // ---- scales and biases of LDS row n = tid, scaled by the row's exponent
    // ew (and the block's largest, ew_max); per tile row: the h exponents of
    // its two 256-feature halves (the staged A rows are brought to the larger
    // one) and the routing weight w with its binary exponent E_w
    {
        const size_t row = (size_t)e * D + nblk * WBN + tid;
        const u32x4 sv = *(const u32x4*)(g.sc[0] + row * C::NG), bv = *(const u32x4*)(g.bi[0] + row * C::NG);
        const uint32_t sw[4] = {sv[0], sv[1], sv[2], sv[3]}, bw[4] = {bv[0], bv[1], bv[2], bv[3]};
        uint32_t pr[C::NG];
        const int ew = scale_row_params<C::NG>(sw, bw, pr);
        uint32_t* dst = &sm.sb[tid * SROW];
        *(u32x4*)(dst) = u32x4{pr[0], pr[1], pr[2], pr[3]};
        *(u32x4*)(dst + 4) = u32x4{pr[4], pr[5], pr[6], pr[7]};
        sm.ew[tid] = ew;
        const int wm = wave_max(ew);
        if (lane == 0) sm.red[wave] = wm;
    }
    if (tid < GEMM_BM) {
        const int sr = seg + m0 + min(tid, rows - 1);
        const int2 e2 = *(const int2*)&g.eh[(size_t)sr * 2];
        const int em = max(e2.x, e2.y);
        sm.fac[tid] = __builtin_bit_cast(uint32_t, f16x2{pow2_f16(e2.x - em), pow2_f16(e2.y - em)});
        const float w = g.wsort[sr];  // sorted by the routing sort: no dependent load
        int ewt;
        __builtin_frexpf(w, &ewt);  // w < 2^ewt
        sm.rw[tid] = __builtin_ldexpf(w, -ewt - PART_BOUND);
        sm.eprow[tid] = em + ewt + PART_BOUND;
    }

    f32x16 acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < 2; nt++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[mt][nt][v] = 0.0f;

    auto mfma_step = [&](auto nmt_c, int abuf, const f16x8 (&bf)[2][4]) {
        constexpr int NMT = decltype(nmt_c)::value;
        const f16* ab = &sm.a[abuf][l32 * LDSB + 32 * kq];
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            f16x8 af[NMT];
#pragma unroll
            for (int mt = 0; mt < NMT; mt++) af[mt] = *(const f16x8*)(ab + mt * 32 * LDSB + 8 * kk);
#pragma unroll
            for (int mt = 0; mt < NMT; mt++)
#pragma unroll
                for (int nt = 0; nt < 2; nt++)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mt], bf[nt][kk], acc[mt][nt], 0, 0, 0);
        }
    };
    // the A rows of step k times their half's factor (k < 4: features
    // 0..255, else 256..511)
    auto store_a = [&](const u32x4 (&av)[2], int k, int buf) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const uint32_t fw = sm.fac[ar0 + 64 * i];
            const f16x2 f = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(fw, fw, k < 4 ? 0x01000100u : 0x03020302u));
            u32x4 v = av[i];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t vj = v[j];
                v[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, vj) * f);
            }
            *(u32x4*)&sm.a[buf][(ar0 + 64 * i) * LDSB + 8 * ac] = v;
        }
    };
    auto load_a = [&](int k, u32x4 (&av)[2]) {
#pragma unroll
        for (int i = 0; i < 2; i++) av[i] = *(const u32x4*)(apt[i] + k * BK);
    };
    auto load_b = [&](int k, u32x4 (&bv)[2]) {
#pragma unroll
        for (int i = 0; i < 2; i++) bv[i] = bpt[i][2 * k];
    };
    auto dequant = [&](int k, const u32x4 (&cb)[2], f16x8 (&bf)[2][4]) {
#pragma unroll
        for (int nt = 0; nt < 2; nt++) {
            const int n = 64 * wave + 32 * nt + l32;
            const u32x4 codes = cb[nt];
            f16x2 s2, b2;
            group_sb(sm.sb[n * SROW + k], s2, b2);
#pragma unroll
            for (int kk = 0; kk < 4; kk++) {
                const uint32_t cw = codes[kk];
                bf[nt][kk] = __builtin_bit_cast(f16x8, q4_word_to_f16x8(cw, s2, b2));
            }
        }
    };
    // ring stage j holds A(j) and the codes of step j; loads run three steps
    // ahead; A(j) sits in LDS buffer j % 2 during step j, the codes stay in
    // the ring
    constexpr int R = 4;
    static_assert(C::NK % R == 0, "K steps must be a multiple of the ring size");
    struct Stage { u32x4 a[2]; u32x4 b[2]; };
    auto main_loop = [&](auto nmt_c) {
        Stage ring[R];
#pragma unroll
        for (int j = 0; j < R - 1; j++) {
            load_a(j, ring[j].a);
            load_b(j, ring[j].b);
        }
        __syncthreads();  // staged scales, biases, exponents, routing weights
        store_a(ring[0].a, 0, 0);
        __syncthreads();
#pragma unroll 1
        for (int k0 = 0; k0 < C::NK; k0 += R) {
#pragma unroll
            for (int j = 0; j < R; j++) {
                const int k = k0 + j;
                Stage& nx = ring[(j + R - 1) % R];
                load_a(min(k + R - 1, C::NK - 1), nx.a);
                load_b(min(k + R - 1, C::NK - 1), nx.b);
                __builtin_amdgcn_sched_barrier(0);
                f16x8 bfr[2][4];
                dequant(k, ring[j].b, bfr);
                mfma_step(nmt_c, j & 1, bfr);
                store_a(ring[(j + 1) % R].a, min(k + 1, C::NK - 1), (j + 1) & 1);
                __syncthreads();
            }
        }
    };
    const int nmt = (rows + 31) >> 5;
    if (nmt >= 4) main_loop(std::integral_constant<int, 4>{});
    else if (nmt == 3) main_loop(std::integral_constant<int, 3>{});
    else if (nmt == 2) main_loop(std::integral_constant<int, 2>{});
    else main_loop(std::integral_constant<int, 1>{});

    // ---- epilogue: partial tile [128 rows][512 outputs] fp16 (routing
    // weight, exponents as PART_BOUND states) in LDS (a and pad), then 16-byte
    // row pieces; the rows' exponents
    constexpr int PS = WBN + 8;
    static_assert(GEMM_BM * PS * sizeof(f16) <= offsetof(WideSmem, sb), "partial tile must fit a, pad");
    f16* pb = &sm.a[0][0];
    auto acc_row = [&](int mt, int v) { return mt * 32 + 8 * (v >> 2) + 4 * kq + (v & 3); };
    int ewmax = sm.red[0];
#pragma unroll
    for (int w = 1; w < 8; w++) ewmax = max(ewmax, sm.red[w]);
#pragma unroll
    for (int nt = 0; nt < 2; nt++) {
        const int col = 64 * wave + 32 * nt + l32;
        const int sh = sm.ew[col] - ewmax;  // <= 0
#pragma unroll
        for (int mt = 0; mt < 4; mt++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int r = acc_row(mt, v);
                pb[r * PS + col] = (f16)__builtin_ldexpf(sm.rw[r] * acc[mt][nt][v], sh);
            }
    }
    uint16_t* const p_out = pinned(g.p_out);
    const __amdgpu_buffer_rsrc_t rp_out = buffer_rsrc(p_out);
    if (tid < rows) g.ep[(size_t)(seg + m0 + tid) * 4 + nblk] = sm.eprow[tid] + ewmax;
    __syncthreads();
    // 128 rows x 64 pieces of 8 outputs: thread tid takes rows tid/64 + 8i,
    // piece tid%64; LDS reads in two halves of 8, each before its stores
    const int c = tid & 63, rb = tid >> 6;
#pragma unroll
    for (int h = 0; h < 2; h++) {
        u32x4 pv[8];
#pragma unroll
        for (int i = 0; i < 8; i++) pv[i] = *(const u32x4*)&pb[(rb + 8 * (8 * h + i)) * PS + 8 * c];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int r = rb + 8 * (8 * h + i);
            if (r < rows) {
                // the cache policy is an immediate of the store, one per
                // branch (two plain stores under a branch were merged into
                // one, losing the hint); byte offsets stay below 2^31 (at most
                // 32768 tokens per pass)
                const int off = (int)(((size_t)(seg + m0 + r) * D + nblk * WBN + 8 * c) * sizeof(uint16_t));
                if (g.stream_nt) __builtin_amdgcn_raw_buffer_store_b128(pv[i], rp_out, off, 0, 2);
                else __builtin_amdgcn_raw_buffer_store_b128(pv[i], rp_out, off, 0, 0);
            }
        }
    }
}

__global__ void __launch_bounds__(512) k_gemm_down_wide(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) WideSmem sm;
    gemm_block_down_wide(g, sm, blockIdx.x);
}

// ---------------------------------------------------------------- wide gate/up
// The routed gate/up on 128-row tiles with 256 features (512 gate and up
// rows) per block: 8 waves, wave w computing all 128 rows against weight
// rows [64w, 64w + 64) (gate and up of features 32w .. 32w + 31) over the
// whole K.  Against two 128-feature blocks the tile's gathered x rows (512
// KB per tile) are read once instead of twice.  Each wave loads the codes
// of its own rows into its register ring and expands each step's codes in
// the step itself (the other wave of the SIMD covers it); staging them in
// LDS first had cost 4 % of the launch.  The LDS holds the x tiles, the
// scales and biases of all 32 groups, and the epilogue's h tile.
struct WideGuSmem {
    f16 a[2][GEMM_BM * LDSB];
    uint32_t pad[2][WBN * BQS];      // unused in the loop: with a and sb, room for the epilogue's h tile
    uint32_t sb[WBN * (D / G + 4)];  // (bias' << 16) | scale', fp16 bits (row-scaled)
    int32_t ea[GEMM_BM];             // the gathered x rows' exponents
    int32_t ew[WBN];                 // the gate/up rows' exponents
};

__device__ __forceinline__ void gemm_block_gu_wide(const GemmArgs& g, WideGuSmem& sm, int bid) {
    using C = GemmCfg<MODE_GU>;
    constexpr int SROW = C::NG + 4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, kq = lane >> 5;

    constexpr int NB = F / (WBN / 2);
    int tile, nblk;
    if (!tile_of_block<NB>(bid, g.tile_count[0], tile, nblk)) return;
    const int4 rec = *(const int4*)&g.tiles[4 * tile];  // one dependent load
    const int e = rec.x, m0 = rec.y, seg = rec.z, rows = rec.w;  // rows: 1 .. GEMM_BM

    // ---- A (x rows gathered through the sort): 16 bytes (chunk ac) of rows
    // ar0 + 64i; rows past the end repeat the last valid row
    const int ac = tid & 7, ar0 = tid >> 3;
    const uint16_t* apt[2];
#pragma unroll
    for (int i = 0; i < 2; i++)
        apt[i] = g.xh + (size_t)(g.perm[seg + m0 + min(ar0 + 64 * i, rows - 1)] / K) * D + 8 * ac;
    // ---- B: block row n is gate (n & 32 == 0) or up row of feature
    // nblk * 256 + 32 (n >> 6) + (n & 31).  Each wave loads the codes of its
    // own rows 64 w + 32 nt + l32 straight into registers in the layout its
    // MFMAs take (lane half kq: 16 bytes = 32 weights of the step), the same
    // 32 bytes per row per instruction a staged copy would load, with no LDS
    // round trip
    auto wrow = [&](int n, int& mat) -> size_t {
        mat = (n >> 5) & 1;
        return (size_t)e * g.gu_rows + nblk * (WBN / 2) + 32 * (n >> 6) + (n & 31);
    };
    const u32x4* bpt[2];
#pragma unroll
    for (int nt = 0; nt < 2; nt++) {
        int mat;
        const size_t row = wrow(64 * wave + 32 * nt + l32, mat);
        bpt[nt] = (const u32x4*)(g.q[mat] + row * (D / 8)) + kq;
    }
    // ---- scales and biases of every group of LDS row n = tid, scaled by
    // the row's exponent; the gathered x rows' exponents
    {
        int mat;
        const size_t row = wrow(tid, mat);
        const uint16_t* sp = g.sc[mat] + row * C::NG;
        const uint16_t* bp = g.bi[mat] + row * C::NG;
        uint32_t sw[C::NG / 2], bw[C::NG / 2];
#pragma unroll
        for (int i = 0; i < C::NG / 8; i++) {
            const u32x4 sv = *(const u32x4*)(sp + 8 * i), bv = *(const u32x4*)(bp + 8 * i);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                sw[4 * i + j] = sv[j];
                bw[4 * i + j] = bv[j];
            }
        }
        uint32_t pr[C::NG];
        sm.ew[tid] = scale_row_params<C::NG>(sw, bw, pr);
        uint32_t* dst = &sm.sb[tid * SROW];
#pragma unroll
        for (int i = 0; i < C::NG / 4; i++) *(u32x4*)(dst + 4 * i) = u32x4{pr[4 * i], pr[4 * i + 1], pr[4 * i + 2], pr[4 * i + 3]};
    }
    if (tid < GEMM_BM) sm.ea[tid] = g.ex[g.perm[seg + m0 + min(tid, rows - 1)] / K];

    f32x16 acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < 2; nt++)
#pragma unroll
            for (int v = 0; v < 16; v++) acc[mt][nt][v] = 0.0f;

    auto mfma_step = [&](auto nmt_c, int abuf, const f16x8 (&bf)[2][4]) {
        constexpr int NMT = decltype(nmt_c)::value;
        const f16* ab = &sm.a[abuf][l32 * LDSB + 32 * kq];
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            f16x8 af[NMT];
#pragma unroll
            for (int mt = 0; mt < NMT; mt++) af[mt] = *(const f16x8*)(ab + mt * 32 * LDSB + 8 * kk);
#pragma unroll
            for (int mt = 0; mt < NMT; mt++)
#pragma unroll
                for (int nt = 0; nt < 2; nt++)
                    acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mt], bf[nt][kk], acc[mt][nt], 0, 0, 0);
        }
    };
    auto dequant = [&](int k, const u32x4 (&cb)[2], f16x8 (&bf)[2][4]) {
#pragma unroll
        for (int nt = 0; nt < 2; nt++) {
            const int n = 64 * wave + 32 * nt + l32;
            const u32x4 codes = cb[nt];
            f16x2 s2, b2;
            group_sb(sm.sb[n * SROW + k], s2, b2);
#pragma unroll
            for (int kk = 0; kk < 4; kk++) {
                const uint32_t cw = codes[kk];
                bf[nt][kk] = __builtin_bit_cast(f16x8, q4_word_to_f16x8(cw, s2, b2));
            }
        }
    };
    // ring stage j holds A(j) and the codes of step j; loads run three steps
    // ahead; A(j) sits in LDS buffer j % 2 during step j, the codes stay in
    // the ring
    constexpr int R = 4;
    static_assert(C::NK % R == 0, "K steps must be a multiple of the ring size");
    struct Stage { u32x4 a[2]; u32x4 b[2]; };
    auto load = [&](int k, Stage& st) {
#pragma unroll
        for (int i = 0; i < 2; i++) st.a[i] = *(const u32x4*)(apt[i] + k * BK);
#pragma unroll
        for (int i = 0; i < 2; i++) st.b[i] = bpt[i][2 * k];
    };
    auto store = [&](const Stage& st, int buf) {
#pragma unroll
        for (int i = 0; i < 2; i++) *(u32x4*)&sm.a[buf][(ar0 + 64 * i) * LDSB + 8 * ac] = st.a[i];
    };
    auto main_loop = [&](auto nmt_c) {
        Stage ring[R];
#pragma unroll
        for (int j = 0; j < R - 1; j++) load(j, ring[j]);
        store(ring[0], 0);
        __syncthreads();  // staged scales and biases; step 0's operands
#pragma unroll 1
        for (int k0 = 0; k0 < C::NK; k0 += R) {
#pragma unroll
            for (int j = 0; j < R; j++) {
                const int k = k0 + j;
                load(min(k + R - 1, C::NK - 1), ring[(j + R - 1) % R]);
                __builtin_amdgcn_sched_barrier(0);
                f16x8 bfr[2][4];
                dequant(k, ring[j].b, bfr);
                mfma_step(nmt_c, j & 1, bfr);
                store(ring[(j + 1) % R], (j + 1) & 1);
                __syncthreads();
            }
        }
    };
    const int nmt = (rows + 31) >> 5;
    if (nmt >= 4) main_loop(std::integral_constant<int, 4>{});
    else if (nmt == 3) main_loop(std::integral_constant<int, 3>{});
    else if (nmt == 2) main_loop(std::integral_constant<int, 2>{});
    else main_loop(std::integral_constant<int, 1>{});

    // ---- epilogue: h tile [128 rows][256 features] fp32 in LDS (a, pad,
    // sb): SwiGLU of the lane's gate and up values with their exponents
    // applied; then per row piece of 8 features: the row's largest |h| over
    // the block's 256 features (32 lanes), its exponent, fp16 in perm8
    // order, 16-byte stores
    constexpr int HS = WBN / 2 + 4;
    static_assert(GEMM_BM * HS * sizeof(float) <= offsetof(WideGuSmem, ea), "h tile must fit a, pad, sb");
    float* hb = (float*)&sm.a[0][0];
    auto acc_row = [&](int mt, int v) { return mt * 32 + 8 * (v >> 2) + 4 * kq + (v & 3); };
    const int f = 32 * wave + l32;  // feature inside the block
    const int eg = sm.ew[64 * wave + l32], eu = sm.ew[64 * wave + 32 + l32];
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int v = 0; v < 16; v++) {
            const int r = acc_row(mt, v);
            const float gv = __builtin_ldexpf(acc[mt][0][v], sm.ea[r] + eg);
            const float uv = __builtin_ldexpf(acc[mt][1][v], sm.ea[r] + eu);
            hb[r * HS + f] = silu_f32(gv) * uv;
        }
    // buffer stores (a flat store also counts as an LDS access, so the LDS
    // reads of the next rows would wait for it)
    const __amdgpu_buffer_rsrc_t rh_out = buffer_rsrc(g.h_out), reh = buffer_rsrc(g.eh);
    __syncthreads();
    // 128 rows x 32 pieces of 8 features: thread tid takes rows tid/32 + 16i,
    // piece tid%32 (a half-wave per row)
    const int c = tid & 31, rb = tid >> 5;
    const int fo = nblk * (WBN / 2) + 8 * c;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int r = rb + 16 * i;
        const f32x4 p0 = *(const f32x4*)&hb[r * HS + 8 * c], p1 = *(const f32x4*)&hb[r * HS + 8 * c + 4];
        const float v[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++) m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
        const int e = row_exp(half32_max(m));
        const u32x4 o = f32x8_to_f16x8_perm_scaled(v, e);
        if (r < rows) {
            // cache policy: see stream_nt (an immediate of the store, one per
            // branch; byte offsets stay below 2^31)
            const int off = (int)(((size_t)(seg + m0 + r) * F + fo) * sizeof(uint16_t));
            if (g.stream_nt) __builtin_amdgcn_raw_buffer_store_b128(o, rh_out, off, 0, 2);
            else __builtin_amdgcn_raw_buffer_store_b128(o, rh_out, off, 0, 0);
            if (c == 0) __builtin_amdgcn_raw_buffer_store_b32((uint32_t)e, reh, (uint32_t)((seg + m0 + r) * 2 + nblk) * 4, 0, 0);
        }
    }
}

__global__ void __launch_bounds__(512) k_gemm_gu_wide(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) WideGuSmem sm;
    gemm_block_gu_wide(g, sm, blockIdx.x);
}

template <int MODE>
__global__ void __launch_bounds__(GEMM_THREADS) k_gemm(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) GemmSmem<MODE> sm;
    gemm_block<MODE>(g, sm, blockIdx.x);
}

// The router logits and the shared expert's gate/up read only x, so they
// share one launch: blocks [0, n_router) compute logits, the rest the shared
// gate/up (either alone fills only part of the chip at a few thousand tokens).
constexpr size_t ROUTER_SGU_SMEM = sizeof(GemmSmem<MODE_ROUTER>) > sizeof(GemmSmem<MODE_SGU>)
                                       ? sizeof(GemmSmem<MODE_ROUTER>) : sizeof(GemmSmem<MODE_SGU>);
__global__ void __launch_bounds__(GEMM_THREADS) k_gemm_router_sgu(GemmArgs g, int n_router) {
    __shared__ __attribute__((aligned(16))) char sm[ROUTER_SGU_SMEM];
    if ((int)blockIdx.x < n_router)
        gemm_block<MODE_ROUTER>(g, *reinterpret_cast<GemmSmem<MODE_ROUTER>*>(sm), blockIdx.x);
    else
        gemm_block<MODE_SGU>(g, *reinterpret_cast<GemmSmem<MODE_SGU>*>(sm), blockIdx.x - n_router);
}

// y = sum_r partial_r * 2^ep_r (+ the residual), for layers without a
// shared expert.
__global__ void __launch_bounds__(256) k_combine_routed(const uint16_t* __restrict__ p, const int32_t* __restrict__ ep,
                                                        const int32_t* __restrict__ pos_of, const uint16_t* resid,
                                                        uint16_t* y, int T) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= T * D) return;
    const int t = i / D, o = i % D;
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < K; r++) {
        const int pos = pos_of[t * K + r];
        sum += __builtin_ldexpf((float)__builtin_bit_cast(f16, p[(size_t)pos * D + o]), ep[(size_t)pos * 4 + o / 512]);
    }
    if (resid) sum += bf16_to_f32(resid[i]);
    y[i] = f32_to_bf16_rne(sum);
}

int gemm_bm(int) { return GEMM_BM; }  // the routed tiles the sort builds

hipError_t launch_router_gemm(const uint16_t* xh, const int32_t* ex, const uint16_t* wr2, const int32_t* er,
                              const float* bias, float* logits, const uint16_t* shw, const int32_t* es, uint16_t* hs,
                              int32_t* ehs, int T, const Tracer& tr, hipStream_t s) {
    GemmArgs g = {};
    g.xh = xh; g.ex = ex; g.wr2 = wr2; g.er = er; g.rbias = bias; g.logits = logits; g.T = T;
    const int mt = (T + GEMM_BM - 1) / GEMM_BM;
    const int n_router = dense_grid<MODE_ROUTER>(mt);
    if (shw) {
        g.shw = shw; g.es = es; g.hs_out = hs; g.ehs = ehs;
        const int n_sgu = dense_grid<MODE_SGU>(mt);
        tr.launch(MOE_FFN_KERNEL_ROUTER, k_gemm_router_sgu, dim3(n_router + n_sgu), dim3(GEMM_THREADS), 0, s, g,
                  n_router);
    } else {
        tr.launch(MOE_FFN_KERNEL_ROUTER, k_gemm<MODE_ROUTER>, dim3(n_router), dim3(GEMM_THREADS), 0, s, g);
    }
    return hipGetLastError();
}

hipError_t launch_prefill_gemms(const PrefillGemmParams& p, const Tracer& tr, hipStream_t s) {
    GemmArgs g = {};
    g.xh = p.xh; g.ex = p.ex; g.h = p.h; g.eh = p.eh; g.hs = p.hs; g.ehs = p.ehs; g.ep = p.ep;
    g.shw = p.shw; g.es = p.es;
    g.perm = p.perm; g.pos_of = p.pos_of; g.offs = p.offs; g.tiles = p.tiles; g.tiles_e = p.tiles_e;
    g.tile_count = p.tile_count;
    g.wsort = p.wsort; g.sgate = p.sgate;
    g.gu_rows = p.gu_rows;
    g.T = p.T;
    const int bm = gemm_bm(p.T);
    const int max_tiles = (p.T * K + bm - 1) / bm + E;  // bound on the sort's tile count
    const int mt = (p.T + GEMM_BM - 1) / GEMM_BM;
    auto grid = [](int items) { return dim3(8 * ((items + 7) / 8)); };
    // routed gate/up: 256 features (512 gate + up rows) per block; down: 512 outputs
    g.q[0] = p.gate_q; g.sc[0] = p.gate_s; g.bi[0] = p.gate_b;
    g.q[1] = p.up_q; g.sc[1] = p.up_s; g.bi[1] = p.up_b;
    g.h_out = p.h;
    // h and the partials are written once and read once by the next launch:
    // while the partials fit the 256 MB memory-side cache the next launch
    // finds both there (4K tokens: 134 MB of partials; non-temporal stores
    // made that step 3 us slower); beyond it, stored non-temporal they stop
    // evicting the weights and x rows the GEMMs re-read (32K tokens: gate/up
    // 1077 -> 1062 us, down 865 -> 818 us, combine 365 -> 341 us)
    g.stream_nt = (size_t)p.T * K * D * sizeof(uint16_t) > ((size_t)256 << 20);
    tr.launch(MOE_FFN_KERNEL_EXPERT_GU, k_gemm_gu_wide, dim3(routed_grid<F / (WBN / 2)>(max_tiles)), dim3(512), 0, s,
              g);
    // (the shared gate/up ran with the router logits)
    // routed down
    g.q[0] = p.down_q; g.sc[0] = p.down_s; g.bi[0] = p.down_b;
    g.p_out = p.partial;
    tr.launch(MOE_FFN_KERNEL_EXPERT_DOWN, k_gemm_down_wide, grid(max_tiles * (D / WBN)), dim3(512), 0, s, g);
    // combine
    if (p.shw) {
        g.p_in = p.partial; g.y = p.y; g.resid = p.resid;
        tr.launch(MOE_FFN_KERNEL_COMBINE, k_gemm<MODE_SDOWN>, dim3(dense_grid<MODE_SDOWN>(mt)), dim3(GEMM_THREADS), 0,
                  s, g);
    } else {
        tr.launch(MOE_FFN_KERNEL_COMBINE, k_combine_routed, dim3((p.T * D + 255) / 256), dim3(256), 0, s,
                  (const uint16_t*)p.partial, (const int32_t*)p.ep, (const int32_t*)p.pos_of, p.resid, p.y, p.T);
    }
    return hipGetLastError();
}

}  // namespace moe
