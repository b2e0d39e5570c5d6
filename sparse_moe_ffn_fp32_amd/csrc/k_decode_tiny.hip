// Decode path for T <= 8 tokens: weight streaming on the vector ALUs.
//
// Lily engine page, "Dekodavimas: sumazinti perkeliamu baitu kieki vienam
// tokenui": batch-1 decode is a GEMV bound by the bytes moved per token, and
// a group of lanes cooperates on one output while reading different parts of
// its weight row.  With at most eight tokens a matrix-core tile would be
// half or more padding, so here every weight row is read by one wave: lane l takes
// the l-th 16-byte piece of the row (64 lanes = 1 KB, whole cache lines per
// load instruction), forms dot products with v_dot2 on pairs, and the wave
// sums the 64 partials in a fixed order (DPP and lane swaps).  Each launch is spread
// over at least 256 blocks and each wave issues all of its loads before it
// consumes any, so a launch costs one memory round trip.
//
// Weights stay exact: 4-bit codes become 128 + q (bf16) against bf16 x
// (gate/up) or against h held as two bf16 planes hi + lo (down: 16
// significant bits and the whole fp32 range, so a large h cannot overflow
// its storage), and each 32-element piece is finished in fp32 as
// s * dot(code, x) + (b - 128 s) * sum(x over the piece).  The piece sums of
// x come from the first launch, those of h from the down launch's own
// staging.
//
// Every kernel is compiled per token count (T = 1 .. 8), so that all loop
// bounds are constants: a load in a loop with a run-time trip count or under
// a run-time guard makes the compiler copy registers and wait for it at once.
//
// Every weight stream here is read once per call, in whole cache lines per
// load instruction, so the weight loads are non-temporal (evict first): they
// leave the cache to what is read again (x, h, the logits) and to the down
// rows launch C reads ahead for launch D (T=1 40-layer step 510 -> 488 us).
// Paths that read a line in two halves from two instructions keep normal
// loads (the first half's line could go before the second half is read).
//
// Launches:
//   A  router logits (fp32 weights, 4 experts per block, K halves over wave
//      pairs) and shared gate/up + SwiGLU (4 features per block, one row per
//      wave); one block copies x into the codes' K order, sums its pieces
//      and computes the shared-expert gate, from one round trip.
//      For the block entry point every block of A first RMS-normalises the
//      rows itself (no launch of its own), and the copy block also writes
//      the normalised rows out.
//   C  routed gate/up + SwiGLU: block = one (token, rank) pair x 8 features
//      (16 from three tokens on); each wave derives the pair's expert from
//      the token's logits (DPP top-8) so no routing launch is needed; up to
//      four tokens each block also pulls the down rows stage D will read
//      into cache; shared down (8 rows per block).
//   D  routed down: block = 8 output rows x every pair; h staged in LDS;
//      then the combine  y = sum_{r=0..7} w_r * down_r + sgate * shexp (+ the
//      residual of the block entry point)  in fixed order with one bf16
//      rounding.
#include "../../include/moe_ffn.h"
#include "decode_common.h"

namespace moe {

constexpr int TA_ROUTER_BLK = E / 4;  // 4 experts per block (8 waves)
constexpr int TA_SHARED_BLK = FS / 4; // 4 features (8 rows) per block
// Features per routed gate/up block: 8 up to two tokens, 16 from three (at
// three and four tokens the launch then keeps all of its blocks resident at
// once, and each token is ranked half as often); a block of chunk fc reads
// ahead the 4 * feat down rows 4 feat * fc .. of its expert.
__host__ __device__ constexpr int tc_feat(int nt) { return nt >= 3 ? 16 : 8; }
constexpr int TC_SDOWN_BLK = D / 8;   // shared-down blocks, 8 rows each
constexpr int TD_ROWS = 8;            // output rows per down block
constexpr int TD_THREADS = 512;       // threads per down block (8 waves)
constexpr int XPIECES = D / 32;       // 32-element pieces of an x row

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 16-bit pairs from a u32 passed by value.  (Bit-casting a vector-element
// expression directly is miscompiled by clang 22: it reads element 0.)
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }
__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Dot product of one u32 of eight 4-bit codes, as (magic + q) pairs in the
// perm8 order, with four 16-bit activation pairs (one u32x4, perm8).
__device__ __forceinline__ float dot_codes_bf16(uint32_t w, const u32x4& x, float acc) {
    const u32x4 c = nibble_codes(w, 0x43434343u);  // bf16 128 + q
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t cj = c[j], xj = x[j];
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(cj), as_bf16x2(xj), acc, false);
    }
    return acc;
}
// The same codes against an activation held as two bf16 planes (hi + lo).
__device__ __forceinline__ float dot_codes_bf16_2(uint32_t w, const u32x4& hh, const u32x4& hl, float acc) {
    const u32x4 c = nibble_codes(w, 0x43434343u);  // bf16 128 + q
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t cj = c[j], hj = hh[j], lj = hl[j];
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(cj), as_bf16x2(hj), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(cj), as_bf16x2(lj), acc, false);
    }
    return acc;
}

// bf16 scale or bias of quantisation group g from a row's [groups] array:
// one u32 load covers groups g & ~1 and g | 1.
__device__ __forceinline__ float group_param(uint32_t pairw, int g) {
    return (g & 1) ? hi_bf16(pairw) : lo_bf16(pairw);
}

// ------------------------------------------------------------------ A
// Block entry point: the RMS normalisation of the NT residual rows
// (qwen35moe Forward-Pass Design, "Block scaffold"; ds4.c study notes Part 3,
// section 3, trace 1: x / sqrt(mean(x^2) + eps) * weight, squares summed in
// double) runs inside every block of this launch instead of in a launch of
// its own.  Thread tid of the 512 holds elements 4 tid .. 4 tid + 3 of each
// row (hx, nw: loaded before the block's own weight loads); the sum of
// squares is reduced in one fixed order (lane order within a wave by a
// butterfly, then waves 0..7), so every block forms bit-identical normalised
// rows, each value rounded once from double to bf16.  They are left in LDS
// (xs, [NT][D/2] u32) for the block's dot products.
template <int NT>
__device__ __forceinline__ void norm_rows_to_lds(const u32x2 (&hx)[NT], const f32x4& nw, float eps,
                                                 double (*red)[NT], uint32_t* xs, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const double v0 = lo_bf16(hx[t][0]), v1 = hi_bf16(hx[t][0]), v2 = lo_bf16(hx[t][1]), v3 = hi_bf16(hx[t][1]);
        double ss = v0 * v0;
        ss += v1 * v1;
        ss += v2 * v2;
        ss += v3 * v3;
        ss = wave_sum_f64(ss);
        if (lane == 0) red[wave][t] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; t++) {
        double ss = red[0][t];
#pragma unroll
        for (int w = 1; w < 8; w++) ss += red[w][t];
        const double scale = 1.0 / __builtin_sqrt(ss / (double)D + (double)eps);
        const double v0 = lo_bf16(hx[t][0]), v1 = hi_bf16(hx[t][0]), v2 = lo_bf16(hx[t][1]), v3 = hi_bf16(hx[t][1]);
        u32x2 o;
        o[0] = (uint32_t)f64_to_bf16_rne(v0 * scale * (double)nw[0]) |
               ((uint32_t)f64_to_bf16_rne(v1 * scale * (double)nw[1]) << 16);
        o[1] = (uint32_t)f64_to_bf16_rne(v2 * scale * (double)nw[2]) |
               ((uint32_t)f64_to_bf16_rne(v3 * scale * (double)nw[3]) << 16);
        *(u32x2*)(xs + t * (D / 2) + 2 * tid) = o;
    }
    __syncthreads();
}

// The rows of x as they are, staged in LDS by the block (elements
// 4 tid .. 4 tid + 3 of every token per thread).
template <int NT>
__device__ __forceinline__ void copy_rows_to_lds(const u32x2 (&hx)[NT], uint32_t* xs, int tid) {
#pragma unroll
    for (int t = 0; t < NT; t++) *(u32x2*)(xs + t * (D / 2) + 2 * tid) = hx[t];
    __syncthreads();
}

// NT = T tokens (compiled per token count: every loop bound is a constant);
// NORM: x is the residual stream, normalised here first (a.nw, a.eps).
// From two tokens on (and always with NORM) the router and shared blocks
// read x from a copy in LDS: every wave needs all of x over its K range,
// and at four tokens the waves of one block had re-read 64-128 KB of x from
// the cache.
template <int NT, bool NORM>
__global__ void __launch_bounds__(512) k_tiny_a(DecodeArgs a) {
    constexpr bool XS = NORM || NT >= 2;  // x from LDS
    __shared__ float red[8][2 * NT];
    __shared__ double red64[8][NT];
    __shared__ uint32_t xs[XS ? NT * (D / 2) : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.x;
    u32x2 hx[NT];
    f32x4 nw;
    if (XS) {
#pragma unroll
        for (int t = 0; t < NT; t++) hx[t] = *(const u32x2*)(a.x + (size_t)t * D + 4 * tid);
    }
    if (NORM) nw = *(const f32x4*)(a.nw + 4 * tid);
    if (b == TA_ROUTER_BLK + TA_SHARED_BLK) {
        // x -> perm8 copy (pairs j, j+4 of every 8-block), its 32-element
        // piece sums and the shared-expert gate, from one round trip: thread
        // tid < 256 (waves 0-3) holds elements 8 tid .. 8 tid + 7 of every
        // token
        u32x4 gi = u32x4{0u, 0u, 0u, 0u};
        if (wave < 4 && a.sgi) gi = ((const u32x4*)a.sgi)[tid];
        if (NORM) norm_rows_to_lds<NT>(hx, nw, a.eps, red64, xs, tid);
        if (wave < 4) {  // every wave reaches the barrier below
            u32x4 d[NT];
#pragma unroll
            for (int t = 0; t < NT; t++) {
                if (NORM) {
                    d[t] = ((const u32x4*)(xs + t * (D / 2)))[tid];
                    ((u32x4*)(a.xn + (size_t)t * D))[tid] = d[t];
                } else {
                    d[t] = ((const u32x4*)(a.x + (size_t)t * D))[tid];
                }
            }
#pragma unroll
            for (int t = 0; t < NT; t++) {
                u32x4 o;
                o[0] = (d[t][0] & 0xffffu) | (d[t][2] << 16);
                o[1] = (d[t][0] >> 16) | (d[t][2] & 0xffff0000u);
                o[2] = (d[t][1] & 0xffffu) | (d[t][3] << 16);
                o[3] = (d[t][1] >> 16) | (d[t][3] & 0xffff0000u);
                ((u32x4*)(a.xp + (size_t)t * D))[tid] = o;
                float s = 0.0f, z = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t xj = d[t][j], gj = gi[j];
                    s += lo_bf16(xj) + hi_bf16(xj);
                    z += lo_bf16(xj) * lo_bf16(gj) + hi_bf16(xj) * hi_bf16(gj);
                }
                // one lane quad holds one 32-element piece
                s = quad_sum(s);
                if ((lane & 3) == 0) a.xsum[t * XPIECES + (tid >> 2)] = s;
                z = wave_sum(z);
                if (lane == 0) red[wave][t] = z;
            }
        }
        __syncthreads();
        if (tid < NT) {
            const float z = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
            a.sgate[tid] = a.sgi ? 1.0f / (1.0f + __expf(-z)) : 1.0f;
        }
        return;
    }
    if (b < TA_ROUTER_BLK) {
        // experts 4b + (wave >> 1); the wave pair splits the row's 512 pieces
        // of 4 fp32 weights (K = 4c) into alternating 64-piece runs
        const int e = 4 * b + (wave >> 1), kh = wave & 1;
        const float* wrow = a.wr + (size_t)e * D;
        f32x4 wv[4];
        u32x2 xv[NT][4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int c = lane + 64 * (2 * i + kh);
            wv[i] = __builtin_nontemporal_load((const f32x4*)(wrow + 4 * c));
            if (!XS)
#pragma unroll
                for (int t = 0; t < NT; t++) xv[t][i] = *(const u32x2*)(a.x + (size_t)t * D + 4 * c);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load above first: one round trip
        if (XS) {
            if (NORM) norm_rows_to_lds<NT>(hx, nw, a.eps, red64, xs, tid);
            else copy_rows_to_lds<NT>(hx, xs, tid);
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int t = 0; t < NT; t++) xv[t][i] = *(const u32x2*)(xs + t * (D / 2) + 2 * (lane + 64 * (2 * i + kh)));
        }
        float acc[NT];
#pragma unroll
        for (int t = 0; t < NT; t++) {
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                s += wv[i][0] * lo_bf16(xv[t][i][0]);
                s += wv[i][1] * hi_bf16(xv[t][i][0]);
                s += wv[i][2] * lo_bf16(xv[t][i][1]);
                s += wv[i][3] * hi_bf16(xv[t][i][1]);
            }
            acc[t] = wave_sum(s);
        }
        if (lane == 0)
#pragma unroll
            for (int t = 0; t < NT; t++) red[wave][t] = acc[t];
        __syncthreads();
        if (tid < 4 * NT) {
            const int r = tid / NT, t = tid % NT;
            const float s = red[2 * r][t] + red[2 * r + 1][t];
            a.logits[(size_t)t * E + 4 * b + r] = s + (a.rbias ? a.rbias[4 * b + r] : 0.0f);
        }
        return;
    }
    // shared gate/up: features f0 .. f0 + 3; wave w: gate row f0 + w (w < 4),
    // up row f0 + w - 4 (w >= 4); lane piece c = lane + 64 i holds 8 bf16 at
    // K = 8c
    if (!a.sg) return;
    const int f0 = 4 * (b - TA_ROUTER_BLK);
    const uint16_t* wrow = (wave < 4 ? a.sg : a.su) + (size_t)(f0 + (wave & 3)) * D;
    u32x4 wv[4], xv[NT][4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int c = lane + 64 * i;
        wv[i] = __builtin_nontemporal_load((const u32x4*)(wrow + 8 * c));
        if (!XS)
#pragma unroll
            for (int t = 0; t < NT; t++) xv[t][i] = *(const u32x4*)(a.x + (size_t)t * D + 8 * c);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above first: one round trip
    if (XS) {
        if (NORM) norm_rows_to_lds<NT>(hx, nw, a.eps, red64, xs, tid);
        else copy_rows_to_lds<NT>(hx, xs, tid);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int t = 0; t < NT; t++) xv[t][i] = *(const u32x4*)(xs + t * (D / 2) + 4 * (lane + 64 * i));
    }
#pragma unroll
    for (int t = 0; t < NT; t++) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++)
                {
                    const uint32_t wj = wv[i][j], xj = xv[t][i][j];
                    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wj), as_bf16x2(xj), s, false);
                }
        s = wave_sum(s);
        if (lane == 0) red[wave][t] = s;
    }
    __syncthreads();
    if (tid < 4 * NT) {
        const int i = tid / NT, t = tid % NT;
        a.hs[(size_t)t * FS + f0 + i] = silu_f32(red[i][t]) * red[4 + i][t];
    }
}

// ------------------------------------------------------------------ C
template <int NT, bool HASH>
__global__ void __launch_bounds__(256) k_tiny_c(DecodeArgs a, int n_gu_blocks) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if ((int)blockIdx.x >= n_gu_blocks) {
        // shared down: rows o0 + 2w, o0 + 2w + 1; lane piece = 8 bf16 at K = 8 lane
        if (!a.sd) return;
        const int o = TD_ROWS * (blockIdx.x - n_gu_blocks) + 2 * wave;
        u32x4 wv[2];
        f32x4 hv[NT][2];
#pragma unroll
        for (int r = 0; r < 2; r++) wv[r] = __builtin_nontemporal_load((const u32x4*)(a.sd + (size_t)(o + r) * FS + 8 * lane));
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const float* hrow = a.hs + (size_t)t * FS + 8 * lane;
            hv[t][0] = *(const f32x4*)hrow;
            hv[t][1] = *(const f32x4*)(hrow + 4);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load above first: one round trip
#pragma unroll
        for (int r = 0; r < 2; r++)
#pragma unroll
            for (int t = 0; t < NT; t++) {
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    s += lo_bf16(wv[r][j]) * hv[t][j >> 1][2 * (j & 1)];
                    s += hi_bf16(wv[r][j]) * hv[t][j >> 1][2 * (j & 1) + 1];
                }
                s = wave_sum(s);
                if (lane == 0) a.ys[(size_t)t * D + o + r] = s;
            }
        return;
    }
    // routed gate/up: pair p = (token t, rank r), features f0 .. f0 + FEAT - 1
    constexpr int FEAT = tc_feat(NT), FW = FEAT / 4, NR = 2 * FW;  // per wave: FW features, NR rows
    const int p = blockIdx.x / (F / FEAT), fc = blockIdx.x % (F / FEAT);
    const int t = p >> 3, r = p & 7;
    const int f0 = FEAT * fc;
    // x in the codes' K order and its piece sums do not depend on the routing
    u32x4 xv[4];
    const uint16_t* xrow = a.xp + (size_t)t * D + 32 * lane;
#pragma unroll
    for (int i = 0; i < 4; i++) xv[i] = *(const u32x4*)(xrow + 8 * i);
    const float xs = a.xsum[t * XPIECES + lane];
    // every wave ranks the token's experts itself (no LDS hand-off and no
    // barrier before the code loads), only as far as rank r (a rank-r block
    // is done after r + 1 rounds, so most blocks issue their code loads
    // earlier); the rank-7 blocks form all eight and one wave of one of them
    // writes the token's routing
    int e;
    {
        float sel_v[K];
        int sel_i[K];
#pragma unroll
        for (int k = 0; k < K; k++) sel_i[k] = 0;
        token_select<HASH>(a, t, lane, sel_v, sel_i, r + 1);
        if (wave == 0 && r == K - 1 && fc == 0) write_token_route<HASH>(a, t, lane, sel_v, sel_i, nullptr);  // sgate: stage A
        int er = sel_i[0];
#pragma unroll
        for (int k = 1; k < K; k++) er = (k == r) ? sel_i[k] : er;
        e = __builtin_amdgcn_readfirstlane(er) & (E - 1);
    }
    // wave w: features f0 + FW w .. f0 + FW w + FW - 1; rows q < FW: gate of
    // feature q, q >= FW: up of feature q - FW
    const size_t row0 = (size_t)e * a.gu_rows + f0 + FW * wave;
    // lane piece: 32 codes at K = 32 lane (4 u32), group lane / 2
    u32x4 cv[NR];
    uint32_t sv[NR], bv[NR];
#pragma unroll
    for (int q = 0; q < NR; q++) {
        const size_t row = row0 + (q % FW);
        const uint32_t* qp = q < FW ? a.gq : a.uq;
        const uint16_t* sp = q < FW ? a.gs : a.us;
        const uint16_t* bp = q < FW ? a.gb : a.ub;
        // read once: non-temporal, so they do not push the down rows read
        // ahead below (for stage D) out of the cache
        cv[q] = __builtin_nontemporal_load((const u32x4*)(qp + row * (D / 8) + 4 * lane));
        sv[q] = *(const uint32_t*)(sp + row * (D / G) + 2 * (lane >> 2));
        bv[q] = *(const uint32_t*)(bp + row * (D / G) + 2 * (lane >> 2));
    }
    // Down rows 4 FEAT fc .. 4 FEAT fc + 4 FEAT - 1 of this pair's expert,
    // which stage D reads next: one dword per 64 bytes (FEAT KB of codes,
    // FEAT / 16 KB each of scales and biases) pulls them into cache in this
    // same round trip.  Stage D's blocks take these rows on this block's XCD
    // (block id mod 8 = fc mod 8).  Up to four tokens only: from five on this
    // launch is bandwidth-bound and the read-ahead lengthens it by more than
    // it saves D (T=6 33.5 -> 33.0 us, T=8 41.6 -> 40.6 us without it; T=3
    // 22.1 -> 22.4 us without it).
    constexpr int PF_ROWS = 4 * FEAT, PF_CODES = PF_ROWS * (F / 2) / 64, PF_SB = PF_ROWS * (F / G) * 2 / 64;
    static_assert(PF_CODES <= 256 && 2 * PF_SB <= 256, "at most one code and one scale/bias dword per thread");
    uint32_t pf = 0, pf2 = 0;
    if constexpr (NT <= 4) {
        const size_t drow0 = (size_t)e * D + PF_ROWS * fc;
        if (tid < PF_CODES) pf = a.dq[drow0 * (F / 8) + 16 * tid];
        // the scale and bias dwords: threads from PF_CODES on, wrapping round
        const int j = (tid + 256 - PF_CODES) & 255;
        if (j < PF_SB) pf2 = *(const uint32_t*)(a.ds + drow0 * (F / G) + 32 * j);
        else if (j < 2 * PF_SB) pf2 = *(const uint32_t*)(a.db + drow0 * (F / G) + 32 * (j - PF_SB));
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above first: one round trip
    float out[NR];
    const int g = lane >> 1;
#pragma unroll
    for (int q = 0; q < NR; q++) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; i++) acc = dot_codes_bf16(cv[q][i], xv[i], acc);
        const float s = group_param(sv[q], g), bb = group_param(bv[q], g);
        out[q] = wave_sum(s * acc + (bb - 128.0f * s) * xs);
    }
    if (lane < FW) {
        float og = out[0], ou = out[FW];
#pragma unroll
        for (int i = 1; i < FW; i++)
            if (lane == i) {
                og = out[i];
                ou = out[FW + i];
            }
        const int f = f0 + FW * wave + lane;
        const float hv = silu_f32(og) * ou;
        const int pc = (f & ~7) | perm8_pos(f & 7);
        uint16_t hh, hlo;
        split_bf16(hv, hh, hlo);
        a.h[(size_t)p * F + pc] = hh;
        a.hl[(size_t)p * F + pc] = hlo;
    }
    asm volatile("" ::"v"(pf), "v"(pf2));  // the prefetch completes before the wave ends
}

// ------------------------------------------------------------------ D
// NT = T tokens (compiled per token count: every loop bound is a constant).
template <int NT>
__global__ void __launch_bounds__(TD_THREADS) k_tiny_d(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t hl[2][NT * K][F];  // h of every pair, bf16 hi, lo planes, perm8
    __shared__ float hsum[NT * K][F / 32];                               // piece sums of h
    __shared__ float dv[NT * K][TD_ROWS];                             // down outputs
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int T = NT, NP = T * K;
    // Row tile: block id b runs on XCD b % 8; stage C's block for feature
    // chunk fc (rows 4 FEAT fc .., row tiles TPC fc .. TPC fc + TPC - 1) ran
    // on XCD fc % 8, so b takes a row tile of a chunk with fc % 8 = b % 8.
    constexpr int TPC = tc_feat(NT) * 4 / TD_ROWS;  // row tiles per chunk
    const int xcd = blockIdx.x & 7, jb = blockIdx.x >> 3;
    const int o0 = TD_ROWS * (TPC * (8 * (jb / TPC) + xcd) + jb % TPC);
    // Every load of the block is issued before any is waited for, in the
    // order of use: the expert ids, h, the codes, the combine's operands.
    // Loads sit under no lane-dependent branch (the compiler would wait for
    // such a load at once) and no address waits on another load except the
    // codes' on the expert ids, which come from one load per lane shared
    // through lane shuffles (a load per unit would wait for each in turn).
    const int e_lane = a.idx[min(lane, NP - 1)] & (E - 1);  // lane l: expert of pair min(l, 8T - 1)
    // h of every pair: 8T rows x 64 pieces of 16 bytes, pieces tid + 512 i
    constexpr int NH = NP * (F / 8) / TD_THREADS;
    u32x4 hv[NH], hw[NH];
#pragma unroll
    for (int i = 0; i < NH; i++) {
        hv[i] = *(const u32x4*)(a.h + (size_t)(tid + TD_THREADS * i) * 8);
        hw[i] = *(const u32x4*)(a.hl + (size_t)(tid + TD_THREADS * i) * 8);
    }
    // units u = (pair u >> 3, row u & 7); lanes 16j .. 16j+15 share a unit,
    // lane piece c = lane & 15 holds 32 codes at K = 32c.  Wave w takes the
    // units 8T*w .. 8T*w + 8T - 1, four per load instruction (1 KB).
    const int c = lane & 15, sub = lane >> 4;
    constexpr int nj = 2 * T;
    u32x4 cv[nj];
    uint32_t sv[nj], bv[nj];
#pragma unroll
    for (int j = 0; j < nj; j++) {
        const int u = (wave * nj + j) * 4 + sub;
        const int pp = u >> 3, i = u & 7;
        const size_t row = (size_t)__shfl(e_lane, pp) * D + o0 + i;
        cv[j] = __builtin_nontemporal_load((const u32x4*)(a.dq + row * (F / 8) + 4 * c));
        sv[j] = *(const uint32_t*)(a.ds + row * (F / G) + 2 * (c >> 2));
        bv[j] = *(const uint32_t*)(a.db + row * (F / G) + 2 * (c >> 2));
    }
    // the combine's operands: thread tid < T * TD_ROWS takes (token tid / 8,
    // row tid % 8); the others load a clamped copy they never use
    const int ct = min(tid / TD_ROWS, T - 1), ci = tid % TD_ROWS;
    float wr[K];
#pragma unroll
    for (int r = 0; r < K; r++) wr[r] = a.w[ct * K + r];
    const float sgv = a.sg ? a.sgate[ct] : 0.0f;
    const float ysv = a.sg ? a.ys[(size_t)ct * D + o0 + ci] : 0.0f;
    const float rsv = a.resid ? bf16_to_f32(a.resid[(size_t)ct * D + o0 + ci]) : 0.0f;
    // stage h (8T rows x 1 KB) and its piece sums: thread takes 16-byte
    // pieces tid + 512 i (loaded above, before the codes: h is needed first)
#pragma unroll
    for (int i = 0; i < NH; i++) {
        const int q = tid + TD_THREADS * i;
        const int pp = q / (F / 8), k8 = q % (F / 8);
        const u32x4 v = hv[i], vl = hw[i];
        // piece 4c + w (lane c's w-th) at 4c + (w ^ (c >> 2)): the 16 lanes
        // reading one w then hit 16 distinct 16-byte bank slots
        const int ks = (k8 & ~3) | ((k8 & 3) ^ ((k8 >> 4) & 3));
        *(u32x4*)&hl[0][pp][8 * ks] = v;
        *(u32x4*)&hl[1][pp][8 * ks] = vl;
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t vj = v[j], lj = vl[j];
            s += (lo_bf16(vj) + lo_bf16(lj)) + (hi_bf16(vj) + hi_bf16(lj));
        }
        // four consecutive threads (one lane quad) hold one 32-element piece
        s = quad_sum(s);
        if ((k8 & 3) == 0) hsum[pp][k8 >> 2] = s;
    }
    __syncthreads();
    const int g = c >> 1;
    // two units at a time: units j0 and j0 + 1 (j0 even) are rows sub and
    // 4 + sub of one pair, so they share one read of its h piece (both
    // planes and the piece sum) from LDS
    static_assert(nj % 2 == 0, "unit pairs");
#pragma unroll
    for (int j0 = 0; j0 < nj; j0 += 2) {
        const int pp = ((wave * nj + j0) * 4 + sub) >> 3;
        u32x4 hh[4], hw[4];
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const int ws = w ^ ((c >> 2) & 3);
            hh[w] = *(const u32x4*)&hl[0][pp][32 * c + 8 * ws];
            hw[w] = *(const u32x4*)&hl[1][pp][32 * c + 8 * ws];
        }
        const float hs = hsum[pp][c];
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            const int j = j0 + jj;
            float acc = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; w++) acc = dot_codes_bf16_2(cv[j][w], hh[w], hw[w], acc);
            const float s = group_param(sv[j], g), bb = group_param(bv[j], g);
            const float v = row16_sum(s * acc + (bb - 128.0f * s) * hs);
            if (c == 0) dv[pp][4 * jj + sub] = v;
        }
    }
    __syncthreads();
    if (tid < T * TD_ROWS) {
        const int t = tid / TD_ROWS, i = tid % TD_ROWS;
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < K; r++) sum += wr[r] * dv[t * K + r][i];
        if (a.sg) sum += sgv * ysv;
        if (a.resid) sum += rsv;  // the residual, last before the one rounding
        a.y[(size_t)t * D + o0 + i] = f32_to_bf16_rne(sum);
    }
}

template <int NT>
hipError_t launch_tiny(const DecodeArgs& a, const Tracer& tr, hipStream_t s) {
    const int n_gu = NT * K * (F / tc_feat(NT));
    const dim3 ga(TA_ROUTER_BLK + TA_SHARED_BLK + 1);
    if (a.nw)
        tr.launch(MOE_FFN_KERNEL_ROUTER, k_tiny_a<NT, true>, ga, dim3(512), 0, s, a);
    else
        tr.launch(MOE_FFN_KERNEL_ROUTER, k_tiny_a<NT, false>, ga, dim3(512), 0, s, a);
    const dim3 gc(n_gu + (a.sd ? TC_SDOWN_BLK : 0));
    if (a.tid2eid)
        tr.launch(MOE_FFN_KERNEL_EXPERT_GU, k_tiny_c<NT, true>, gc, dim3(256), 0, s, a, n_gu);
    else
        tr.launch(MOE_FFN_KERNEL_EXPERT_GU, k_tiny_c<NT, false>, gc, dim3(256), 0, s, a, n_gu);
    tr.launch(MOE_FFN_KERNEL_EXPERT_DOWN, k_tiny_d<NT>, dim3(D / TD_ROWS), dim3(TD_THREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode_tiny(const DecodeArgs& a, const Tracer& tr, hipStream_t s) {
    static_assert(TINY_T == 8, "one case per token count");
    switch (a.T) {
        case 1: return launch_tiny<1>(a, tr, s);
        case 2: return launch_tiny<2>(a, tr, s);
        case 3: return launch_tiny<3>(a, tr, s);
        case 4: return launch_tiny<4>(a, tr, s);
        case 5: return launch_tiny<5>(a, tr, s);
        case 6: return launch_tiny<6>(a, tr, s);
        case 7: return launch_tiny<7>(a, tr, s);
        case 8: return launch_tiny<8>(a, tr, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
