// Decode path (T <= 64): bandwidth-bound expert GEMVs on skinny MFMA tiles.
//
// Lily engine page: batch-1 decode is a GEMV bound by the bytes moved per
// token ("Dekodavimas: sumazinti perkeliamu baitu kieki vienam tokenui"), and
// its single-row weight path has a group of lanes cooperate on outputs while
// reading different parts of the weight matrix.  Here a wave reads 16 weight
// rows at a time and multiplies them against up to 16 token columns with one
// v_mfma_f32_16x16x32 per 32 inputs: the matrix core does the dot products,
// so the vector ALUs only unpack nibbles and apply the per-group affine.
//
// Weights stay exact: the codes enter the MFMA as 128 + q (bf16) or 1024 + q
// (fp16), both exact, and every quantisation group's partial dot product is
// finished in fp32 as  s * acc + (b - c*s) * sum(x over the group), where the
// group sum of the activations comes from one more MFMA against a ones
// operand.  "Rows on N": the 16 weight rows are the MFMA's N columns, so each
// lane holds one weight row and needs one scale and one bias per group.
//
// Every wave issues all of its global loads up front, in the order it
// consumes them, from addresses that are always valid (token slots past the
// end reuse slot 0's row and their results are dropped), so the loads overlap
// one another instead of waiting one by one.
//
// Launches (all on the caller's stream):
//   A  router logits (fp32 weights split exactly into three bf16 terms) and
//      the shared expert's gate/up + SwiGLU, K split over the 16 waves of a
//      block and reduced in LDS in fixed order; x in the K order of the codes.
//      The last router block to finish does the routing: softmax/top-8/
//      renormalise per token, sgate, and the distinct experts with their
//      (token, rank) pairs.
//   C  routed gate/up + SwiGLU per (distinct expert, 32 features), K split in
//      four; and the shared expert's down projection.
//   D  routed down projection per (16 output rows, 8 distinct experts); the
//      last block to finish a row tile does the combine
//      y = sum_{r=0..7} w_r * down_r + sgate * shexp  in fixed order with one
//      bf16 rounding (no float atomics).
// The arrival counters live in the zero-initialised head of the workspace;
// each is returned to zero by the block that sees the last arrival, so every
// call leaves them ready for the next.
//
// Indices read back from the workspace are clamped to their ranges before
// they address memory.
#include "../../include/moe_ffn.h"
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int N_ROUTER_BLK = E / 16;
constexpr int N_SGU_BLK = FS / 16;
constexpr int N_SDOWN_BLK = D / 16;
constexpr int N_ROW_TILES = D / 16;

__device__ __forceinline__ f32x4 mfma16_bf16(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_f16(const f16x8& a, const f16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// One u32 of eight nibbles -> eight codes c + q in perm8 order; `magic`
// holds the bit pattern of c in both 16-bit halves (0x4300 for bf16 128,
// 0x6400 for fp16 1024).
__device__ __forceinline__ u32x4 nibbles_to_codes(uint32_t w, uint32_t magic) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; j++) o[j] = ((w >> (4 * j)) & 0x000f000fu) | magic;
    return o;
}

// Group g's bf16 from a vector of eight packed bf16 (two per dword), as fp32.
__device__ __forceinline__ float bf16_at(const u32x4& v, int g) {
    const uint32_t d = v[g >> 1];
    return __uint_as_float((g & 1) ? (d & 0xffff0000u) : (d << 16));
}

// Eight fp32 -> three bf16x8 with v = hi + mid + lo exactly.
__device__ __forceinline__ void split3(const float* v, u32x4& hi, u32x4& mid, u32x4& lo) {
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t u = __float_as_uint(v[j]);
        h[j] = u & 0xffff0000u;
        const float r1 = v[j] - __uint_as_float(h[j]);
        m[j] = __float_as_uint(r1) & 0xffff0000u;
        l[j] = __float_as_uint(r1 - __uint_as_float(m[j]));
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
        hi[j] = (h[2 * j] >> 16) | h[2 * j + 1];
        mid[j] = (m[2 * j] >> 16) | m[2 * j + 1];
        lo[j] = (l[2 * j] >> 16) | (l[2 * j + 1] & 0xffff0000u);
    }
}

// Eight fp32 -> bf16x8 hi (truncated) + lo (rounded remainder): hi + lo
// carries 16 significant bits.
__device__ __forceinline__ void split2(const float* v, u32x4& hi, u32x4& lo) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        h[j] = __float_as_uint(v[j]) & 0xffff0000u;
        l[j] = f32_to_bf16_rne(v[j] - __uint_as_float(h[j]));
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
        hi[j] = (h[2 * j] >> 16) | h[2 * j + 1];
        lo[j] = l[2 * j] | (l[2 * j + 1] << 16);
    }
}

struct DecodeArgs {
    const uint16_t* x;
    int T;
    const float* wr;
    const float* rbias;
    const uint16_t *sgi, *sg, *su, *sd;  // shared expert (sg == nullptr: none)
    const uint32_t *gq, *uq, *dq;
    const uint16_t *gs, *gb, *us, *ub, *ds, *db;
    float* logits;   // [T, E]
    uint16_t* xp;    // bf16 [T, D], perm8
    float* hs;       // [T, FS] shared SwiGLU output
    float* ys;       // [T, D] shared down output
    uint16_t* h;     // fp16 [8T, F] (pair-major), perm8
    float* part;     // [8T, D] routed down outputs (when a row tile spans blocks)
    int32_t* arrive_a; // [1] arrival counter of the router blocks of stage A
    int32_t* arrive; // [N_ROW_TILES] arrival counters of stage D
    int32_t* idx;
    float* w;
    float* sgate;
    int32_t* nuniq;  // [1]
    int32_t* uexp;   // [E]
    int32_t* ucnt;   // [E]
    int32_t* uoff;   // [E]
    int32_t* pairs;  // [8T] (t*8 + r), grouped by distinct expert, t ascending
    uint16_t* y;
};

// ------------------------------------------------------------------ routing
// Run by the last router block of stage A (1024 threads) once every logit is
// in memory: softmax/top-8/renormalise and sgate per token (one wave per
// token), then the distinct experts in increasing id order, each with its
// (token, rank) pairs in token order.
__device__ void route_block(const DecodeArgs& a, int* sidx, int* scan_a, int* scan_b) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T;
    for (int t = wave; t < T; t += 16) {
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; c++) v[c] = a.logits[(size_t)t * E + lane + 64 * c];
        float sel_v[K];
        int sel_i[K];
        wave_top8(v, lane, sel_v, sel_i);
        // norm_topk_prob: the softmax normaliser cancels, so the weights are
        // the softmax of the eight selected logits
        float p[K], s = 0.0f;
#pragma unroll
        for (int r = 0; r < K; r++) {
            p[r] = __expf(sel_v[r] - sel_v[0]);
            s += p[r];
        }
        const float inv = 1.0f / s;
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
            sidx[t * K + lane] = iv;
        }
        float z = 0.0f;
        if (a.sgi) {
            const u32x4* xp = (const u32x4*)(a.x + (size_t)t * D + 32 * lane);
            const u32x4* gp = (const u32x4*)(a.sgi + 32 * lane);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const u32x4 xv = xp[q], gv = gp[q];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    z += __uint_as_float(xv[j] << 16) * __uint_as_float(gv[j] << 16);
                    z += __uint_as_float(xv[j] & 0xffff0000u) * __uint_as_float(gv[j] & 0xffff0000u);
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
        }
        if (lane == 0) a.sgate[t] = a.sgi ? 1.0f / (1.0f + __expf(-z)) : 1.0f;
    }
    __syncthreads();
    int cnt = 0;
    const int e = tid;
    if (e < E)
        for (int i = 0; i < T * K; i++) cnt += sidx[i] == e;
    if (e < E) {
        scan_a[e] = cnt > 0;
        scan_b[e] = cnt;
    }
    __syncthreads();
    for (int off = 1; off < E; off <<= 1) {  // inclusive scans
        int va = 0, vb = 0;
        if (e < E && e >= off) {
            va = scan_a[e - off];
            vb = scan_b[e - off];
        }
        __syncthreads();
        if (e < E) {
            scan_a[e] += va;
            scan_b[e] += vb;
        }
        __syncthreads();
    }
    if (e < E && cnt > 0) {
        const int u = scan_a[e] - 1;
        int j = scan_b[e] - cnt;
        a.uexp[u] = e;
        a.ucnt[u] = cnt;
        a.uoff[u] = j;
        for (int i = 0; i < T * K; i++)
            if (sidx[i] == e) a.pairs[j++] = i;
    }
    if (tid == 0) a.nuniq[0] = scan_a[E - 1];
}

// ------------------------------------------------------------------ stage A
// Router blocks: 16 experts; shared blocks: 16 gate + 16 up rows.  Wave w
// takes K in [128w, 128w + 128).
template <int NMT>
__global__ void __launch_bounds__(1024) k_dec_stage_a(DecodeArgs a) {
    __shared__ float red[16][NMT * 16][17];
    __shared__ int sidx[64 * K], scan_a[E], scan_b[E];
    __shared__ int last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int T = a.T;
    const int b = blockIdx.x;
    if (b == N_ROUTER_BLK + N_SGU_BLK) {  // x -> perm8 copy
        for (int i = tid; i < T * (D / 8); i += 1024) {
            const u32x4 d = ((const u32x4*)a.x)[i];
            u32x4 o;
            o[0] = (d[0] & 0xffffu) | (d[2] << 16);
            o[1] = (d[0] >> 16) | (d[2] & 0xffff0000u);
            o[2] = (d[1] & 0xffffu) | (d[3] << 16);
            o[3] = (d[1] >> 16) | (d[3] & 0xffff0000u);
            ((u32x4*)a.xp)[i] = o;
        }
        return;
    }
    const bool router = b < N_ROUTER_BLK;
    if (!router && !a.sg) return;
    const int row0 = router ? 16 * b : 16 * (b - N_ROUTER_BLK);
    const int kb = 128 * wave + 8 * kq;

    // activation row of this lane's A operand (row = lane % 16); token slots
    // past T read token 0's row and are dropped
    const uint16_t* xrow[NMT];
#pragma unroll
    for (int m = 0; m < NMT; m++) {
        const int t = 16 * m + n;
        xrow[m] = a.x + (size_t)(t < T ? t : 0) * D + kb;
    }
    f32x4 acc0[NMT], acc1[NMT];
#pragma unroll
    for (int m = 0; m < NMT; m++) acc0[m] = acc1[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (router) {
        const float* wrow = a.wr + (size_t)(row0 + n) * D + kb;
        u32x4 wv[4][2], xv[4][NMT];
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            wv[ks][0] = *(const u32x4*)(wrow + 32 * ks);
            wv[ks][1] = *(const u32x4*)(wrow + 32 * ks + 4);
#pragma unroll
            for (int m = 0; m < NMT; m++) xv[ks][m] = *(const u32x4*)(xrow[m] + 32 * ks);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                v[j] = __uint_as_float(wv[ks][0][j]);
                v[4 + j] = __uint_as_float(wv[ks][1][j]);
            }
            u32x4 hi, mid, lo;
            split3(v, hi, mid, lo);
#pragma unroll
            for (int m = 0; m < NMT; m++) {
                const bf16x8 av = as_bf16x8(xv[ks][m]);
                acc0[m] = mfma16_bf16(av, as_bf16x8(lo), acc0[m]);
                acc0[m] = mfma16_bf16(av, as_bf16x8(mid), acc0[m]);
                acc0[m] = mfma16_bf16(av, as_bf16x8(hi), acc0[m]);
            }
        }
    } else {
        const uint16_t* grow = a.sg + (size_t)(row0 + n) * D + kb;
        const uint16_t* urow = a.su + (size_t)(row0 + n) * D + kb;
        u32x4 gv[4], uv[4], xv[4][NMT];
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            gv[ks] = *(const u32x4*)(grow + 32 * ks);
            uv[ks] = *(const u32x4*)(urow + 32 * ks);
#pragma unroll
            for (int m = 0; m < NMT; m++) xv[ks][m] = *(const u32x4*)(xrow[m] + 32 * ks);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
#pragma unroll
            for (int m = 0; m < NMT; m++) {
                const bf16x8 av = as_bf16x8(xv[ks][m]);
                acc0[m] = mfma16_bf16(av, as_bf16x8(gv[ks]), acc0[m]);
                acc1[m] = mfma16_bf16(av, as_bf16x8(uv[ks]), acc1[m]);
            }
    }
    // sum the 16 K-slices in LDS in wave order: first acc0, then acc1
    float s0[2] = {0.f, 0.f};
    for (int pass = 0; pass < (router ? 1 : 2); pass++) {
#pragma unroll
        for (int m = 0; m < NMT; m++)
#pragma unroll
            for (int v = 0; v < 4; v++) red[wave][16 * m + 4 * kq + v][n] = pass ? acc1[m][v] : acc0[m][v];
        __syncthreads();
        if (tid < T * 16) {
            const int t = tid >> 4, c = tid & 15;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < 16; w++) s += red[w][t][c];
            s0[pass] = s;
        }
        __syncthreads();
    }
    if (tid < T * 16) {
        const int t = tid >> 4, c = tid & 15;
        if (router) a.logits[(size_t)t * E + row0 + c] = s0[0] + (a.rbias ? a.rbias[row0 + c] : 0.0f);
        else a.hs[(size_t)t * FS + row0 + c] = silu_f32(s0[0]) * s0[1];
    }
    if (!router) return;
    // the last router block to finish routes every token
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const int prev = __hip_atomic_fetch_add(a.arrive_a, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        last = prev == N_ROUTER_BLK - 1;
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    if (tid == 0) *a.arrive_a = 0;  // every router block has arrived: ready for the next call
    route_block(a, sidx, scan_a, scan_b);
}

// ------------------------------------------------------------------ stage C
// One wave: 16 features of one distinct expert, gate and up, 8 quantisation
// groups (512 inputs), for the token tiles of the expert one at a time.  The
// partial sums of token slot 16m + 4kq + v and feature n go to red_g/red_u.
__device__ __forceinline__ void gu_wave(const DecodeArgs& a, size_t row, int gq8, int cnt, int off, int lane,
                                        float (*red_g)[16], float (*red_u)[16]) {
    const int n = lane & 15, kq = lane >> 4;
    const size_t sbase = row * (D / G) + gq8;
    const u32x4 gsv = *(const u32x4*)(a.gs + sbase), gbv = *(const u32x4*)(a.gb + sbase);
    const u32x4 usv = *(const u32x4*)(a.us + sbase), ubv = *(const u32x4*)(a.ub + sbase);
    const uint32_t* gw_p = a.gq + row * (D / 8) + 8 * gq8 + 2 * kq;
    const uint32_t* uw_p = a.uq + row * (D / 8) + 8 * gq8 + 2 * kq;
    u32x2 gw[8], uw[8];
    u32x4 xa[8][2];
    const int tk = a.T * K - 1;
    const uint16_t* xrow = a.xp + (size_t)(min(max(a.pairs[off + (n < cnt ? n : 0)], 0), tk) >> 3) * D;
#pragma unroll
    for (int g = 0; g < 8; g++) {  // loads in the order they are consumed
        gw[g] = *(const u32x2*)(gw_p + 8 * g);
        uw[g] = *(const u32x2*)(uw_p + 8 * g);
        const int wd = 8 * (gq8 + g) + 2 * kq;
        xa[g][0] = *(const u32x4*)(xrow + 8 * wd);
        xa[g][1] = *(const u32x4*)(xrow + 8 * wd + 8);
    }
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};  // bf16 1.0
    const int nm = (cnt + 15) >> 4;
#pragma unroll 1
    for (int m = 0; m < nm; m++) {
        if (m > 0) {  // later token tiles (more than 16 tokens on this expert)
            const int slot = 16 * m + n;
            xrow = a.xp + (size_t)(min(max(a.pairs[off + (slot < cnt ? slot : 0)], 0), tk) >> 3) * D;
#pragma unroll
            for (int g = 0; g < 8; g++) {
                const int wd = 8 * (gq8 + g) + 2 * kq;
                xa[g][0] = *(const u32x4*)(xrow + 8 * wd);
                xa[g][1] = *(const u32x4*)(xrow + 8 * wd + 8);
            }
        }
        f32x4 og = {0.f, 0.f, 0.f, 0.f}, ou = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < 8; g++) {
            const float s_g = bf16_at(gsv, g), s_u = bf16_at(usv, g);
            const float c_g = bf16_at(gbv, g) - 128.0f * s_g, c_u = bf16_at(ubv, g) - 128.0f * s_u;
            const bf16x8 a0 = as_bf16x8(xa[g][0]), a1 = as_bf16x8(xa[g][1]);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 ag = mfma16_bf16(a0, as_bf16x8(nibbles_to_codes(gw[g][0], 0x43004300u)), z);
            ag = mfma16_bf16(a1, as_bf16x8(nibbles_to_codes(gw[g][1], 0x43004300u)), ag);
            f32x4 au = mfma16_bf16(a0, as_bf16x8(nibbles_to_codes(uw[g][0], 0x43004300u)), z);
            au = mfma16_bf16(a1, as_bf16x8(nibbles_to_codes(uw[g][1], 0x43004300u)), au);
            f32x4 xs = mfma16_bf16(a0, as_bf16x8(ones), z);
            xs = mfma16_bf16(a1, as_bf16x8(ones), xs);
#pragma unroll
            for (int v = 0; v < 4; v++) {
                og[v] += s_g * ag[v] + c_g * xs[v];
                ou[v] += s_u * au[v] + c_u * xs[v];
            }
        }
#pragma unroll
        for (int v = 0; v < 4; v++) {
            red_g[16 * m + 4 * kq + v][n] = og[v];
            red_u[16 * m + 4 * kq + v][n] = ou[v];
        }
    }
}

__global__ void __launch_bounds__(512) k_dec_stage_c(DecodeArgs a, int max_u) {
    __shared__ float red[2][4][2][64][16];  // [gate/up][K quarter][feature group][token slot][feature]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int T = a.T;
    if ((int)blockIdx.x >= max_u * (F / 32)) {
        // ---- shared expert down: ys[t, o0+n] = sum_j Wsd[o0+n, j] hs[t, j],
        // hs split into bf16 hi + lo; wave w takes K in [64w, 64w+64)
        if (!a.sg) return;
        const int o0 = 16 * (blockIdx.x - max_u * (F / 32));
        const int k0 = 64 * wave + 8 * kq;
        const uint16_t* wrow = a.sd + (size_t)(o0 + n) * FS + k0;
        const u32x4 b0 = *(const u32x4*)(wrow), b1 = *(const u32x4*)(wrow + 32);
        const int nm = (T + 15) / 16;
        float(*sred)[64][16] = (float(*)[64][16])red;  // [8][64][16]
#pragma unroll 1
        for (int m = 0; m < nm; m++) {
            const int t = 16 * m + n;
            const float* hrow = a.hs + (size_t)(t < T ? t : 0) * FS + k0;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const f32x4 p0 = *(const f32x4*)(hrow + 32 * ks), p1 = *(const f32x4*)(hrow + 32 * ks + 4);
                float v[8];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    v[j] = p0[j];
                    v[4 + j] = p1[j];
                }
                u32x4 hi, lo;
                split2(v, hi, lo);
                const bf16x8 bv = as_bf16x8(ks ? b1 : b0);
                acc = mfma16_bf16(as_bf16x8(lo), bv, acc);
                acc = mfma16_bf16(as_bf16x8(hi), bv, acc);
            }
#pragma unroll
            for (int v = 0; v < 4; v++) sred[wave][16 * m + 4 * kq + v][n] = acc[v];
        }
        __syncthreads();
        for (int i = tid; i < T * 16; i += 512) {
            const int t = i >> 4, c = i & 15;
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < 8; w++) s += sred[w][t][c];
            a.ys[(size_t)t * D + o0 + c] = s;
        }
        return;
    }
    // ---- routed gate/up: 32 features (2 groups of 16) x 4 K quarters
    const int u = blockIdx.x / (F / 32), chunk = blockIdx.x % (F / 32);
    if (u >= min(a.nuniq[0], max_u)) return;
    const int e = a.uexp[u] & (E - 1), cnt = min(max(a.ucnt[u], 1), T);
    const int off = min(max(a.uoff[u], 0), T * K - cnt);
    const int fg = wave & 1, kq4 = wave >> 1;
    gu_wave(a, (size_t)e * F + 32 * chunk + 16 * fg + n, 8 * kq4, cnt, off, lane, red[0][kq4][fg], red[1][kq4][fg]);
    __syncthreads();
    // quarters summed in order 0..3, then SwiGLU; h stored in perm8 order
    for (int i = tid; i < cnt * 32; i += 512) {
        const int slot = i >> 5, fl = i & 31;
        const int g2 = fl >> 4, c = fl & 15;
        float gg = 0.f, uu = 0.f;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            gg += red[0][q][g2][slot][c];
            uu += red[1][q][g2][slot][c];
        }
        const int f = 32 * chunk + fl;
        const int pc = (f & ~7) | perm8_pos(f & 7);
        const f16 hv = (f16)(silu_f32(gg) * uu);
        a.h[(size_t)min(max(a.pairs[off + slot], 0), T * K - 1) * F + pc] = __builtin_bit_cast(uint16_t, hv);
    }
}

// ------------------------------------------------------------------ stage D
// One wave: the routed down projection of 16 output rows for one distinct
// expert, its token tiles one at a time; results land in P[pair][row] (LDS)
// or in the global partials.
__device__ __forceinline__ void down_wave(const DecodeArgs& a, int e, int cnt, int off, int o0, int lane,
                                          float (*P)[17], bool to_lds) {
    const int n = lane & 15, kq = lane >> 4;
    const size_t row = (size_t)e * D + o0 + n;
    const u32x4 sv = *(const u32x4*)(a.ds + row * (F / G));
    const u32x4 bv = *(const u32x4*)(a.db + row * (F / G));
    u32x2 wv[8];
    u32x4 ha[8][2];
    const int tk = a.T * K - 1;
    const uint16_t* hrow = a.h + (size_t)min(max(a.pairs[off + (n < cnt ? n : 0)], 0), tk) * F;
#pragma unroll
    for (int g = 0; g < 8; g++) {  // loads in the order they are consumed
        wv[g] = *(const u32x2*)(a.dq + row * (F / 8) + 8 * g + 2 * kq);
        const int wd = 8 * g + 2 * kq;
        ha[g][0] = *(const u32x4*)(hrow + 8 * wd);
        ha[g][1] = *(const u32x4*)(hrow + 8 * wd + 8);
    }
    const u32x4 ones = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};  // fp16 1.0
    const int nm = (cnt + 15) >> 4;
#pragma unroll 1
    for (int m = 0; m < nm; m++) {
        if (m > 0) {
            const int slot = 16 * m + n;
            hrow = a.h + (size_t)min(max(a.pairs[off + (slot < cnt ? slot : 0)], 0), tk) * F;
#pragma unroll
            for (int g = 0; g < 8; g++) {
                const int wd = 8 * g + 2 * kq;
                ha[g][0] = *(const u32x4*)(hrow + 8 * wd);
                ha[g][1] = *(const u32x4*)(hrow + 8 * wd + 8);
            }
        }
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < 8; g++) {
            const float s = bf16_at(sv, g);
            const float c = bf16_at(bv, g) - 1024.0f * s;
            const f16x8 a0 = as_f16x8(ha[g][0]), a1 = as_f16x8(ha[g][1]);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 acc = mfma16_f16(a0, as_f16x8(nibbles_to_codes(wv[g][0], 0x64006400u)), z);
            acc = mfma16_f16(a1, as_f16x8(nibbles_to_codes(wv[g][1], 0x64006400u)), acc);
            f32x4 hsum = mfma16_f16(a0, as_f16x8(ones), z);
            hsum = mfma16_f16(a1, as_f16x8(ones), hsum);
#pragma unroll
            for (int v = 0; v < 4; v++) o[v] += s * acc[v] + c * hsum[v];
        }
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int slot = 16 * m + 4 * kq + v;
            if (slot < cnt) {
                const int p = min(max(a.pairs[off + slot], 0), tk);
                if (to_lds) P[p][n] = o[v];
                else a.part[(size_t)p * D + o0 + n] = o[v];
            }
        }
    }
}

__global__ void __launch_bounds__(512) k_dec_stage_d(DecodeArgs a) {
    __shared__ float P[64 * K][17];
    __shared__ int last;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T;
    const int rt = blockIdx.x % N_ROW_TILES, ch = blockIdx.x / N_ROW_TILES;
    const int o0 = 16 * rt;
    const int nu = min(max(a.nuniq[0], 0), min(T * K, E));
    const int nch = (nu + 7) >> 3;
    if (ch >= nch) return;
    const bool single = nch == 1;  // the whole row tile in this block: keep partials in LDS
    const int u = 8 * ch + wave;
    if (u < nu) {
        const int cnt = min(max(a.ucnt[u], 1), T);
        down_wave(a, a.uexp[u] & (E - 1), cnt, min(max(a.uoff[u], 0), T * K - cnt), o0, lane, P, single);
    }
    if (!single) {
        // publish this block's partials; the last block of the row tile combines
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const int prev = __hip_atomic_fetch_add(&a.arrive[rt], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            last = prev == nch - 1;
        }
        __syncthreads();
        if (!last) return;
        __threadfence();
        if (tid == 0) a.arrive[rt] = 0;  // all blocks of this row tile have arrived
    } else {
        __syncthreads();
    }
    for (int i = tid; i < T * 16; i += 512) {
        const int t = i >> 4, c = i & 15;
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < K; r++) {
            const float pv = single ? P[t * K + r][c] : a.part[(size_t)(t * K + r) * D + o0 + c];
            sum += a.w[t * K + r] * pv;
        }
        if (a.sg) sum += a.sgate[t] * a.ys[(size_t)t * D + o0 + c];
        a.y[(size_t)t * D + o0 + c] = f32_to_bf16_rne(sum);
    }
}

// ------------------------------------------------------------------ host
size_t decode_workspace_bytes(int T, DecodeLayout* L) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    DecodeLayout l{};
    size_t o = WS_COUNTER_BYTES;
    l.logits = o; o += up((size_t)T * E * 4);
    l.xp = o;     o += up((size_t)T * D * 2);
    l.hs = o;     o += up((size_t)T * FS * 4);
    l.ys = o;     o += up((size_t)T * D * 4);
    l.h = o;      o += up((size_t)T * K * F * 2);
    l.part = o;   o += up((size_t)T * K * D * 4);
    l.idx = o;    o += up((size_t)T * K * 4);
    l.w = o;      o += up((size_t)T * K * 4);
    l.sgate = o;  o += up((size_t)T * 4);
    l.nuniq = o;  o += up(4);
    l.uexp = o;   o += up(E * 4);
    l.ucnt = o;   o += up(E * 4);
    l.uoff = o;   o += up(E * 4);
    l.pairs = o;  o += up((size_t)T * K * 4);
    l.total = o;
    if (L) *L = l;
    return o;
}

template <int NMT>
static void launch_decode_t(const DecodeArgs& a, const Tracer& tr, hipStream_t s) {
    const int max_u = a.T * K < E ? a.T * K : E;
    tr.before(MOE_FFN_KERNEL_ROUTER, s);
    hipLaunchKernelGGL(k_dec_stage_a<NMT>, dim3(N_ROUTER_BLK + N_SGU_BLK + 1), dim3(1024), 0, s, a);
    tr.after(MOE_FFN_KERNEL_ROUTER, s);
    tr.before(MOE_FFN_KERNEL_EXPERT_GU, s);
    hipLaunchKernelGGL(k_dec_stage_c, dim3(max_u * (F / 32) + (a.sg ? N_SDOWN_BLK : 0)), dim3(512), 0, s, a, max_u);
    tr.after(MOE_FFN_KERNEL_EXPERT_GU, s);
    tr.before(MOE_FFN_KERNEL_EXPERT_DOWN, s);
    tr.before(MOE_FFN_KERNEL_COMBINE, s);
    hipLaunchKernelGGL(k_dec_stage_d, dim3(N_ROW_TILES * ((max_u + 7) / 8)), dim3(512), 0, s, a);
    tr.after(MOE_FFN_KERNEL_EXPERT_DOWN, s);
    tr.after(MOE_FFN_KERNEL_COMBINE, s);
}

hipError_t launch_decode(const DecodeParams& p, char* ws, const Tracer& tr, hipStream_t s) {
    DecodeLayout L;
    decode_workspace_bytes(p.T, &L);
    DecodeArgs a{};
    a.x = p.x; a.T = p.T;
    a.wr = p.router_w; a.rbias = p.router_b;
    a.sgi = p.sh_gate_inp; a.sg = p.sh_gate; a.su = p.sh_up; a.sd = p.sh_down;
    a.gq = p.gate_q; a.uq = p.up_q; a.dq = p.down_q;
    a.gs = p.gate_s; a.gb = p.gate_b; a.us = p.up_s; a.ub = p.up_b; a.ds = p.down_s; a.db = p.down_b;
    a.logits = (float*)(ws + L.logits);
    a.xp = (uint16_t*)(ws + L.xp);
    a.hs = (float*)(ws + L.hs);
    a.ys = (float*)(ws + L.ys);
    a.h = (uint16_t*)(ws + L.h);
    a.part = (float*)(ws + L.part);
    a.arrive_a = (int32_t*)(ws + WS_ARRIVE_A);
    a.arrive = (int32_t*)(ws + WS_ARRIVE_D);
    a.idx = p.idx ? p.idx : (int32_t*)(ws + L.idx);
    a.w = p.w ? p.w : (float*)(ws + L.w);
    a.sgate = (float*)(ws + L.sgate);
    a.nuniq = (int32_t*)(ws + L.nuniq);
    a.uexp = (int32_t*)(ws + L.uexp);
    a.ucnt = (int32_t*)(ws + L.ucnt);
    a.uoff = (int32_t*)(ws + L.uoff);
    a.pairs = (int32_t*)(ws + L.pairs);
    a.y = p.y;
    const int nmt = (p.T + 15) / 16;
    switch (nmt) {
        case 1: launch_decode_t<1>(a, tr, s); break;
        case 2: launch_decode_t<2>(a, tr, s); break;
        case 3: launch_decode_t<3>(a, tr, s); break;
        default: launch_decode_t<4>(a, tr, s); break;
    }
    return hipGetLastError();
}

}  // namespace moe
