// Decode path for 8 < T <= 64 tokens: bandwidth-bound expert GEMVs on skinny
// MFMA tiles (T <= 8 runs k_decode_tiny.hip).
//
// Lily engine page: batch-1 decode is a GEMV bound by the bytes moved per
// token ("Dekodavimas: sumazinti perkeliamu baitu kieki vienam tokenui"), and
// its single-row weight path has a group of lanes cooperate on outputs while
// reading different parts of the weight matrix.  Here a wave reads 16 weight
// rows at a time and multiplies them against up to 16 token columns with one
// v_mfma_f32_16x16x32 per 32 inputs: the matrix core does the dot products,
// so the vector ALUs only unpack nibbles and apply the per-group affine.
//
// Weights stay exact: the codes enter the MFMA as 128 + q (bf16, exact)
// against bf16 x (gate/up) or against h held as two bf16 planes hi + lo
// (down: 16 significant bits with the whole fp32 range, so a large h cannot
// overflow its storage), and every quantisation group's partial dot product
// is finished in fp32 as  s * acc + (b - 128 s) * sum(x over the group), where
// the group sums of the activations are formed once per token tile when it is
// staged in LDS.  "Rows on N": the 16 weight rows are the MFMA's N columns, so each
// lane holds one weight row and needs one scale and one bias per group.
//
// Every wave issues its global loads up front, in the order it consumes
// them, from addresses that are always valid (token slots past the end reuse
// slot 0's row and their results are dropped), so the loads overlap one
// another instead of waiting one by one.
//
// No block waits on another block inside a kernel: on gfx950 a device-scope
// release/acquire writes back and invalidates a whole XCD's L2 and costs as
// much as a kernel boundary, so the only global synchronisation is the
// stream order between launches.
//
// Launches (all on the caller's stream):
//   A      router logits (fp32 weights split exactly into three bf16 terms)
//          and the shared expert's gate/up rows against every token, K
//          split over blocks of (32 rows, 256 inputs), each block's four
//          64-input sub-slices summed in LDS in fixed order, the sums left
//          as slice partials; x copied into the K order of the codes, sgate.
//   top-k  the slice partials added in fixed order: per token the logits
//          (+ bias), top-8 and renormalised weights; the shared SwiGLU.
//   C      routed gate/up + SwiGLU: 256 persistent workgroups build the
//          distinct-expert and pair lists in LDS and stream their
//          (distinct expert, 128 features) items, each wave a full K sweep
//          of 16 gate and 16 up rows with a deep load ring; extra blocks:
//          the shared expert's down projection.
//   D      routed down, streamed the same way over (distinct expert, 128
//          output rows) items, fp32 partials per pair.
//   combine  y = sum_{r=0..7} w_r * partial_r + sgate * shexp  in fixed order
//          with one bf16 rounding (no float atomics).
//
// Indices read back from the workspace are clamped to their ranges before
// they address memory.
#include "../../include/moe_ffn.h"
#include "decode_common.h"

namespace moe {

constexpr int N_SDOWN_BLK = D / 16;

__device__ __forceinline__ f32x4 mfma16_bf16(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Wave-uniform read of memory that no kernel of the launch writes, through
// the constant address space so it becomes a scalar load.
__device__ __forceinline__ int ld_uniform(const int32_t* p, int i) {
    return ((const __attribute__((address_space(4))) int32_t*)p)[i];
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





// Sum of a u32x4 of eight bf16 (as fp32), then over the 8 consecutive lanes
// holding one 64-element quantisation group of a row (lane quads, then
// half-rows): every lane of the eight ends with the group's sum, in a fixed
// order.
__device__ __forceinline__ float group_sum8(const u32x4& v) {
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint32_t w = v[j];
        s += __uint_as_float(w << 16) + __uint_as_float(w & 0xffff0000u);
    }
    s = quad_sum(s);
    return s + dpp_mov<0x141>(s);  // row_half_mirror: the other quad of the eight
}

// ------------------------------------------------------------------ stage A
// The router rows (fp32) and the shared expert's gate and up rows (bf16)
// against every token, with K split over blocks: block = (group of 32 rows,
// K slice of 256); 8 router groups, 16 gate and 16 up groups, 8 slices each,
// 320 blocks of 512 threads (two fit a compute unit), each reading at most
// 32 KB of weights and T x 512 bytes of x, so the bytes and the router's
// plane splitting spread over the whole chip: blocks of (8 rows, 16 tokens)
// over the whole K read 64 KB of weights and 64 KB of x each, and at 8
// tokens only 98 of them existed, 32 of them holding all the router work
// (8.3 us for 6.3 MB).  Wave w takes the 16-row tile w & 1 and the K
// sub-slice w >> 1 (64 inputs) for every token tile; the four sub-slices
// are summed in LDS in order and the block's sums leave as partials
// pa[slice][t][row] (rows: 256 router, 512 gate, 512 up), which the routing
// launch adds in slice order.  The last ceil(T / 2) blocks copy x into the
// K order of the codes and form the shared-expert gate.
constexpr int SA_ROWS = 32;                  // rows per group
constexpr int SA_KS = 256;                   // K per slice
constexpr int SA_NS = D / SA_KS;             // slices
constexpr int SA_NROWS = E + 2 * FS;         // partial rows: router, gate, up
constexpr int SA_NGRP = SA_NROWS / SA_ROWS;  // 40 groups, the 8 router groups first
constexpr int SA_NGRP_R = E / SA_ROWS;
constexpr int SA_BLOCKS = SA_NGRP * SA_NS;
static_assert(E % SA_ROWS == 0 && FS % SA_ROWS == 0 && SA_KS == 4 * 64, "four 64-input sub-slices per slice");

template <int NMT>  // token tiles of 16
__global__ void __launch_bounds__(512) k_dec_stage_a(DecodeArgs a) {
    __shared__ float red[4][16 * NMT][SA_ROWS + 1];  // [K sub-slice][token][row]
    __shared__ float zs[8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int T = a.T;
    const int b = blockIdx.x;
    if (b >= SA_BLOCKS) {
        // x -> perm8 copy: 2 tokens (512 pieces of 16 bytes) per block, and
        // their shared-expert gate sgate = sigmoid(gate_inp . x) (1 without
        // a gate vector): thread tid holds piece tid % 256 of token tid / 256,
        // the token's four waves summed in wave order
        const int i = 512 * (b - SA_BLOCKS) + tid;
        const bool live = i < T * (D / 8);
        const u32x4 d = ((const u32x4*)a.x)[live ? i : 0];
        u32x4 g = u32x4{0u, 0u, 0u, 0u};
        if (a.sgi) g = ((const u32x4*)a.sgi)[tid & (D / 8 - 1)];
        if (live) {
            u32x4 o;
            o[0] = (d[0] & 0xffffu) | (d[2] << 16);
            o[1] = (d[0] >> 16) | (d[2] & 0xffff0000u);
            o[2] = (d[1] & 0xffffu) | (d[3] << 16);
            o[3] = (d[1] >> 16) | (d[3] & 0xffff0000u);
            ((u32x4*)a.xp)[i] = o;
        }
        float z = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t xj = d[j], gj = g[j];
            z += __uint_as_float(xj << 16) * __uint_as_float(gj << 16);
            z += __uint_as_float(xj & 0xffff0000u) * __uint_as_float(gj & 0xffff0000u);
        }
        z = wave_sum(z);
        if (lane == 0) zs[wave] = z;
        __syncthreads();
        const int t = 2 * (b - SA_BLOCKS) + tid;
        if (tid < 2 && t < T) {
            const float zt = ((zs[4 * tid] + zs[4 * tid + 1]) + zs[4 * tid + 2]) + zs[4 * tid + 3];
            a.sgate[t] = a.sgi ? 1.0f / (1.0f + __expf(-zt)) : 1.0f;
        }
        return;
    }
    const int grp = b % SA_NGRP, sl = b / SA_NGRP;
    const bool router = grp < SA_NGRP_R;
    if (!router && !a.sg) return;
    const int nt = wave & 1, ks = wave >> 1;
    const int k0 = SA_KS * sl + 64 * ks + 8 * kq;  // this lane's inputs: k0 .. k0 + 7 and k0 + 32 .. k0 + 39
    const int prow = SA_ROWS * grp + 16 * nt + n;  // B column n: this partial row
    // A rows: token 16 mt + n (slots past T read token 0's row; dropped)
    u32x4 xv[NMT][2];
#pragma unroll
    for (int mt = 0; mt < NMT; mt++) {
        const int t = 16 * mt + n;
        const uint16_t* xr = a.x + (size_t)(t < T ? t : 0) * D + k0;
        xv[mt][0] = *(const u32x4*)xr;
        xv[mt][1] = *(const u32x4*)(xr + 32);
    }
    f32x4 acc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; mt++) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (router) {
        const float* wrow = a.wr + (size_t)prow * D + k0;
        u32x4 wv[2][2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            wv[j][0] = *(const u32x4*)(wrow + 32 * j);
            wv[j][1] = *(const u32x4*)(wrow + 32 * j + 4);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep every load above: one round trip, not one per use
#pragma unroll
        for (int j = 0; j < 2; j++) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                v[q] = __uint_as_float(wv[j][0][q]);
                v[4 + q] = __uint_as_float(wv[j][1][q]);
            }
            u32x4 hi, mid, lo;
            split3(v, hi, mid, lo);
#pragma unroll
            for (int mt = 0; mt < NMT; mt++) {
                const bf16x8 av = as_bf16x8(xv[mt][j]);
                acc[mt] = mfma16_bf16(av, as_bf16x8(lo), acc[mt]);
                acc[mt] = mfma16_bf16(av, as_bf16x8(mid), acc[mt]);
                acc[mt] = mfma16_bf16(av, as_bf16x8(hi), acc[mt]);
            }
        }
    } else {
        const int r = prow - E;  // gate rows 0 .. FS - 1, then up rows
        const uint16_t* wrow = (r < FS ? a.sg + (size_t)r * D : a.su + (size_t)(r - FS) * D) + k0;
        u32x4 wv[2];
#pragma unroll
        for (int j = 0; j < 2; j++) wv[j] = *(const u32x4*)(wrow + 32 * j);
        __builtin_amdgcn_sched_barrier(0);  // keep every load above: one round trip, not one per use
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int mt = 0; mt < NMT; mt++) acc[mt] = mfma16_bf16(as_bf16x8(xv[mt][j]), as_bf16x8(wv[j]), acc[mt]);
    }
    // lane (n, kq) holds tokens 16 mt + 4 kq .. + 3 of column n; the four K
    // sub-slices summed in order, one partial per (token, row)
#pragma unroll
    for (int mt = 0; mt < NMT; mt++)
#pragma unroll
        for (int v = 0; v < 4; v++) red[ks][16 * mt + 4 * kq + v][16 * nt + n] = acc[mt][v];
    __syncthreads();
    float* const pa = a.pa + (size_t)sl * T * SA_NROWS + SA_ROWS * grp;
#pragma unroll
    for (int i = tid; i < 16 * NMT * SA_ROWS; i += 512) {
        const int t = i / SA_ROWS, c = i % SA_ROWS;
        const float v = ((red[0][t][c] + red[1][t][c]) + red[2][t][c]) + red[3][t][c];
        if (t < T) pa[(size_t)t * SA_NROWS + c] = v;
    }
}

// ------------------------------------------------------------------ routing
// One wave per token: DPP top-8 of the logits (or the hash table's column)
// and the renormalised weights.  Many small blocks, so the 8T arg-max rounds
// spread over the chip (one block for all tokens made the rounds compete
// for one compute unit's SIMDs: 11 us slower at 64 tokens).
// The stage-A partials are finished here: a token's logits are the slice
// partials added in slice order plus the router bias (in LDS, then the
// top-8), and the blocks after the routing ones form the shared SwiGLU
// hs = silu(gate) * up from the gate and up partials, four features per
// thread.
template <bool HASH>
__global__ void __launch_bounds__(256) k_dec_topk(DecodeArgs a) {
    __shared__ float lg[4][E];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T;
    const int nb = (T + 3) / 4;
    if ((int)blockIdx.x >= nb) {
        const int i = 256 * ((int)blockIdx.x - nb) + tid;
        const int t = i / (FS / 4), f = 4 * (i % (FS / 4));
        if (t >= T) return;
        const float* pg = a.pa + (size_t)t * SA_NROWS + E + f;
        f32x4 gp[SA_NS], up[SA_NS];
#pragma unroll
        for (int s = 0; s < SA_NS; s++) {
            gp[s] = *(const f32x4*)(pg + (size_t)s * T * SA_NROWS);
            up[s] = *(const f32x4*)(pg + (size_t)s * T * SA_NROWS + FS);
        }
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            float g = 0.0f, u = 0.0f;
#pragma unroll
            for (int s = 0; s < SA_NS; s++) {
                g += gp[s][j];
                u += up[s][j];
            }
            o[j] = silu_f32(g) * u;
        }
        *(f32x4*)(a.hs + (size_t)t * FS + f) = o;
        return;
    }
    const int t = 4 * blockIdx.x + wave;
    if (t >= T) return;
    float p[SA_NS][4], bias[4];
#pragma unroll
    for (int c = 0; c < 4; c++) {
        bias[c] = a.rbias ? a.rbias[lane + 64 * c] : 0.0f;
#pragma unroll
        for (int s = 0; s < SA_NS; s++) p[s][c] = a.pa[((size_t)s * T + t) * SA_NROWS + lane + 64 * c];
    }
#pragma unroll
    for (int c = 0; c < 4; c++) {
        float v = 0.0f;
#pragma unroll
        for (int s = 0; s < SA_NS; s++) v += p[s][c];
        lg[wave][lane + 64 * c] = v + bias[c];
    }
    float sel_v[K];
    int sel_i[K];
    select_experts<HASH>(lg[wave], a.tid2eid, a.n_vocab, HASH ? a.token_ids[t] : 0, lane, sel_v, sel_i);
    write_token_route<HASH>(a, t, lane, sel_v, sel_i, nullptr);
}

// The distinct experts in increasing id order, each with its (token, rank)
// pairs in token order, built in LDS by every workgroup of stages C and D
// from the T*8 expert ids (2 KB): cheaper than a launch of its own between
// top-k and stage C plus the dependent loads of its lists (expert count,
// then the lists, then the pairs).  An assignment's place among equal
// experts comes from ballots over the 8 bits of the expert id (within a
// wave) plus per-wave counts (across waves).
struct RouteSmem {
    int wcnt[8][E];     // per-wave counts of each expert, then per-wave offsets
    int start[E];       // first pair slot of each expert
    int uexp[E];        // distinct expert u: its id,
    int ucnt[E];        //   its pair count,
    int uoff[E];        //   its first pair slot
    int pairs[64 * K];  // pair ids (t*8 + r) grouped by expert, t ascending
    int wtot[8];
    int nu;             // distinct experts
};

// 512 threads, one assignment each (T*8 <= 512); every thread must call it.
__device__ void build_route(const DecodeArgs& a, RouteSmem& rs) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = a.T * K;
    const bool valid = tid < N;
    const int e = valid ? a.idx[tid] & (E - 1) : 0;
    for (int i = tid; i < 8 * E; i += 512) (&rs.wcnt[0][0])[i] = 0;
    __syncthreads();
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; bit++) {
        const uint64_t bb = __ballot((e >> bit) & 1);
        peers &= ((e >> bit) & 1) ? bb : ~bb;
    }
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & lt);
    if (valid && rank == 0) rs.wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    // experts tid < E (waves 0..3): per-wave counts -> per-wave offsets and
    // the total; one scan of (total << 16 | distinct) gives both prefixes
    int cnt = 0;
    if (tid < E) {
#pragma unroll
        for (int w = 0; w < 8; w++) {
            const int v = rs.wcnt[w][tid];
            rs.wcnt[w][tid] = cnt;
            cnt += v;
        }
    }
    int incl = wave_incl_scan((cnt << 16) | (cnt > 0));
    if (lane == 63) rs.wtot[wave] = incl;
    __syncthreads();
    if (tid < E) {
        for (int w = 0; w < wave; w++) incl += rs.wtot[w];
        const int first = (incl >> 16) - cnt;
        rs.start[tid] = first;
        if (cnt > 0) {
            const int u = (incl & 0xffff) - 1;
            rs.uexp[u] = tid;
            rs.ucnt[u] = cnt;
            rs.uoff[u] = first;
        }
        if (tid == E - 1) rs.nu = incl & 0xffff;
    }
    __syncthreads();
    if (valid) rs.pairs[rs.start[e] + rs.wcnt[wave][e] + rank] = tid;
    __syncthreads();
}

// The work units of items i0 .. i1 - 1 (at most 64; item = (distinct
// expert, chunk of `step` rows), the chunks of an expert consecutive), one
// per (item, token tile of up to 16), in order: expert, first row, tokens in
// the tile, tile parity, first pair slot.  The parity flips with every new
// token tile (consecutive items of one expert with one tile share it).  Wave
// 0 only, lane j for item i0 + j: first units and parities from one prefix
// sum of (tiles << 16 | flips) over the lanes.
__device__ void build_units(const RouteSmem& rs, int i0, int i1, int nch, int step, int T, int (*unit)[8],
                            int* n_units) {
    const int lane = threadIdx.x & 63;
    const int ni = i1 - i0;
    const bool live = lane < ni;
    const int it = i0 + min(lane, ni - 1);
    const int u = it / nch, chunk = it % nch;
    const int cnt = min(max(rs.ucnt[u], 1), T);
    const int ex = rs.uexp[u] & (E - 1);
    const int off = min(max(rs.uoff[u], 0), T * K - cnt);
    const int u_prev = __shfl_up(u, 1);
    const int first_flip = (lane > 0 && (u != u_prev || cnt > 16)) ? 1 : 0;
    const int tiles = live ? (cnt + 15) >> 4 : 0;
    const int flips = live ? first_flip + tiles - 1 : 0;  // parity flips at this item's units
    const int incl = wave_incl_scan((tiles << 16) | flips);
    const int u0 = (incl >> 16) - tiles, f0 = (incl & 0xffff) - flips;
    for (int m = 0; m < tiles; m++) {
        int* un = unit[u0 + m];
        un[0] = ex;
        un[1] = chunk * step;
        un[2] = min(16, cnt - 16 * m);
        un[3] = (f0 + first_flip + m) & 1;
        un[4] = off + 16 * m;
    }
    if (lane == 63) *n_units = incl >> 16;
}

// ------------------------------------------------------------------ stage C
// Routed gate/up, streamed.  The work units are (distinct expert, 128
// features, token tile of up to 16 tokens); GU_BLOCKS persistent workgroups
// (one per compute unit) each take a contiguous run of (expert, 128
// features) items, so consecutive units mostly share an expert and its
// token tile (at 64 tokens every workgroup takes the four items of one
// expert).  Wave w owns the gate and up rows of features 16w .. 16w + 15 of
// a unit over the whole K, one quantisation group (64 inputs) per step, so
// no partial sums cross waves.  The codes of the next GU_RING groups stay
// in flight across unit boundaries.  A unit's token tile sits in LDS; a new
// tile loads into registers during the last body of the unit before it and
// is stored between two barriers (one LDS buffer, so that a routed
// workgroup and a shared-down workgroup fit on one compute unit).
constexpr int GU_FEAT = 128;                 // features per item
constexpr int GU_NCH = F / GU_FEAT;          // items per expert
constexpr int GU_RING = 16;                  // groups of codes in flight per wave
constexpr int GU_BLOCKS = 256;               // persistent routed workgroups
constexpr int GU_ITEMS = E * GU_NCH / GU_BLOCKS;  // at most this many items each
constexpr int GU_UNITS = GU_ITEMS * 4;       // token tiles of 16: at most 64 tokens per expert
static_assert(GU_ITEMS <= 64, "one wave builds the unit table");
constexpr int XS_STRIDE = D + 8;             // bf16 per staged x row (16-byte pad)
struct GuSmem {
    uint16_t xs[16][XS_STRIDE];              // token tile of x (bf16, perm8 K order)
    float xsum[D / G][16];                   // its sums over each quantisation group
    int unit[GU_UNITS][8];                   // expert, first feature, tokens in the tile, tile parity, first pair
    int pairs[GU_UNITS][16];                 // pair ids of each unit's token slots
    int n_units;
};

__device__ __forceinline__ void gu_stream(const DecodeArgs& a, int bid, GuSmem& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int T = a.T;
    const int tk = T * K - 1;
    // the routing lists, in the token tile's space (not yet in use)
    static_assert(sizeof(RouteSmem) <= sizeof(sm.xs), "routing lists fit the token tile");
    RouteSmem& rs = *reinterpret_cast<RouteSmem*>(&sm.xs[0][0]);
    build_route(a, rs);
    const int nu = min(max(rs.nu, 0), min(T * K, E));
    const int n_items = nu * GU_NCH;
    const int q = (n_items + GU_BLOCKS - 1) / GU_BLOCKS;  // <= GU_ITEMS
    const int i0 = bid * q, i1 = min(i0 + q, n_items);
    if (i0 >= i1) return;
    constexpr int NGRP = D / G;  // 32
    static_assert(NGRP == 2 * GU_RING && GU_RING % 8 == 0, "two ring bodies per unit, whole scale vectors");

    // ---- unit table (at most 4 items x 4 tiles)
    if (wave == 0) build_units(rs, i0, i1, GU_NCH, GU_FEAT, T, sm.unit, &sm.n_units);
    __syncthreads();
    const int n_units = sm.n_units;
    if (tid < n_units * 16) {  // pair ids of every unit's token slots (slots >= tc repeat the last)
        const int k = tid >> 4, sl = tid & 15;
        sm.pairs[k][sl] = min(max(rs.pairs[sm.unit[k][4] + min(sl, sm.unit[k][2] - 1)], 0), tk);
    }
    __syncthreads();

    // x rows of a token tile: 16 rows x 256 pieces of 16 bytes; waves 4h ..
    // 4h+3 take rows h + 2i (wave-uniform), piece tid % 256.  Every row is
    // loaded and stored (rows >= tc repeat the last token; no lane reads
    // them): a load under a lane-dependent branch makes the compiler wait
    // for it at once.
    const int xc = tid & 255, xr0 = tid >> 8;
    auto load_x = [&](int k, u32x4 (&xv)[8]) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int pr = __builtin_amdgcn_readfirstlane(sm.pairs[k][xr0 + 2 * i]);
            xv[i] = *(const u32x4*)(a.xp + (size_t)(pr >> 3) * D + 8 * xc);
        }
    };
    auto store_x = [&](const u32x4 (&xv)[8]) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            *(u32x4*)&sm.xs[xr0 + 2 * i][8 * xc] = xv[i];
            const float gs = group_sum8(xv[i]);  // pieces 8g .. 8g + 7: one group
            if ((xc & 7) == 0) sm.xsum[xc >> 3][xr0 + 2 * i] = gs;
        }
    };
    // this lane's gate/up row in unit k (clamped to the last unit); gate and
    // up share one row layout, so one byte offset serves both code arrays
    auto row_of = [&](int k) {
        const int kk = min(k, n_units - 1);
        return (uint32_t)(__builtin_amdgcn_readfirstlane(sm.unit[kk][0]) * a.gu_rows + __builtin_amdgcn_readfirstlane(sm.unit[kk][1])) +
               (uint32_t)(16 * wave + n);
    };
    const __amdgpu_buffer_rsrc_t rgq = buffer_rsrc(a.gq), ruq = buffer_rsrc(a.uq);
    const __amdgpu_buffer_rsrc_t rgq0 = empty_rsrc(a.gq), ruq0 = empty_rsrc(a.uq);
    const int n_bodies = __builtin_amdgcn_readfirstlane(2 * n_units);
    // codes move as group pairs: lane (n, kq) loads words 4kq .. 4kq+3 of
    // the 16 words of pair p (groups 2p, 2p+1) of row n, so one instruction
    // reads 64 contiguous bytes of each of 16 rows (twice the run of one
    // group, which streams markedly faster)
    auto ld_codes = [&](__amdgpu_buffer_rsrc_t r, uint32_t row, int p) {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (row * (D / 8) + 4 * kq) * 4, 64 * p, 0));
    };
    // the four lanes of row n (kq = 0..3, one per 16-lane row) each load one
    // of the row's gate scales, gate biases, up scales, up biases (eight
    // groups per load) and swap them across lane rows when used
    const uint16_t* sarr = kq == 0 ? a.gs : kq == 1 ? a.gb : kq == 2 ? a.us : a.ub;
    auto ld_sc = [&](uint32_t row, int b) { return *(const u32x4*)(sarr + (size_t)row * (D / G) + 8 * b); };

    // ---- prologue: unit 0's scales and token tile, then the codes of its
    // first body (issued last, so that neither the tile store below nor the
    // first use of the scales in the loop waits for them)
    u32x4 sc0 = ld_sc(row_of(0), 0), sc1 = ld_sc(row_of(0), 1);
    u32x4 xv[8];
    load_x(0, xv);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NPAIR = GU_RING / 2;  // ring slots: group pairs
    u32x4 gw[NPAIR], uw[NPAIR];
    {
        const uint32_t r0 = row_of(0);
#pragma unroll
        for (int q = 0; q < NPAIR; q++) {
            gw[q] = ld_codes(rgq, r0, q);
            uw[q] = ld_codes(ruq, r0, q);
        }
    }
    store_x(xv);
    __syncthreads();

    f32x4 og = {0.f, 0.f, 0.f, 0.f}, ou = {0.f, 0.f, 0.f, 0.f};
    u32x4 xn[8];
    // bodies of GU_RING groups, two per unit: ring slot q holds pair q of the
    // body and is refilled with pair q of the next body (past the last body:
    // through an empty resource, so nothing is fetched); the scale vectors
    // of the next body load at its start
#pragma unroll 1
    for (int bb = 0; bb < n_bodies; bb++) {
        const int k = bb >> 1, half = bb & 1;
        const uint32_t rn = row_of((bb + 1) >> 1);
        const bool more = bb + 1 < n_bodies;  // wave-uniform
        const __amdgpu_buffer_rsrc_t rg = more ? rgq : rgq0, ru = more ? ruq : ruq0;
        const int ghn = GU_RING * ((bb + 1) & 1);  // first group of the next body
        const u32x4 scn0 = ld_sc(rn, ghn / 8), scn1 = ld_sc(rn, ghn / 8 + 1);
        const bool next_tile = half == 1 && k + 1 < n_units && sm.unit[k + 1][3] != sm.unit[k][3];
        if (next_tile) load_x(k + 1, xn);
        // A row: token slot n.  After the regrouping below, lane kq holds
        // words wq = 4(kq & 1) + 2(kq >> 1) and wq + 1 of each group, so its
        // x slice starts at K offset 8 wq.
        const uint16_t* xrow = &sm.xs[min(n, sm.unit[k][2] - 1)][32 * (kq & 1) + 16 * (kq >> 1)];
        uint32_t sgs = 0, sgb = 0, sus = 0, sub = 0;
        u32x4 bg[4], bu[4];
#pragma unroll
        for (int gi = 0; gi < GU_RING; gi++) {
            const int g = GU_RING * half + gi, q = gi >> 1;
            if ((gi & 1) == 0) {
                // regroup pair q so each MFMA sees a single group: swapping
                // words 0/2 and 1/3 between lanes kq and kq + 2 leaves lanes
                // kq = 0..3 holding words {0,4,2,6} (w0), {1,5,3,7} (w1) of
                // the first group and {8,12,10,14}, {9,13,11,15} of the second
                const auto g02 = __builtin_amdgcn_permlane32_swap(gw[q][0], gw[q][2], false, false);
                const auto g13 = __builtin_amdgcn_permlane32_swap(gw[q][1], gw[q][3], false, false);
                const auto u02 = __builtin_amdgcn_permlane32_swap(uw[q][0], uw[q][2], false, false);
                const auto u13 = __builtin_amdgcn_permlane32_swap(uw[q][1], uw[q][3], false, false);
                // expand the slot's codes first, then refill the slot: the
                // refill can take the slot's own registers, so the loop
                // back-edge needs no copies (a copy would wait for its load
                // and drain the ring)
                bg[0] = nibble_codes(g02[0], 0x43434343u); bg[1] = nibble_codes(g13[0], 0x43434343u);
                bg[2] = nibble_codes(g02[1], 0x43434343u); bg[3] = nibble_codes(g13[1], 0x43434343u);
                bu[0] = nibble_codes(u02[0], 0x43434343u); bu[1] = nibble_codes(u13[0], 0x43434343u);
                bu[2] = nibble_codes(u02[1], 0x43434343u); bu[3] = nibble_codes(u13[1], 0x43434343u);
                __builtin_amdgcn_sched_barrier(0);
                gw[q] = ld_codes(rg, rn, ghn / 2 + q);
                uw[q] = ld_codes(ru, rn, ghn / 2 + q);
            }
            const int h2 = 2 * (gi & 1);
            const bf16x8 a0 = as_bf16x8(*(const u32x4*)(xrow + 64 * g));
            const bf16x8 a1 = as_bf16x8(*(const u32x4*)(xrow + 64 * g + 8));
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 ag = mfma16_bf16(a0, as_bf16x8(bg[h2]), z);
            ag = mfma16_bf16(a1, as_bf16x8(bg[h2 + 1]), ag);
            f32x4 au = mfma16_bf16(a0, as_bf16x8(bu[h2]), z);
            au = mfma16_bf16(a1, as_bf16x8(bu[h2 + 1]), au);
            const f32x4 xsum = *(const f32x4*)&sm.xsum[g][4 * kq];  // token slots 4kq .. 4kq + 3
            const int gs8 = gi & 7;
            if ((gs8 & 1) == 0) {
                // dword gs8/2 of the four arrays: after the 16-lane swap p0
                // holds the even lane row's array (kq & ~1), p1 the odd one's;
                // the 32-lane swaps then give rows 0/1 and 2/3
                const uint32_t d = (gi < 8 ? sc0 : sc1)[gs8 >> 1];
                const auto p = __builtin_amdgcn_permlane16_swap(d, d, false, false);
                const auto q0 = __builtin_amdgcn_permlane32_swap((uint32_t)p[0], (uint32_t)p[0], false, false);
                const auto q1 = __builtin_amdgcn_permlane32_swap((uint32_t)p[1], (uint32_t)p[1], false, false);
                sgs = q0[0]; sus = q0[1]; sgb = q1[0]; sub = q1[1];
            }
            const bool hi = gs8 & 1;
            const float s_g = __uint_as_float(hi ? (sgs & 0xffff0000u) : (sgs << 16));
            const float s_u = __uint_as_float(hi ? (sus & 0xffff0000u) : (sus << 16));
            const float c_g = __uint_as_float(hi ? (sgb & 0xffff0000u) : (sgb << 16)) - 128.0f * s_g;
            const float c_u = __uint_as_float(hi ? (sub & 0xffff0000u) : (sub << 16)) - 128.0f * s_u;
#pragma unroll
            for (int v = 0; v < 4; v++) {
                og[v] = __builtin_fmaf(c_g, xsum[v], __builtin_fmaf(s_g, ag[v], og[v]));
                ou[v] = __builtin_fmaf(c_u, xsum[v], __builtin_fmaf(s_u, au[v], ou[v]));
            }
        }
        sc0 = scn0;
        sc1 = scn1;
        if (half == 1) {
            // ---- SwiGLU for token slots 4kq + v, feature f (perm8 position)
            const int tc = sm.unit[k][2];
            const int f = sm.unit[k][1] + 16 * wave + n;
            const int pc = (f & ~7) | perm8_pos(f & 7);
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int slot = 4 * kq + v;
                if (slot < tc) {
                    uint16_t hh, hlo;
                    split_bf16(silu_f32(og[v]) * ou[v], hh, hlo);
                    a.h[(size_t)sm.pairs[k][slot] * F + pc] = hh;
                    a.hl[(size_t)sm.pairs[k][slot] * F + pc] = hlo;
                }
            }
            og = f32x4{0.f, 0.f, 0.f, 0.f};
            ou = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // the tile is the only LDS the loop writes: the waves meet only where
        // it changes (every wave has left the old tile, then the new one is
        // stored and published); at 64 tokens a workgroup keeps one tile and
        // its waves never wait for each other
        if (next_tile) {
            __syncthreads();
            store_x(xn);
            __syncthreads();
        }
    }
}

// Blocks [0, GU_BLOCKS) are the routed workgroups, blocks from GU_BLOCKS on
// the shared expert's down projection.  A workgroup of this kernel takes a
// whole compute unit (its register count allows two waves per SIMD), so the
// routed workgroups come first: all of them start at once, and the shared
// blocks run on the compute units whose routed workgroup has no items (or
// finished).  The other order delayed about a hundred routed workgroups by
// a shared block's lifetime.
__global__ void __launch_bounds__(512) k_dec_stage_c(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[sizeof(GuSmem)];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int T = a.T;
    if ((int)blockIdx.x >= GU_BLOCKS) {
        // ---- shared expert down: ys[t, o0+n] = sum_j Wsd[o0+n, j] hs[t, j],
        // hs split into bf16 hi + lo; wave w takes K in [64w, 64w+64)
        if (!a.sg) return;
        float(*sred)[16][16] = (float(*)[16][16])smem;  // [8][16][16]
        const int o0 = 16 * ((int)blockIdx.x - GU_BLOCKS);
        const int k0 = 64 * wave + 8 * kq;
        const uint16_t* wrow = a.sd + (size_t)(o0 + n) * FS + k0;
        const u32x4 b0 = *(const u32x4*)(wrow), b1 = *(const u32x4*)(wrow + 32);
#pragma unroll 1
        for (int m = 0; m < (T + 15) / 16; m++) {
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
            if (m > 0) __syncthreads();
#pragma unroll
            for (int v = 0; v < 4; v++) sred[wave][4 * kq + v][n] = acc[v];
            __syncthreads();
            if (tid < 256) {
                const int tl = tid >> 4, c = tid & 15;
                const int t2 = 16 * m + tl;
                float s = 0.f;
#pragma unroll
                for (int w = 0; w < 8; w++) s += sred[w][tl][c];
                if (t2 < T) a.ys[(size_t)t2 * D + o0 + c] = s;
            }
        }
        return;
    }
    gu_stream(a, (int)blockIdx.x, *reinterpret_cast<GuSmem*>(smem));
}

// ------------------------------------------------------------------ stage D
// Routed down, streamed like stage C.  The work units are (distinct expert,
// 128 output rows, token tile of up to 16 tokens); DN_BLOCKS persistent
// workgroups each take a contiguous run of (expert, 128 rows) items, so
// consecutive units mostly share an expert and its token tile.  Wave w owns
// output rows 16w .. 16w + 15 of a unit over K = F (eight quantisation
// groups, moved as four group pairs like the gate/up codes); the codes of
// the next DN_RING groups (two units) stay in flight across unit
// boundaries, and the next unit's token tile loads while the current one
// computes.  Partials per (pair, output) in fp32.
constexpr int DN_ROWS = 128;                        // output rows per item
constexpr int DN_NCH = D / DN_ROWS;                 // items per expert
constexpr int DN_BLOCKS = 256;                      // persistent workgroups
constexpr int DN_ITEMS = E * DN_NCH / DN_BLOCKS;    // at most this many items each
constexpr int DN_UNITS = DN_ITEMS * 4;              // token tiles of 16: at most 64 tokens per expert
static_assert(DN_ITEMS <= 64, "one wave builds the unit table");
constexpr int DN_RING = 16;                         // groups of codes in flight per wave
constexpr int HS_STRIDE = F + 8;                    // fp16 per staged h row (16-byte pad)
struct DnSmem {
    uint16_t hs[2][2][16][HS_STRIDE];  // token tiles of h (bf16 hi, lo planes, perm8 order), two buffers
    float hsum[2][F / G][16];          // their sums over each quantisation group
    int unit[DN_UNITS][8];          // expert, first output row, tokens in the tile, h buffer, first pair
    int pairs[DN_UNITS][16];        // pair ids of each unit's token slots
    int n_units;
};

__global__ void __launch_bounds__(512) k_dec_stage_d(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) DnSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int T = a.T;
    const int tk = T * K - 1;
    // the routing lists, in the h tiles' space (not yet in use)
    static_assert(sizeof(RouteSmem) <= sizeof(sm.hs), "routing lists fit the h tiles");
    RouteSmem& rs = *reinterpret_cast<RouteSmem*>(&sm.hs[0][0][0][0]);
    build_route(a, rs);
    const int nu = min(max(rs.nu, 0), min(T * K, E));
    const int n_items = nu * DN_NCH;
    const int q = (n_items + DN_BLOCKS - 1) / DN_BLOCKS;  // <= DN_ITEMS
    const int i0 = blockIdx.x * q, i1 = min(i0 + q, n_items);
    if (i0 >= i1) return;

    // ---- unit table (at most 16 items x 4 tiles)
    if (wave == 0) build_units(rs, i0, i1, DN_NCH, DN_ROWS, T, sm.unit, &sm.n_units);
    __syncthreads();
    const int n_units = sm.n_units;
    // pair ids of every unit's token slots (slots >= tc repeat the last)
#pragma unroll
    for (int i = 0; i < DN_UNITS * 16 / 512; i++) {
        const int t = tid + 512 * i, k = t >> 4, sl = t & 15;
        if (k < n_units) sm.pairs[k][sl] = min(max(rs.pairs[sm.unit[k][4] + min(sl, sm.unit[k][2] - 1)], 0), tk);
    }
    __syncthreads();

    // h rows of a unit's token tile: 16 rows x 64 pieces of 16 bytes; thread
    // tid takes piece tid % 64 of rows tid / 64 + 8i.  Every row is loaded
    // and stored (slots >= tc repeat the last token; no lane reads them):
    // a load under a lane-dependent branch makes the compiler wait for it
    // at once.
    const int hc = tid & 63, hr0 = tid >> 6;
    auto load_h = [&](int k, u32x4 (&hv)[4]) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const size_t off = (size_t)sm.pairs[k][hr0 + 8 * i] * F + 8 * hc;
            hv[i] = *(const u32x4*)(a.h + off);
            hv[2 + i] = *(const u32x4*)(a.hl + off);
        }
    };
    auto store_h = [&](int k, const u32x4 (&hv)[4]) {
        const int buf = sm.unit[k][3];
#pragma unroll
        for (int i = 0; i < 2; i++) {
            *(u32x4*)&sm.hs[buf][0][hr0 + 8 * i][8 * hc] = hv[i];
            *(u32x4*)&sm.hs[buf][1][hr0 + 8 * i][8 * hc] = hv[2 + i];
            const float gs = group_sum8(hv[i]) + group_sum8(hv[2 + i]);  // hi + lo of one group
            if ((hc & 7) == 0) sm.hsum[buf][hc >> 3][hr0 + 8 * i] = gs;
        }
    };
    // code and scale offsets of this lane's output row in unit k
    const __amdgpu_buffer_rsrc_t rdq = buffer_rsrc(a.dq), rdq0 = empty_rsrc(a.dq);
    const int n_units_s = __builtin_amdgcn_readfirstlane(n_units);
    auto row_of = [&](int k) {
        const int kk = min(k, n_units - 1);
        return (uint32_t)(__builtin_amdgcn_readfirstlane(sm.unit[kk][0]) * D + __builtin_amdgcn_readfirstlane(sm.unit[kk][1])) +
               (uint32_t)(16 * wave + n);
    };
    // lane (n, kq) loads words 4kq .. 4kq+3 of group pair p of row n
    auto ld_codes = [&](__amdgpu_buffer_rsrc_t r, uint32_t row, int p) {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (row * (F / 8) + 4 * kq) * 4, 64 * p, 0));
    };
    auto ld_sc = [&](uint32_t row, u32x4& sv, u32x4& bv) {
        sv = *(const u32x4*)(a.ds + (size_t)row * (F / G));
        bv = *(const u32x4*)(a.db + (size_t)row * (F / G));
    };

    // ---- prologue: scales and token tile of unit 0, then the codes of
    // units 0 and 1 (issued last, so that neither the tile store below nor
    // the first use of the scales in the loop waits for them)
    u32x4 sv, bv;
    ld_sc(row_of(0), sv, bv);
    u32x4 hv0[4];
    load_h(0, hv0);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NPAIR = F / G / 2;  // group pairs per unit
    u32x4 ring[DN_RING / 2];
    {
        const uint32_t r0 = row_of(0), r1 = row_of(1);
#pragma unroll
        for (int q = 0; q < NPAIR; q++) ring[q] = ld_codes(rdq, r0, q);
        const __amdgpu_buffer_rsrc_t r = 1 < n_units_s ? rdq : rdq0;
#pragma unroll
        for (int q = 0; q < NPAIR; q++) ring[NPAIR + q] = ld_codes(r, r1, q);
    }
    store_h(0, hv0);
    __syncthreads();

    static_assert(DN_RING == 2 * (F / G), "the ring holds two units");
    // bodies of two units: ring slot 4(k % 2) + q holds pair q of unit k and
    // is refilled with pair q of unit k + 2 (past the last unit: nothing)
#pragma unroll 1
    for (int k0 = 0; k0 < n_units; k0 += 2) {
#pragma unroll
        for (int uu = 0; uu < 2; uu++) {
            const int k = k0 + uu;
            const bool active = k < n_units;
            const int kc = min(k, n_units - 1);
            const bool next_tile = k + 1 < n_units && sm.unit[k + 1][3] != sm.unit[kc][3];
            u32x4 hv[4];
            if (next_tile) load_h(k + 1, hv);
            u32x4 svn, bvn;
            ld_sc(row_of(k + 1), svn, bvn);
            const uint32_t rn = row_of(k + 2);
            // past the last unit the refills go through an empty resource
            const __amdgpu_buffer_rsrc_t rr = k + 2 < n_units_s ? rdq : rdq0;
            // A row: token slot n, at the K offset of the words this lane
            // holds after the regrouping (as in the gate/up stage)
            const int hb = sm.unit[kc][3], hslot = min(n, sm.unit[kc][2] - 1), hk = 32 * (kq & 1) + 16 * (kq >> 1);
            const uint16_t* hrow = &sm.hs[hb][0][hslot][hk];
            const uint16_t* lrow = &sm.hs[hb][1][hslot][hk];
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
            u32x4 b[4];
#pragma unroll
            for (int g = 0; g < 8; g++) {
                const int rs = NPAIR * uu + (g >> 1);
                if ((g & 1) == 0) {
                    // regroup the pair (one group per MFMA), expand the
                    // slot's codes, then refill the slot (no register copy
                    // across the loop back-edge)
                    const auto w02 = __builtin_amdgcn_permlane32_swap(ring[rs][0], ring[rs][2], false, false);
                    const auto w13 = __builtin_amdgcn_permlane32_swap(ring[rs][1], ring[rs][3], false, false);
                    b[0] = nibble_codes(w02[0], 0x43434343u); b[1] = nibble_codes(w13[0], 0x43434343u);
                    b[2] = nibble_codes(w02[1], 0x43434343u); b[3] = nibble_codes(w13[1], 0x43434343u);
                    __builtin_amdgcn_sched_barrier(0);
                    ring[rs] = ld_codes(rr, rn, g >> 1);
                }
                const int h2 = 2 * (g & 1);
                const bf16x8 a0 = as_bf16x8(*(const u32x4*)(hrow + 64 * g));
                const bf16x8 a1 = as_bf16x8(*(const u32x4*)(hrow + 64 * g + 8));
                const bf16x8 l0 = as_bf16x8(*(const u32x4*)(lrow + 64 * g));
                const bf16x8 l1 = as_bf16x8(*(const u32x4*)(lrow + 64 * g + 8));
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                f32x4 acc = mfma16_bf16(a0, as_bf16x8(b[h2]), z);
                acc = mfma16_bf16(a1, as_bf16x8(b[h2 + 1]), acc);
                acc = mfma16_bf16(l0, as_bf16x8(b[h2]), acc);
                acc = mfma16_bf16(l1, as_bf16x8(b[h2 + 1]), acc);
                const f32x4 hsum = *(const f32x4*)&sm.hsum[hb][g][4 * kq];  // token slots 4kq .. 4kq + 3
                const float sg = bf16_at(sv, g);
                const float cg = bf16_at(bv, g) - 128.0f * sg;
#pragma unroll
                for (int v = 0; v < 4; v++) o[v] = __builtin_fmaf(cg, hsum[v], __builtin_fmaf(sg, acc[v], o[v]));
            }
            if (active) {
                const int tc = sm.unit[k][2];
                const int orow = sm.unit[k][1] + 16 * wave + n;
#pragma unroll
                for (int v = 0; v < 4; v++) {
                    const int slot = 4 * kq + v;
                    if (slot < tc) a.part[(size_t)sm.pairs[k][slot] * D + orow] = o[v];
                }
            }
            sv = svn;
            bv = bvn;
            // the tile buffers are the only LDS the loop writes: the other
            // buffer's last reader finished before the barrier that published
            // the current tile, and the barrier below publishes the next one;
            // units that keep their tile need no barrier
            if (next_tile) {
                store_h(k + 1, hv);
                __syncthreads();
            }
        }
    }
}

// y = sum_{r=0..7} w_r * partial_r + sgate * shexp (+ the residual), fixed
// order, one bf16 rounding (T > 8).
__global__ void __launch_bounds__(256) k_dec_combine(DecodeArgs a) {
    // four consecutive outputs per thread (16-byte partial loads)
    const int i = 4 * (blockIdx.x * 256 + threadIdx.x);
    if (i >= a.T * D) return;
    const int t = i / D, o = i % D;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < K; r++) {
        const float w = a.w[t * K + r];
        const f32x4 p = *(const f32x4*)&a.part[(size_t)(t * K + r) * D + o];
#pragma unroll
        for (int j = 0; j < 4; j++) sum[j] += w * p[j];
    }
    if (a.sg) {
        const float g = a.sgate[t];
        const f32x4 ys = *(const f32x4*)&a.ys[i];
#pragma unroll
        for (int j = 0; j < 4; j++) sum[j] += g * ys[j];
    }
    if (a.resid) {
        const u32x2 rv = *(const u32x2*)&a.resid[i];
        sum[0] += bf16_to_f32(rv[0] & 0xffffu);
        sum[1] += bf16_to_f32(rv[0] >> 16);
        sum[2] += bf16_to_f32(rv[1] & 0xffffu);
        sum[3] += bf16_to_f32(rv[1] >> 16);
    }
    u32x2 out;
    out[0] = (uint32_t)f32_to_bf16_rne(sum[0]) | ((uint32_t)f32_to_bf16_rne(sum[1]) << 16);
    out[1] = (uint32_t)f32_to_bf16_rne(sum[2]) | ((uint32_t)f32_to_bf16_rne(sum[3]) << 16);
    *(u32x2*)&a.y[i] = out;
}

// ------------------------------------------------------------------ host
size_t decode_workspace_bytes(int T, DecodeLayout* L) {
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    DecodeLayout l{};
    size_t o = 0;
    l.logits = o; o += up((size_t)T * E * 4);
    l.xp = o;     o += up((size_t)T * D * 2);
    l.hs = o;     o += up((size_t)T * FS * 4);
    l.ys = o;     o += up((size_t)T * D * 4);
    l.h = o;      o += up((size_t)T * K * F * 2 * 2);  // hi and lo planes
    l.part = o;   o += up(T > TINY_T ? (size_t)T * K * D * 4 : 0);
    l.idx = o;    o += up((size_t)T * K * 4);
    l.w = o;      o += up((size_t)T * K * 4);
    l.sgate = o;  o += up((size_t)T * 4);
    l.xsum = o;   o += up(T <= TINY_T ? (size_t)T * (D / 32) * 4 : 0);
    l.total = o;
    if (L) *L = l;
    return o;
}

static void launch_decode_t(const DecodeArgs& a, const Tracer& tr, hipStream_t s) {
    const int nmt = (a.T + 15) / 16;  // token tiles of 16
    const int n_gu = GU_BLOCKS;
    const dim3 ga(SA_BLOCKS + (a.T + 1) / 2);
    switch (nmt) {
        case 1: tr.launch(MOE_FFN_KERNEL_ROUTER, k_dec_stage_a<1>, ga, dim3(512), 0, s, a); break;
        case 2: tr.launch(MOE_FFN_KERNEL_ROUTER, k_dec_stage_a<2>, ga, dim3(512), 0, s, a); break;
        case 3: tr.launch(MOE_FFN_KERNEL_ROUTER, k_dec_stage_a<3>, ga, dim3(512), 0, s, a); break;
        default: tr.launch(MOE_FFN_KERNEL_ROUTER, k_dec_stage_a<4>, ga, dim3(512), 0, s, a); break;
    }
    const dim3 gt((a.T + 3) / 4 + (a.sg ? (a.T * FS / 4 + 255) / 256 : 0));
    if (a.tid2eid)
        hipLaunchKernelGGL(k_dec_topk<true>, gt, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_dec_topk<false>, gt, dim3(256), 0, s, a);
    const int n_sd = a.sg ? N_SDOWN_BLK : 0;
    tr.launch(MOE_FFN_KERNEL_EXPERT_GU, k_dec_stage_c, dim3(n_gu + n_sd), dim3(512), 0, s, a);
    tr.launch(MOE_FFN_KERNEL_EXPERT_DOWN, k_dec_stage_d, dim3(DN_BLOCKS), dim3(512), 0, s, a);
    tr.launch(MOE_FFN_KERNEL_COMBINE, k_dec_combine, dim3((a.T * D / 4 + 255) / 256), dim3(256), 0, s, a);
}

hipError_t launch_decode(const DecodeParams& p, char* ws, const Tracer& tr, hipStream_t s) {
    DecodeLayout L;
    decode_workspace_bytes(p.T, &L);
    DecodeArgs a{};
    a.x = p.x; a.T = p.T;
    a.wr = p.router_w; a.rbias = p.router_b; a.wscale = p.wscale; a.gating = p.gating;
    a.tid2eid = p.tid2eid; a.token_ids = p.token_ids; a.n_vocab = p.n_vocab;
    a.sgi = p.sh_gate_inp; a.sg = p.sh_gate; a.su = p.sh_up; a.sd = p.sh_down;
    a.gq = p.gate_q; a.uq = p.up_q; a.dq = p.down_q;
    a.gs = p.gate_s; a.gb = p.gate_b; a.us = p.up_s; a.ub = p.up_b; a.ds = p.down_s; a.db = p.down_b;
    a.gu_rows = p.gu_rows;
    a.logits = (float*)(ws + L.logits);
    a.xp = (uint16_t*)(ws + L.xp);
    a.hs = (float*)(ws + L.hs);
    a.ys = (float*)(ws + L.ys);
    a.h = (uint16_t*)(ws + L.h);
    a.hl = a.h + (size_t)p.T * K * F;
    a.part = (float*)(ws + L.part);
    a.pa = a.part;  // stage A's partials: read by the routing launch before stage D writes part
    a.idx = p.idx ? p.idx : (int32_t*)(ws + L.idx);
    a.w = p.w ? p.w : (float*)(ws + L.w);
    a.sgate = (float*)(ws + L.sgate);
    a.xsum = (float*)(ws + L.xsum);
    a.y = p.y;
    a.resid = p.resid;
    if (p.T <= TINY_T) {
        // the normalisation runs inside the first launch
        a.nw = p.norm_w;
        a.eps = p.eps;
        a.xn = p.xn;
        return launch_decode_tiny(a, tr, s);
    }
    if (p.norm_w) {
        const hipError_t e = launch_rmsnorm(p.x, p.norm_w, p.eps, p.xn, p.T, s);
        if (e != hipSuccess) return e;
        a.x = p.xn;
    }
    launch_decode_t(a, tr, s);
    return hipGetLastError();
}

}  // namespace moe
