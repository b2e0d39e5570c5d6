// Token->expert histogram, prefix scan and stable counting sort (subsystem 2).
//
// The grouped expert GEMMs need each expert's routed rows stored together.
// As on the Lily engine page ("Palikti ekspertu marsrutizavima GPU" -- keep
// expert routing on the GPU), a histogram counts the assignments per expert,
// a prefix scan turns counts into start offsets, a scatter writes every
// assignment into its expert's segment, and a tile map lists the fixed-size
// row tiles the GEMMs process.  Nothing returns to the host.  The histogram
// of every SORT_CH-assignment chunk is counted by the top-k launch as it
// selects (k_router.hip); this file holds the rest in one launch.
//
// Assignment a = t*8 + r is token t's r-th selected expert.  The scatter is
// stable: inside an expert's segment assignments keep increasing a (i.e.
// token) order, so the permutation is a pure function of the routing.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int SORT_CH = 2048;  // assignments per histogram/scatter block

// One launch after the histograms (a one-block scan launch between them
// and the scatter had cost 11 us at 4K tokens, all latency):
//
// Blocks 0 .. nblk-1 place the assignments of histogram block b: each forms
// its own bases, base[e] = offs[e] + sum over blocks b' < b of cnt[b'][e],
// with offs the exclusive scan of the expert totals, then walks its chunk in
// assignment order (stable), 1024 at a time: perm[pos] = a, pos_of[a] = pos,
// and the routing weight in sorted order, wsort[pos] = w[a].
// Ranks among equal experts inside a wave come from ballots on the 8 bits of
// the expert id, across waves from per-wave counts.
//
// Block nblk writes offs[0..E] and the tile map: record i is tiles[4i ..
// 4i+3] = {expert, first row of the tile within the expert's segment,
// segment start, rows in the tile (1..bm)}; tile_count[0] = number of tiles.
// The records are listed longest first: tiles with four live 32-row groups
// (every full tile, and partial tiles of more than 96 rows), then three,
// two, one; inside a class in expert order.  The grouped GEMMs take work
// items in this order, and blocks are started in id order as compute units
// free up, so the longest items start first and the short ones fill the
// tail (list scheduling, longest first).  tiles_e holds the same records in
// expert order.
constexpr int PLACE_THREADS = 1024;  // four threads per expert for the count passes
constexpr int PLACE_WAVES = PLACE_THREADS / 64;

// Exclusive scans of NS sets of 256 values, value e of set j held by thread
// e < 256 (waves 0..3; every thread calls it, the others pass 0 and get 0):
// one DPP scan per wave and set, then the wave totals through LDS, with one
// barrier for all the sets.  tot[j] = set j's total, in every thread.
// wtot: LDS of 4 * NS ints, not used by the caller until its next barrier.
template <int NS>
__device__ __forceinline__ void scan_256(const int (&v)[NS], int (&excl)[NS], int (&tot)[NS], int* wtot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int incl[NS];
#pragma unroll
    for (int j = 0; j < NS; j++) {
        incl[j] = wave_incl_scan(tid < 256 ? v[j] : 0);
        if (wave < 4 && lane == 63) wtot[4 * j + wave] = incl[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NS; j++) {
        int before = 0, all = 0;
#pragma unroll
        for (int w = 0; w < 4; w++) {
            const int t = wtot[4 * j + w];
            before += w < wave ? t : 0;
            all += t;
        }
        tot[j] = all;
        excl[j] = tid < 256 ? before + incl[j] - v[j] : 0;
    }
}

// Quarter qt of the histogram rows (thread tid = 256 qt + e): expert e's
// count over all rows (into part_t[qt][e]) and over the rows before `upto`
// (into part_p[qt][e]), sixteen independent loads at a time.
__device__ __forceinline__ void count_quarter(const int32_t* __restrict__ cnt, int nblk, int upto, int (*part_t)[E],
                                              int (*part_p)[E]) {
    const int tid = threadIdx.x, e = tid & (E - 1), qt = tid >> 8;
    const int nq = (nblk + 3) / 4, b_lo = qt * nq, b_hi = min(nblk, b_lo + nq);
    int t = 0, p = 0;
    for (int b0 = b_lo; b0 < b_hi; b0 += 16) {
        int c[16];
#pragma unroll
        for (int i = 0; i < 16; i++) c[i] = b0 + i < b_hi ? cnt[(b0 + i) * E + e] : 0;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            t += c[i];
            p += b0 + i < upto ? c[i] : 0;
        }
    }
    part_t[qt][e] = t;
    if (part_p) part_p[qt][e] = p;
}

__device__ void place_chunk(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt, int nblk,
                            int32_t* __restrict__ perm, int32_t* __restrict__ pos_of, const float* __restrict__ wt,
                            float* __restrict__ wsort, int N) {
    __shared__ int wtot[4];
    __shared__ int part_t[4][E], part_p[4][E];
    __shared__ int base[E];
    __shared__ int wcnt[PLACE_WAVES][E];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, b = blockIdx.x;
    // this chunk's expert ids and routing weights, loaded with the counts
    int eid[SORT_CH / PLACE_THREADS];
    float wa[SORT_CH / PLACE_THREADS];
#pragma unroll
    for (int i = 0; i < SORT_CH / PLACE_THREADS; i++) {
        const int a = b * SORT_CH + i * PLACE_THREADS + tid;
        eid[i] = idx[min(a, N - 1)];  // past the end: a copy, never placed
        wa[i] = wt[min(a, N - 1)];
    }
    count_quarter(cnt, nblk, b, part_t, part_p);
    for (int i = tid; i < PLACE_WAVES * E; i += PLACE_THREADS) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    const int e = tid & (E - 1);
    const int total = part_t[0][e] + part_t[1][e] + part_t[2][e] + part_t[3][e];
    const int before = part_p[0][e] + part_p[1][e] + part_p[2][e] + part_p[3][e];
    const int tv[1] = {total};
    int off[1], all[1];
    scan_256<1>(tv, off, all, wtot);
    if (tid < 256) base[e] = off[0] + before;
    __syncthreads();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int i = 0; i < SORT_CH / PLACE_THREADS; i++) {
        const int a = b * SORT_CH + i * PLACE_THREADS + tid;
        const bool valid = a < N;
        const int ea = eid[i];
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; bit++) {
            const uint64_t bb = __ballot((ea >> bit) & 1);
            peers &= ((ea >> bit) & 1) ? bb : ~bb;
        }
        const int rank = __popcll(peers & lt);
        if (valid && rank == 0) wcnt[wave][ea] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int pos = base[ea] + rank;
            for (int w = 0; w < wave; w++) pos += wcnt[w][ea];
            perm[pos] = a;
            pos_of[a] = pos;
            wsort[pos] = wa[i];
        }
        __syncthreads();
        if (tid < E) {
            int add = 0;
#pragma unroll
            for (int w = 0; w < PLACE_WAVES; w++) {
                add += wcnt[w][tid];
                wcnt[w][tid] = 0;
            }
            base[tid] += add;
        }
        __syncthreads();
    }
}

__device__ void tile_map(const int32_t* __restrict__ cnt, int nblk, int32_t* __restrict__ offs,
                         int32_t* __restrict__ tiles, int32_t* __restrict__ tiles_e, int32_t* __restrict__ tile_count,
                         int bm) {
    __shared__ int wtot[4 * 6];
    __shared__ int part_t[4][E];
    __shared__ int start4[E + 1];  // exclusive start of each expert's tiles in the four-group class
    __shared__ int starte[E + 1];  // the same in expert order
    __shared__ int s_run[E], s_off[E];
    const int tid = threadIdx.x, e = tid & (E - 1);
    count_quarter(cnt, nblk, 0, part_t, nullptr);
    __syncthreads();
    const int run = part_t[0][e] + part_t[1][e] + part_t[2][e] + part_t[3][e];  // expert e's assignments
    // classes: live 32-row groups of each tile (4 for a full tile)
    const int n_full = run / bm, part_rows = run - n_full * bm;
    const int g_part = (part_rows + 31) >> 5;  // 0 when there is no partial tile
    // the scanned sets: the expert's assignments, its tiles with 4, 3, 2, 1
    // live groups, and all its tiles
    int sv[6];
    sv[0] = run;
    sv[1] = n_full + (g_part == 4);
#pragma unroll
    for (int q = 1; q < 4; q++) sv[1 + q] = (g_part == 4 - q);
    sv[5] = n_full + (part_rows > 0);
    int sx[6], st[6];
    scan_256<6>(sv, sx, st, wtot);
    const int off = sx[0], toff = sx[5], ntot = st[5];
    int cls[4], start[4], tot[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        cls[q] = sv[1 + q];
        start[q] = sx[1 + q];
        tot[q] = st[1 + q];
    }
    if (tid < 256) {
        s_run[e] = run;
        s_off[e] = off;
        offs[e] = off;
        if (e == E - 1) offs[E] = off + run;
    }
    if (tid < 256) {
        start4[e] = start[0];
        starte[e] = toff;
        if (e == E - 1) {
            start4[E] = tot[0];
            starte[E] = ntot;
        }
    }
    __syncthreads();
    // four-group class: tile p belongs to the expert whose range holds it
    for (int p = tid; p < tot[0]; p += PLACE_THREADS) {
        int lo = 0, hi = E - 1;  // largest x with start4[x] <= p (empty ranges share starts)
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (start4[mid] <= p) lo = mid;
            else hi = mid - 1;
        }
        const int j = p - start4[lo];
        *(int4*)&tiles[4 * p] = make_int4(lo, j * bm, s_off[lo], min(bm, s_run[lo] - j * bm));
    }
    // the other classes: at most one (partial) tile per expert
    if (tid < 256) {
        int base = tot[0];
#pragma unroll
        for (int q = 1; q < 4; q++) {
            if (cls[q]) *(int4*)&tiles[4 * (base + start[q])] = make_int4(e, n_full * bm, off, part_rows);
            base += tot[q];
        }
        if (e == 0) tile_count[0] = base;
    }
    // the same records in expert order (each expert's tiles in row order)
    for (int p = tid; p < ntot; p += PLACE_THREADS) {
        int lo = 0, hi = E - 1;  // largest x with starte[x] <= p
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (starte[mid] <= p) lo = mid;
            else hi = mid - 1;
        }
        const int j = p - starte[lo];
        *(int4*)&tiles_e[4 * p] = make_int4(lo, j * bm, s_off[lo], min(bm, s_run[lo] - j * bm));
    }
}

__global__ void __launch_bounds__(PLACE_THREADS) k_sort_place(const int32_t* __restrict__ idx,
                                                              const int32_t* __restrict__ cnt, int nblk,
                                                              int32_t* __restrict__ offs, int32_t* __restrict__ tiles,
                                                              int32_t* __restrict__ tiles_e,
                                                              int32_t* __restrict__ tile_count,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ pos_of,
                                                              const float* __restrict__ w,
                                                              float* __restrict__ wsort, int N, int bm) {
    if ((int)blockIdx.x == nblk) tile_map(cnt, nblk, offs, tiles, tiles_e, tile_count, bm);
    else place_chunk(idx, cnt, nblk, perm, pos_of, w, wsort, N);
}

hipError_t launch_sort(const int32_t* idx, int N, int32_t* cnt, int32_t* offs, int32_t* tiles, int32_t* tiles_e,
                       int32_t* tile_count, int32_t* perm, int32_t* pos_of, const float* w, float* wsort, int bm,
                       hipStream_t s) {
    const int nblk = (N + SORT_CH - 1) / SORT_CH;  // the histograms come from the top-k launch
    hipLaunchKernelGGL(k_sort_place, dim3(nblk + 1), dim3(PLACE_THREADS), 0, s, idx, cnt, nblk, offs, tiles, tiles_e,
                       tile_count, perm, pos_of, w, wsort, N, bm);
    return hipGetLastError();
}

int sort_blocks(int N) { return (N + SORT_CH - 1) / SORT_CH; }
int sort_chunk() { return SORT_CH; }

}  // namespace moe
