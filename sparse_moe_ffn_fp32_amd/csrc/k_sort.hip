// Token->expert histogram, prefix scan and stable counting sort (subsystem 2).
//
// The grouped expert GEMMs need each expert's routed rows stored together.
// As on the Lily engine page ("Palikti ekspertu marsrutizavima GPU" -- keep
// expert routing on the GPU), a histogram counts the assignments per expert,
// a prefix scan turns counts into start offsets, a scatter writes every
// assignment into its expert's segment, and a tile map lists the fixed-size
// row tiles the GEMMs process.  Nothing returns to the host.
//
// Assignment a = t*8 + r is token t's r-th selected expert.  The scatter is
// stable: inside an expert's segment assignments keep increasing a (i.e.
// token) order, so the permutation is a pure function of the routing.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int SORT_CH = 2048;  // assignments per histogram/scatter block

__global__ void __launch_bounds__(256) k_sort_hist(const int32_t* __restrict__ idx, int32_t* __restrict__ cnt, int N) {
    __shared__ int h[E];
    h[threadIdx.x] = 0;
    __syncthreads();
    const int base = blockIdx.x * SORT_CH;
#pragma unroll
    for (int i = 0; i < SORT_CH / 256; i++) {
        int a = base + i * 256 + threadIdx.x;
        if (a < N) atomicAdd(&h[idx[a]], 1);
    }
    __syncthreads();
    cnt[blockIdx.x * E + threadIdx.x] = h[threadIdx.x];
}

// Exclusive scan of 256 ints held one per thread; returns the total.
__device__ int block_exclusive_scan_256(int v, int* smem, int& total) {
    const int tid = threadIdx.x;
    smem[tid] = v;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        int t = tid >= off ? smem[tid - off] : 0;
        __syncthreads();
        smem[tid] += t;
        __syncthreads();
    }
    int incl = smem[tid];
    total = smem[255];
    __syncthreads();
    return incl - v;
}

// One block: per-(block, expert) bases, expert offsets offs[0..E], and the
// tile map: record i is tiles[4i .. 4i+3] = {expert, first row of the tile
// within the expert's segment, segment start, rows in the tile (1..bm)};
// tile_count[0] = number of tiles.
__global__ void __launch_bounds__(256) k_sort_scan(int32_t* __restrict__ cnt, int nblk, int32_t* __restrict__ offs,
                                                   int32_t* __restrict__ tiles, int32_t* __restrict__ tile_count,
                                                   int bm) {
    __shared__ int smem[256];
    const int e = threadIdx.x;
    int run = 0;
    for (int b = 0; b < nblk; b++) {
        int c = cnt[b * E + e];
        cnt[b * E + e] = run;
        run += c;
    }
    int total;
    const int off = block_exclusive_scan_256(run, smem, total);
    for (int b = 0; b < nblk; b++) cnt[b * E + e] += off;
    offs[e] = off;
    if (e == E - 1) offs[E] = off + run;
    const int nt = (run + bm - 1) / bm;
    int ntot;
    const int toff = block_exclusive_scan_256(nt, smem, ntot);
    for (int j = 0; j < nt; j++)
        *(int4*)&tiles[4 * (toff + j)] = make_int4(e, j * bm, off, min(bm, run - j * bm));
    if (e == 0) tile_count[0] = ntot;
}

// Stable scatter: perm[pos] = a and pos_of[a] = pos.  Each block walks its
// chunk in assignment order, 256 at a time; ranks among equal experts inside
// a wave come from ballots on the 8 bits of the expert id.
__global__ void __launch_bounds__(256) k_sort_scatter(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
                                                      int32_t* __restrict__ perm, int32_t* __restrict__ pos_of, int N) {
    __shared__ int base[E];
    __shared__ int wcnt[4][E];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    base[tid] = cnt[blockIdx.x * E + tid];
#pragma unroll
    for (int w = 0; w < 4; w++) wcnt[w][tid] = 0;
    __syncthreads();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int i = 0; i < SORT_CH / 256; i++) {
        const int a = blockIdx.x * SORT_CH + i * 256 + tid;
        const bool valid = a < N;
        const int e = valid ? idx[a] : 0;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; bit++) {
            uint64_t b = __ballot((e >> bit) & 1);
            peers &= ((e >> bit) & 1) ? b : ~b;
        }
        const int rank = __popcll(peers & lt);
        if (valid && rank == 0) wcnt[wave][e] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int pos = base[e] + rank;
            for (int w = 0; w < wave; w++) pos += wcnt[w][e];
            perm[pos] = a;
            pos_of[a] = pos;
        }
        __syncthreads();
        base[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
#pragma unroll
        for (int w = 0; w < 4; w++) wcnt[w][tid] = 0;
        __syncthreads();
    }
}

hipError_t launch_sort(const int32_t* idx, int N, int32_t* cnt, int32_t* offs, int32_t* tiles, int32_t* tile_count,
                       int32_t* perm, int32_t* pos_of, int bm, hipStream_t s) {
    const int nblk = (N + SORT_CH - 1) / SORT_CH;
    hipLaunchKernelGGL(k_sort_hist, dim3(nblk), dim3(256), 0, s, idx, cnt, N);
    hipLaunchKernelGGL(k_sort_scan, dim3(1), dim3(256), 0, s, cnt, nblk, offs, tiles, tile_count, bm);
    hipLaunchKernelGGL(k_sort_scatter, dim3(nblk), dim3(256), 0, s, idx, cnt, perm, pos_of, N);
    return hipGetLastError();
}

int sort_blocks(int N) { return (N + SORT_CH - 1) / SORT_CH; }

}  // namespace moe
