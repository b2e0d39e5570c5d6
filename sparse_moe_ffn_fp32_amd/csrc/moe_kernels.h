// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Optional pair of events for one kernel id (MOE_FFN_KERNEL_*): the launch
// of that kernel goes through hipExtLaunchKernelGGL, which stamps the events
// with the kernel's own start and end.
struct Tracer {
    int kernel = 0;
    hipEvent_t start = nullptr, stop = nullptr;
    template <typename... KArgs, typename... Args>
    void launch(int id, void (*k)(KArgs...), dim3 grid, dim3 block, size_t shm, hipStream_t s, Args... args) const {
        if (id == kernel && start && stop)
            hipExtLaunchKernelGGL(k, grid, block, shm, s, start, stop, 0, args...);
        else
            hipLaunchKernelGGL(k, grid, block, shm, s, args...);
    }
};


// ---- router (k_router.hip)
// one launch: router fp32 -> fp16 hi/lo planes wr2 [2, E, D] with row
// exponents er [E]; shared bf16 (when sg != nullptr) -> fp16 shw [gate | up |
// down] with row exponents es [2 FS + D]; x bf16 [T, D] -> fp16 xh (perm8)
// with row exponents ex [T], and the shared-expert gate sgate [T] =
// sigmoid(gate_inp . x), 1 without gate_inp; cnt [n_cnt] zeroed
hipError_t launch_prep(const float* wr, uint16_t* wr2, int32_t* er, const uint16_t* sg, const uint16_t* su,
                       const uint16_t* sd, uint16_t* shw, int32_t* es, const uint16_t* x, uint16_t* xh, int32_t* ex,
                       const uint16_t* gate_inp, float* sgate, int T, int32_t* cnt, int n_cnt, hipStream_t s);
// wscale multiplies every renormalised routing weight
// tid2eid != nullptr: hash routing with token_ids [T] (n_vocab table columns)
// cnt [N / chunk, E] (zeroed before): the assignments a of each chunk a / chunk
// counted per expert (the sort's histograms)
hipError_t launch_topk(const float* logits, int32_t* idx, float* w, float wscale, int gating, const int32_t* tid2eid,
                       const int32_t* token_ids, int n_vocab, int T, int32_t* cnt, int chunk, hipStream_t s);

// ---- routing sort (k_sort.hip)
int sort_blocks(int N);
int sort_chunk();  // assignments per histogram chunk
// cnt: the per-chunk expert counts (launch_topk); tiles: the tile records
// longest first; tiles_e: the same records in expert order; w: the routing
// weights by assignment, wsort: the same by sorted position
hipError_t launch_sort(const int32_t* idx, int N, int32_t* cnt, int32_t* offs, int32_t* tiles, int32_t* tiles_e,
                       int32_t* tile_count, int32_t* perm, int32_t* pos_of, const float* w, float* wsort, int bm,
                       hipStream_t s);

// ---- grouped GEMMs (k_gemm.hip)
struct PrefillGemmParams {
    const uint16_t* xh;
    const int32_t* ex;   // [T] exponents of the fp16 x rows
    const uint16_t* shw; // shared expert fp16 [gate FS x D | up FS x D | down D x FS]
    const int32_t* es;   // their row exponents [2 FS + D]
    uint16_t* h;
    int32_t* eh;         // [N_assign, 2] exponents of h (per 256-feature half)
    uint16_t* hs;
    int32_t* ehs;        // [T, 4] exponents of the shared h (per 128 features)
    int32_t* ep;         // [N_assign, 4] exponents of the partials (per 512 outputs)
    const int32_t* perm;
    const int32_t* pos_of;
    const int32_t* offs;
    const int32_t* tiles;     // tile records, longest first
    const int32_t* tiles_e;   // the same records in expert order
    const int32_t* tile_count;
    const float* wsort;  // [N_assign] routing weight of each expert-sorted position
    const float* sgate;
    const uint32_t *gate_q, *up_q, *down_q;
    const uint16_t *gate_s, *up_s, *down_s;
    const uint16_t *gate_b, *up_b, *down_b;
    int gu_rows;  // rows per expert in the gate/up arrays (F, or 2F for the fused layout)
    uint16_t* partial;  // fp16 [N_assign, D], times 2^-ep
    const uint16_t* resid;  // bf16 [T, D] added to y before its rounding, or nullptr
    uint16_t* y;
    int T;
};
int gemm_bm(int T);  // rows per routed tile for a prefill pass of T tokens
// router logits, and the shared expert's gate/up + SwiGLU into hs (ehs)
// when shw != nullptr
hipError_t launch_router_gemm(const uint16_t* xh, const int32_t* ex, const uint16_t* wr2, const int32_t* er,
                              const float* bias, float* logits, const uint16_t* shw, const int32_t* es, uint16_t* hs,
                              int32_t* ehs, int T, const Tracer& tr, hipStream_t s);
hipError_t launch_prefill_gemms(const PrefillGemmParams& p, const Tracer& tr, hipStream_t s);
// xn[T, D] bf16 = RMS-normalised h times w (k_norm.hip)
hipError_t launch_rmsnorm(const uint16_t* h, const float* w, float eps, uint16_t* xn, int T, hipStream_t s);

// ---- decode path (k_decode.hip), T <= 64
struct DecodeLayout {
    size_t logits, xp, hs, ys, h, part, idx, w, sgate, xsum, total;
};
struct DecodeParams {
    const uint16_t* x;
    int T;
    const float *router_w, *router_b;
    float wscale;  // factor on the renormalised routing weights
    int gating;    // MOE_FFN_GATING_*
    const int32_t* tid2eid;    // hash routing table [K, n_vocab] or nullptr
    const int32_t* token_ids;  // [T] with the table
    int n_vocab;
    const uint16_t *sh_gate_inp, *sh_gate, *sh_up, *sh_down;  // sh_gate == nullptr: no shared expert
    const uint32_t *gate_q, *up_q, *down_q;
    const uint16_t *gate_s, *gate_b, *up_s, *up_b, *down_s, *down_b;
    int gu_rows;   // rows per expert in the gate/up arrays (F, or 2F for the fused layout)
    int32_t* idx;  // user outputs or nullptr
    float* w;
    const uint16_t* resid;  // bf16 [T, D] added to y before its rounding, or nullptr
    // norm_w != nullptr: x is the un-normalised residual stream; the path
    // first forms xn = bf16(RMSNorm(x) * norm_w) (written to xn) and runs the
    // FFN on it
    const float* norm_w;
    float eps;
    uint16_t* xn;  // [T, D]
    uint16_t* y;
};
size_t decode_workspace_bytes(int T, DecodeLayout* L);
hipError_t launch_decode(const DecodeParams& p, char* ws, const Tracer& tr, hipStream_t s);

}  // namespace moe
