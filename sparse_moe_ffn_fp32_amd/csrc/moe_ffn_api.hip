// C-ABI entry points: argument validation, workspace carve-up, path choice,
// launches on the caller's stream.  See include/moe_ffn.h for the contract.
#include <atomic>
#include <mutex>

#include "../../include/moe_ffn.h"
#include "moe_common.h"
#include "moe_kernels.h"

// Scratch of moe_ffn_forward_noalloc: one copy per GPU, alive until the
// process ends.  Host code never uses this name as an address (on the host it
// is only a stand-in): the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[MOE_FFN_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace moe;

constexpr size_t ALIGN = 256;
size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

// Byte offsets of every workspace region for T tokens.
struct Layout {
    size_t wr2, er, shw, es, logits, idx, w, sgate, xh, ex, cnt, offs, tiles, tiles_e, tile_count, perm, pos_of, wsort, h, eh,
        hs, ehs, partial, ep, total;
};

Layout layout(int64_t T) {
    const size_t N = (size_t)T * K;
    const int nblk = sort_blocks((int)N);
    const size_t max_tiles = (N + 127) / 128 + E;  // tiles of at least 128 rows
    Layout L{};
    size_t o = 0;
    L.wr2 = o;        o += up((size_t)2 * E * D * 2);
    L.er = o;         o += up((size_t)E * 4);
    L.shw = o;        o += up((size_t)(2 * FS * D + D * FS) * 2);
    L.es = o;         o += up((size_t)(2 * FS + D) * 4);
    L.logits = o;     o += up((size_t)T * E * 4);
    L.idx = o;        o += up(N * 4);
    L.w = o;          o += up(N * 4);
    L.sgate = o;      o += up((size_t)T * 4);
    L.xh = o;         o += up((size_t)T * D * 2);
    L.ex = o;         o += up((size_t)T * 4);
    L.cnt = o;        o += up((size_t)nblk * E * 4);
    L.offs = o;       o += up((E + 1) * 4);
    L.tiles = o;      o += up(max_tiles * 4 * 4);
    L.tiles_e = o;    o += up(max_tiles * 4 * 4);
    L.tile_count = o; o += up(4);
    L.perm = o;       o += up(N * 4);
    L.pos_of = o;     o += up(N * 4);
    L.wsort = o;      o += up(N * 4);
    L.h = o;          o += up(N * F * 2);
    L.eh = o;         o += up(N * 2 * 4);
    L.hs = o;         o += up((size_t)T * FS * 2);
    L.ehs = o;        o += up((size_t)T * 4 * 4);
    L.partial = o;    o += up(N * D * 2);
    L.ep = o;         o += up(N * 4 * 4);
    L.total = o;
    return L;
}

// Both paths' regions, so any path can run in a workspace sized for T; the
// prefill regions are sized for one pass of at most MOE_FFN_PREFILL_CHUNK_T.
size_t workspace_bytes(int64_t T) {
    size_t b = layout(T < MOE_FFN_PREFILL_CHUNK_T ? T : MOE_FFN_PREFILL_CHUNK_T).total;
    if (T <= MOE_FFN_DECODE_MAX_T) {
        const size_t d = decode_workspace_bytes((int)T, nullptr);
        if (d > b) b = d;
    }
    return b;
}

bool dims_ok(const moe_ffn_dims* d) {
    return d->d_model == D && d->n_experts == E && d->top_k == K && d->d_ff == F && d->d_ff_shared == FS &&
           d->group_size == G;
}

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The factor on the renormalised routing weights (0 is read as 1).
float weights_scale(const moe_ffn_router* r) { return r->weights_scale == 0.0f ? 1.0f : r->weights_scale; }

// The gate and up tensors as the kernels see them: row (e, f) of gate at
// gq + (e * rows + f) * D/8 (scales, biases at (e * rows + f) * D/G), the
// same for up.  Separate tensors: rows = F.  Fused [E, 2F, ...] tensor:
// rows = 2F, up = gate + F rows.
struct GateUp {
    const uint32_t *gq, *uq;
    const uint16_t *gs, *us, *gb, *ub;
    int rows;
};
GateUp resolve_gate_up(const moe_ffn_experts* ex) {
    const moe_q4_tensor& g = ex->gate;
    if (ex->gate_up_fused) {
        if (!g.qweight || !g.scales || !g.biases) return {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 2 * F};
        return {g.qweight, g.qweight + (size_t)F * (D / 8), g.scales, g.scales + (size_t)F * (D / G),
                g.biases, g.biases + (size_t)F * (D / G), 2 * F};
    }
    const moe_q4_tensor& u = ex->up;
    return {g.qweight, u.qweight, g.scales, u.scales, g.biases, u.biases, F};
}

// Every argument check except the workspace's.
int validate_args(const moe_ffn_dims* dims, int64_t T, const uint16_t* x, const moe_ffn_router* router,
                  const moe_ffn_experts* ex, const moe_ffn_shared* sh, uint16_t* y, int32_t* topk_idx,
                  float* topk_weight, int path) {
    if (!dims || T < 0 || path < MOE_FFN_PATH_AUTO || path > MOE_FFN_PATH_PREFILL) return MOE_FFN_EINVAL;
    if (!dims_ok(dims)) return MOE_FFN_EUNSUPPORTED;
    if (T > MOE_FFN_MAX_T) return MOE_FFN_EUNSUPPORTED;
    if (T == 0) return MOE_FFN_OK;
    if (!x || !y || !router || !router->weight || !ex) return MOE_FFN_EINVAL;
    if (!(router->weights_scale >= 0.0f) || router->weights_scale == INFINITY) return MOE_FFN_EINVAL;
    if (router->gating != MOE_FFN_GATING_SOFTMAX && router->gating != MOE_FFN_GATING_SQRT_SOFTPLUS) return MOE_FFN_EINVAL;
    if (router->tid2eid && (!router->token_ids || router->n_vocab < 1)) return MOE_FFN_EINVAL;
    if (ex->gate_up_fused != 0 && ex->gate_up_fused != 1) return MOE_FFN_EINVAL;
    if (ex->gate_up_fused && (ex->up.qweight || ex->up.scales || ex->up.biases)) return MOE_FFN_EINVAL;
    const GateUp gu = resolve_gate_up(ex);
    const void* req[] = {gu.gq, gu.gs, gu.gb, gu.uq, gu.us, gu.ub, ex->down.qweight, ex->down.scales, ex->down.biases};
    for (const void* p : req)
        if (!p) return MOE_FFN_EINVAL;
    if (sh && (!sh->gate || !sh->up || !sh->down)) return MOE_FFN_EINVAL;
    for (const void* p : req)
        if (!al16(p)) return MOE_FFN_EALIGN;
    const void* opt[] = {x, y, router->weight, router->bias, topk_idx, topk_weight, router->tid2eid,
                         router->tid2eid ? router->token_ids : nullptr,
                         sh ? sh->gate : nullptr, sh ? sh->up : nullptr, sh ? sh->down : nullptr,
                         sh ? sh->gate_inp : nullptr};
    for (const void* p : opt)
        if (p && !al16(p)) return MOE_FFN_EALIGN;
    if (path == MOE_FFN_PATH_DECODE && T > MOE_FFN_DECODE_MAX_T) return MOE_FFN_EUNSUPPORTED;
    return MOE_FFN_OK;
}

int validate(const moe_ffn_dims* dims, int64_t T, const uint16_t* x, const moe_ffn_router* router,
             const moe_ffn_experts* ex, const moe_ffn_shared* sh, uint16_t* y, int32_t* topk_idx,
             float* topk_weight, void* ws, size_t ws_bytes, int path) {
    const int st = validate_args(dims, T, x, router, ex, sh, y, topk_idx, topk_weight, path);
    if (st != MOE_FFN_OK || T == 0) return st;
    if (ws && !al16(ws)) return MOE_FFN_EALIGN;
    if (!ws || ws_bytes < workspace_bytes(T)) return MOE_FFN_EWORKSPACE;
    return MOE_FFN_OK;
}

// Workspace of the block entry point: the FFN's own, then the normalised
// input of one pass (T tokens on the decode path, at most
// MOE_FFN_PREFILL_CHUNK_T on the prefill path).
size_t block_workspace_bytes(int64_t T) {
    const int64_t tc = T < MOE_FFN_PREFILL_CHUNK_T ? T : MOE_FFN_PREFILL_CHUNK_T;
    return up(workspace_bytes(T)) + up((size_t)tc * D * 2);
}

int run_prefill(int T, const uint16_t* x, const moe_ffn_router* router, const moe_ffn_experts* ex,
                const moe_ffn_shared* sh, uint16_t* y, int32_t* idx_user, float* w_user, char* ws,
                const uint16_t* resid, const Tracer& tr, hipStream_t s) {
    const Layout L = layout(T);
    const int N = T * K;
    auto at = [&](size_t off) { return (void*)(ws + off); };
    uint16_t* wr2 = (uint16_t*)at(L.wr2);
    float* logits = (float*)at(L.logits);
    int32_t* idx = idx_user ? idx_user : (int32_t*)at(L.idx);
    float* w = w_user ? w_user : (float*)at(L.w);
    float* sgate = (float*)at(L.sgate);
    uint16_t* xh = (uint16_t*)at(L.xh);
    int32_t* cnt = (int32_t*)at(L.cnt);
    int32_t* offs = (int32_t*)at(L.offs);
    int32_t* tiles = (int32_t*)at(L.tiles);
    int32_t* tile_count = (int32_t*)at(L.tile_count);
    int32_t* perm = (int32_t*)at(L.perm);
    int32_t* pos_of = (int32_t*)at(L.pos_of);

    int32_t* er = (int32_t*)at(L.er);
    uint16_t* shw = sh ? (uint16_t*)at(L.shw) : nullptr;
    int32_t* es = (int32_t*)at(L.es);
    int32_t* xe = (int32_t*)at(L.ex);

    hipError_t e = hipSuccess;
    auto chk = [&](hipError_t r) { if (e == hipSuccess) e = r; };
    const int n_cnt = sort_blocks(N) * E;
    chk(launch_prep(router->weight, wr2, er, sh ? sh->gate : nullptr, sh ? sh->up : nullptr, sh ? sh->down : nullptr,
                    shw, es, x, xh, xe, sh ? sh->gate_inp : nullptr, sgate, T, cnt, n_cnt, s));
    chk(launch_router_gemm(xh, xe, wr2, er, router->bias, logits, shw, es, (uint16_t*)at(L.hs), (int32_t*)at(L.ehs), T,
                           tr, s));
    chk(launch_topk(logits, idx, w, weights_scale(router), router->gating, router->tid2eid, router->token_ids,
                    router->n_vocab, T, cnt, sort_chunk(), s));
    int32_t* tiles_e = (int32_t*)at(L.tiles_e);
    float* wsort = (float*)at(L.wsort);
    chk(launch_sort(idx, N, cnt, offs, tiles, tiles_e, tile_count, perm, pos_of, w, wsort, gemm_bm(T), s));
    PrefillGemmParams p{};
    p.xh = xh;
    p.ex = xe;
    p.shw = shw;
    p.es = es;
    p.h = (uint16_t*)at(L.h);
    p.eh = (int32_t*)at(L.eh);
    p.hs = (uint16_t*)at(L.hs);
    p.ehs = (int32_t*)at(L.ehs);
    p.ep = (int32_t*)at(L.ep);
    p.perm = perm;
    p.pos_of = pos_of;
    p.offs = offs;
    p.tiles = tiles;
    p.tiles_e = tiles_e;
    p.tile_count = tile_count;
    p.wsort = wsort;
    p.sgate = sgate;
    const GateUp gu = resolve_gate_up(ex);
    p.gate_q = gu.gq; p.gate_s = gu.gs; p.gate_b = gu.gb;
    p.up_q = gu.uq;   p.up_s = gu.us;   p.up_b = gu.ub;
    p.gu_rows = gu.rows;
    p.down_q = ex->down.qweight; p.down_s = ex->down.scales; p.down_b = ex->down.biases;
    p.partial = (uint16_t*)at(L.partial);
    p.resid = resid;
    p.y = y;
    p.T = T;
    chk(launch_prefill_gemms(p, tr, s));
    return e == hipSuccess ? MOE_FFN_OK : MOE_FFN_EHIP;
}

// The FFN of every entry point.  With norm_w == nullptr: y = FFN(x).  With
// norm_w: x is the residual stream, each pass first writes its rows of
// RMSNorm(x) * norm_w (bf16) into xn, runs the FFN on them and adds x to the
// output before its rounding.
int forward_impl(int64_t T, const uint16_t* x, const float* norm_w, float eps, uint16_t* xn,
                 const moe_ffn_router* router, const moe_ffn_experts* experts, const moe_ffn_shared* shared,
                 uint16_t* y, int32_t* topk_idx, float* topk_weight, void* workspace, hipStream_t stream, int path,
                 const moe_ffn_trace* trace) {
    Tracer tr;
    if (trace) {
        tr.kernel = trace->kernel;
        tr.start = (hipEvent_t)trace->start;
        tr.stop = (hipEvent_t)trace->stop;
    }
    const bool decode = path == MOE_FFN_PATH_DECODE || (path == MOE_FFN_PATH_AUTO && T <= MOE_FFN_DECODE_MAX_T);
    if (!decode) {
        // passes over token slices of at most MOE_FFN_PREFILL_CHUNK_T (a
        // traced kernel is bracketed in every pass; the events keep the last)
        for (int64_t c0 = 0; c0 < T; c0 += MOE_FFN_PREFILL_CHUNK_T) {
            const int tc = (int)(T - c0 < MOE_FFN_PREFILL_CHUNK_T ? T - c0 : MOE_FFN_PREFILL_CHUNK_T);
            const uint16_t* xin = x + c0 * D;
            moe_ffn_router rc = *router;  // this slice's token ids
            if (rc.tid2eid) rc.token_ids += c0;
            if (norm_w) {
                if (launch_rmsnorm(x + c0 * D, norm_w, eps, xn, tc, stream) != hipSuccess) return MOE_FFN_EHIP;
                xin = xn;
            }
            const int r = run_prefill(tc, xin, &rc, experts, shared, y + c0 * D,
                                      topk_idx ? topk_idx + c0 * K : nullptr, topk_weight ? topk_weight + c0 * K : nullptr,
                                      (char*)workspace, norm_w ? x + c0 * D : nullptr, tr, stream);
            if (r != MOE_FFN_OK) return r;
        }
        return MOE_FFN_OK;
    }
    DecodeParams p{};
    p.x = x;
    p.norm_w = norm_w;
    p.eps = eps;
    p.xn = xn;
    p.T = (int)T;
    p.router_w = router->weight;
    p.router_b = router->bias;
    p.wscale = weights_scale(router);
    p.gating = router->gating;
    p.tid2eid = router->tid2eid;
    p.token_ids = router->token_ids;
    p.n_vocab = router->n_vocab;
    p.sh_gate_inp = shared ? shared->gate_inp : nullptr;
    p.sh_gate = shared ? shared->gate : nullptr;
    p.sh_up = shared ? shared->up : nullptr;
    p.sh_down = shared ? shared->down : nullptr;
    const GateUp gu = resolve_gate_up(experts);
    p.gate_q = gu.gq; p.gate_s = gu.gs; p.gate_b = gu.gb;
    p.up_q = gu.uq;   p.up_s = gu.us;   p.up_b = gu.ub;
    p.gu_rows = gu.rows;
    p.down_q = experts->down.qweight; p.down_s = experts->down.scales; p.down_b = experts->down.biases;
    p.idx = topk_idx;
    p.w = topk_weight;
    p.resid = norm_w ? x : nullptr;
    p.y = y;
    return launch_decode(p, (char*)workspace, tr, stream) == hipSuccess ? MOE_FFN_OK : MOE_FFN_EHIP;
}

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept per device.
constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch[MAX_DEVICES];
std::mutex g_scratch_mu;

int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MOE_FFN_EHIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_FFN_EHIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_FFN_OK;
}

}  // namespace

extern "C" {

int moe_ffn_forward_noalloc(const moe_ffn_dims* dims, int64_t T, const uint16_t* x, const moe_ffn_router* router,
                            const moe_ffn_experts* experts, const moe_ffn_shared* shared, uint16_t* y,
                            int32_t* topk_idx, float* topk_weight, void* stream) {
    if (dims && dims_ok(dims) && T > MOE_FFN_NOALLOC_MAX_T && T <= MOE_FFN_MAX_T) return MOE_FFN_ETOOBIG;
    int st = validate_args(dims, T, x, router, experts, shared, y, topk_idx, topk_weight, MOE_FFN_PATH_DECODE);
    if (st != MOE_FFN_OK || T == 0) return st;
    if (decode_workspace_bytes((int)T, nullptr) > MOE_FFN_NOALLOC_SCRATCH_BYTES) return MOE_FFN_ETOOBIG;
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != MOE_FFN_OK) return st;
    return forward_impl(T, x, nullptr, 0.0f, nullptr, router, experts, shared, y, topk_idx, topk_weight, ws,
                        (hipStream_t)stream, MOE_FFN_PATH_DECODE, nullptr);
}

size_t moe_ffn_workspace_size(const moe_ffn_dims* dims, int64_t T) {
    if (!dims || !dims_ok(dims) || T <= 0 || T > MOE_FFN_MAX_T) return 0;
    return workspace_bytes(T);
}

int moe_ffn_forward_traced(const moe_ffn_dims* dims, int64_t T, const uint16_t* x, const moe_ffn_router* router,
                           const moe_ffn_experts* experts, const moe_ffn_shared* shared, uint16_t* y,
                           int32_t* topk_idx, float* topk_weight, void* workspace, size_t workspace_bytes,
                           void* stream, int path, const moe_ffn_trace* trace) {
    int st = validate(dims, T, x, router, experts, shared, y, topk_idx, topk_weight, workspace, workspace_bytes,
                      path);
    if (st != MOE_FFN_OK || T == 0) return st;
    return forward_impl(T, x, nullptr, 0.0f, nullptr, router, experts, shared, y, topk_idx, topk_weight, workspace,
                        (hipStream_t)stream, path, trace);
}

size_t moe_ffn_block_workspace_size(const moe_ffn_dims* dims, int64_t T) {
    if (!dims || !dims_ok(dims) || T <= 0 || T > MOE_FFN_MAX_T) return 0;
    return block_workspace_bytes(T);
}

int moe_ffn_block_forward_traced(const moe_ffn_dims* dims, int64_t T, const uint16_t* h, const float* norm_weight,
                                 float eps, const moe_ffn_router* router, const moe_ffn_experts* experts,
                                 const moe_ffn_shared* shared, uint16_t* y, int32_t* topk_idx, float* topk_weight,
                                 void* workspace, size_t ws_bytes, void* stream, int path,
                                 const moe_ffn_trace* trace) {
    // the FFN's own checks, then the norm's, then the larger workspace
    const int st = validate(dims, T, h, router, experts, shared, y, topk_idx, topk_weight, workspace, ws_bytes, path);
    if (T == 0 || (st != MOE_FFN_OK && st != MOE_FFN_EWORKSPACE)) return st;
    if (!norm_weight || !(eps >= 0.0f) || !__builtin_isfinite(eps)) return MOE_FFN_EINVAL;
    if (!al16(norm_weight)) return MOE_FFN_EALIGN;
    if (st != MOE_FFN_OK || ws_bytes < block_workspace_bytes(T)) return MOE_FFN_EWORKSPACE;
    uint16_t* xn = (uint16_t*)((char*)workspace + up(workspace_bytes(T)));
    return forward_impl(T, h, norm_weight, eps, xn, router, experts, shared, y, topk_idx, topk_weight, workspace,
                        (hipStream_t)stream, path, trace);
}

int moe_ffn_block_forward(const moe_ffn_dims* dims, int64_t T, const uint16_t* h, const float* norm_weight, float eps,
                          const moe_ffn_router* router, const moe_ffn_experts* experts, const moe_ffn_shared* shared,
                          uint16_t* y, int32_t* topk_idx, float* topk_weight, void* workspace, size_t workspace_bytes,
                          void* stream) {
    return moe_ffn_block_forward_traced(dims, T, h, norm_weight, eps, router, experts, shared, y, topk_idx,
                                        topk_weight, workspace, workspace_bytes, stream, MOE_FFN_PATH_AUTO, nullptr);
}

int moe_ffn_forward_path(const moe_ffn_dims* dims, int64_t T, const uint16_t* x, const moe_ffn_router* router,
                         const moe_ffn_experts* experts, const moe_ffn_shared* shared, uint16_t* y,
                         int32_t* topk_idx, float* topk_weight, void* workspace, size_t workspace_bytes,
                         void* stream, int path) {
    return moe_ffn_forward_traced(dims, T, x, router, experts, shared, y, topk_idx, topk_weight, workspace,
                                  workspace_bytes, stream, path, nullptr);
}

int moe_ffn_forward(const moe_ffn_dims* dims, int64_t T, const uint16_t* x, const moe_ffn_router* router,
                    const moe_ffn_experts* experts, const moe_ffn_shared* shared, uint16_t* y, int32_t* topk_idx,
                    float* topk_weight, void* workspace, size_t workspace_bytes, void* stream) {
    return moe_ffn_forward_path(dims, T, x, router, experts, shared, y, topk_idx, topk_weight, workspace,
                                workspace_bytes, stream, MOE_FFN_PATH_AUTO);
}

const char* moe_ffn_status_string(int status) {
    switch (status) {
        case MOE_FFN_OK: return "ok";
        case MOE_FFN_EINVAL: return "invalid argument";
        case MOE_FFN_EUNSUPPORTED: return "unsupported shape, size or path";
        case MOE_FFN_EALIGN: return "pointer not 16-byte aligned";
        case MOE_FFN_EWORKSPACE: return "workspace missing or too small";
        case MOE_FFN_EHIP: return "HIP launch error";
        case MOE_FFN_ETOOBIG: return "token count above the no-allocation entry point's maximum";
        default: return "unknown status";
    }
}

}  // extern "C"
