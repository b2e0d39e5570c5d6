"""Helpers of the GPU parity tests: run the HIP library through its C ABI and
compare with the fp64 oracle to the parity bar.

Bar (per token): expert set bit-exact; expert order bit-exact where every
adjacent gap of the oracle's top-(k+1) logits is >= 1e-4; routing weights
within 1e-5; y within relative L2 3e-3 of the oracle (|y|_inf <= 1e-6 where
the oracle output is exactly 0).
"""
from __future__ import annotations

import numpy as np

import oracle
import sparse_moe_ffn_fp32_amd as moe

Y_REL_L2 = 3e-3
W_ABS = 1e-5
ORDER_GAP = 1e-4


def bf16_to_f64(a):
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class GpuRunner:
    def __init__(self, torch):
        self.torch = torch
        self.layers = {}

    def device_layer(self, layer):
        key = id(layer)
        if key not in self.layers:
            self.layers[key] = (layer, moe.DeviceLayer.from_host(layer))
        return self.layers[key][1]

    def run(self, layer, x: np.ndarray, path=moe.PATH_AUTO, dl=None, poison=False, T=None, token_ids=None):
        torch = self.torch
        dl = dl or self.device_layer(layer)
        T = x.shape[0] if T is None else T
        xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
        y = torch.full((max(T, 1), x.shape[1]), -1, dtype=torch.int16, device="cuda")
        idx = torch.full((max(T, 1), 8), -1, dtype=torch.int32, device="cuda")
        w = torch.full((max(T, 1), 8), float("nan"), dtype=torch.float32, device="cuda")
        ws = moe.alloc_workspace(max(T, 1))
        if poison:
            ws.fill_(0xFF)
        tid = None if token_ids is None else torch.from_numpy(np.ascontiguousarray(token_ids, dtype=np.int32)).cuda()
        moe.moe_ffn_forward_path(xd, dl, y, ws, idx, w, path=path, T=T, token_ids=tid)
        torch.cuda.synchronize()
        return (y.cpu().numpy().view(np.uint16)[:T], idx.cpu().numpy()[:T], w.cpu().numpy()[:T])


def routing_check(layer, x, idx_gpu, w_gpu, O=None, tokens=None, token_ids=None):
    """Compare routing on the listed tokens (all when None).  Returns stats."""
    O = O or oracle.get()
    tok = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    r = O.route(layer, x, tokens=tok, want_logits=True, token_ids=token_ids)
    k = layer.dims.top_k
    lg = r["logits"]
    top = -np.sort(-lg, axis=1)[:, : k + 1]
    unique_order = np.all(-np.diff(top, axis=1) >= ORDER_GAP, axis=1)
    if getattr(layer, "tid2eid", None) is not None:
        unique_order[:] = True  # a table's order does not depend on the logits
    gi, gw = idx_gpu[tok], w_gpu[tok]
    set_ok = np.array([set(a) == set(b) for a, b in zip(gi.tolist(), r["idx"].tolist())])
    assert set_ok.all(), f"expert sets differ on tokens {tok[~set_ok][:10]}"
    order_ok = np.all(gi == r["idx"], axis=1)
    assert order_ok[unique_order].all(), f"expert order differs on tokens {tok[unique_order & ~order_ok][:10]}"
    # weights, matched by expert id
    wo = np.zeros_like(gw, dtype=np.float64)
    for n in range(tok.size):
        pos = {int(e): j for j, e in enumerate(r["idx"][n])}
        wo[n] = [r["w"][n][pos[int(e)]] for e in gi[n]]
    werr = np.abs(gw.astype(np.float64) - wo).max()
    assert werr <= W_ABS, f"routing weight error {werr}"
    return dict(tokens=int(tok.size), unique_order=int(unique_order.sum()), w_err=float(werr))


def output_check(layer, x, y_gpu, O=None, tokens=None, nthreads=None, tol=Y_REL_L2, token_ids=None):
    O = O or oracle.get()
    tok = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    ref = O.forward(layer, x, tokens=tok, nthreads=nthreads, token_ids=token_ids)["y"]
    got = bf16_to_f64(y_gpu[tok])
    nrm = np.linalg.norm(ref, axis=1)
    err = np.linalg.norm(got - ref, axis=1)
    zero = nrm == 0
    rel = np.where(zero, 0.0, err / np.where(zero, 1.0, nrm))
    assert np.all(np.abs(got[zero]) <= 1e-6), "non-zero output where the oracle is exactly zero"
    worst = int(np.argmax(rel))
    assert rel.max() <= tol, f"token {tok[worst]}: rel L2 {rel.max():.3e} > {tol}"
    return dict(tokens=int(tok.size), rel_max=float(rel.max()), rel_mean=float(rel.mean()))
