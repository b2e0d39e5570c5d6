"""GPU parity on bf16-legal inputs of extreme magnitude, on every path.

The boundary's input contract is "finite inputs": nothing may overflow or
flush in an intermediate that the fp32/fp64 arithmetic of the method keeps.
Each case scales part of an ordinary seeded layer or activation by a power
of two far outside the fp16 range (or deep into its subnormals), so that a
path holding x, weights, h or the routed partials in plain fp16 would return
inf, NaN or zeros:

  x_outliers    three coordinates of every token at +-1e5 and every routed
                down scale and bias times 2^12: x > 65504, h = silu(g) u of
                order 1e6 .. 1e7, w * down(h) far above 1e3;
  x_tiny        x times 2^-40: x, h and y far below the fp16 subnormals;
  big_routed    routed scales and biases times 2^20 (dequantised weights
                above 65504), no shared expert;
  tiny_routed   routed scales and biases times 2^-30, no shared expert;
  big_shared    shared-expert matrices times 2^22;
  big_router    router weights times 2^24 (logits of order 1e7).

The bar is the parity bar with the routing margin and the routing-weight
tolerance taken relative to the logit scale of the token (fp32 logits carry
a relative, not an absolute, error, about 1e-6 of the largest |logit| here):
the oracle's top-8/top-9 margin is at least 1e-5 of the token's largest
|logit| (tokens are redrawn until it is), expert sets match exactly, the
order matches where every adjacent top-9 gap is at least 1e-5 of that scale, routing weights are within 1e-5 plus 2^-16
times the scale, and y is within relative L2 3e-3 per token.
"""
from __future__ import annotations

import copy
import functools
import sys

import numpy as np
import pytest

import oracle
import synth
import workloads
from gpu_common import GpuRunner, bf16_to_f64, output_check

pytestmark = pytest.mark.gpu

REL_MARGIN = 1e-5


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _scale_bf16(a, f):
    a[:] = synth.f32_to_bf16((synth.bf16_to_f32(a).astype(np.float64) * f).astype(np.float32))


def _outliers(x, rng, mag=1e5, n=3):
    x = x.copy()
    for t in range(x.shape[0]):
        cols = rng.choice(x.shape[1], size=n, replace=False)
        signs = rng.choice([-1.0, 1.0], size=n)
        x[t, cols] = synth.f32_to_bf16((signs * mag).astype(np.float32))
    return x


def _rel_margin(O, layer, x):
    r = O.route(layer, x, want_logits=True)
    scale = np.abs(r["logits"]).max(axis=1)
    return r["margin"] / np.maximum(scale, 1e-300)


@functools.lru_cache(maxsize=None)
def case_layer(name: str):
    """The case's layer (one per case, shared by its token counts)."""
    shared = name not in ("big_routed", "tiny_routed")
    layer = copy.deepcopy(workloads.layer_for(12, shared=shared))
    if name == "x_outliers":
        for arr in (layer.down.scales, layer.down.biases):
            _scale_bf16(arr, 2.0 ** 12)
    elif name in ("big_routed", "tiny_routed"):
        f = 2.0 ** 20 if name == "big_routed" else 2.0 ** -30
        for q in (layer.gate, layer.up, layer.down):
            _scale_bf16(q.scales, f)
            _scale_bf16(q.biases, f)
    elif name == "big_shared":
        for arr in (layer.sh_gate, layer.sh_up, layer.sh_down):
            _scale_bf16(arr, 2.0 ** 22)
    elif name == "big_router":
        layer.router_w = (layer.router_w.astype(np.float64) * 2.0 ** 24).astype(np.float32)
    return layer


def make_case(name: str, T: int):
    """(layer, x) of one case, every token with relative margin >= REL_MARGIN."""
    O = oracle.get()
    seed = 900 + T
    layer = case_layer(name)
    x, _, _ = workloads.enforce_margin(layer, T, seed, O=O)
    if name == "x_tiny":
        _scale_bf16(x, 2.0 ** -40)
    if name == "x_outliers":
        rng = np.random.default_rng(seed)
        x = _outliers(x, rng)
        for _ in range(32):
            bad = np.nonzero(_rel_margin(O, layer, x) < REL_MARGIN)[0]
            if bad.size == 0:
                break
            x[bad] = _outliers(x[bad], rng)
        else:
            raise RuntimeError("could not reach the relative routing margin")
    assert (_rel_margin(O, layer, x) >= REL_MARGIN).all()
    return layer, x


def routing_check_rel(layer, x, idx, w):
    r = oracle.get().route(layer, x, want_logits=True)
    lg = r["logits"]
    scale = np.abs(lg).max(axis=1)
    k = layer.dims.top_k
    top = -np.sort(-lg, axis=1)[:, : k + 1]
    unique_order = np.all(-np.diff(top, axis=1) >= REL_MARGIN * scale[:, None], axis=1)
    set_ok = np.array([set(a) == set(b) for a, b in zip(idx.tolist(), r["idx"].tolist())])
    assert set_ok.all(), f"expert sets differ on tokens {np.nonzero(~set_ok)[0][:10]}"
    order_ok = np.all(idx == r["idx"], axis=1)
    assert order_ok[unique_order].all(), "expert order differs"
    wo = np.zeros_like(w, dtype=np.float64)
    for n in range(x.shape[0]):
        pos = {int(e): j for j, e in enumerate(r["idx"][n])}
        wo[n] = [r["w"][n][pos[int(e)]] for e in idx[n]]
    err = np.abs(w.astype(np.float64) - wo)
    tol = 1e-5 + 2.0 ** -16 * scale[:, None]
    assert (err <= tol).all(), f"routing weight error {err.max()}"


CASES = ["x_outliers", "x_tiny", "big_routed", "tiny_routed", "big_shared", "big_router"]
# (T, path): the T <= 8 decode kernels (3 and 7 tokens), the 8 < T <= 64 decode kernels, the
# prefill path on a ragged tile and on several tiles
RUNS = [(3, 0), (7, 0), (37, 0), (37, 2), (300, 0)]


@pytest.fixture(scope="module")
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_ffn_fp32_amd as moe
    moe.lib()
    return GpuRunner(torch)


@pytest.mark.parametrize("T,path", RUNS, ids=[f"T{t}-{'prefill' if p == 2 else 'auto'}" for t, p in RUNS])
@pytest.mark.parametrize("case", CASES)
def test_extreme_magnitudes(gpu, case, T, path):
    layer, x = make_case(case, T)
    _say(f"range case {case} T={T} path={path}")
    y, idx, w = gpu.run(layer, x, path=path)
    assert np.isfinite(bf16_to_f64(y)).all(), "non-finite output"
    routing_check_rel(layer, x, idx, w)
    _say(output_check(layer, x, y))
