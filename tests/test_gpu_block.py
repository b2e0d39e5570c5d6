"""GPU parity of the block entry point (y = h + FFN(RMSNorm(h) * w)) through
the C ABI against the fp64 oracle's block_forward, on seeded inputs whose
top-8/top-9 margin holds on the normalised rows."""
from __future__ import annotations

import copy
import sys

import numpy as np
import pytest

import oracle
import synth
import workloads
from gpu_common import GpuRunner, bf16_to_f64, Y_REL_L2, W_ABS

pytestmark = pytest.mark.gpu

EPS = float(np.float32(1e-6))  # the same value on both sides
D = 2048


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_ffn_fp32_amd as moe
    moe.lib()
    return GpuRunner(torch)


@pytest.fixture(scope="module")
def layer0():
    return workloads.layer_for(0)


@pytest.fixture(scope="module")
def norm_w():
    rng = np.random.default_rng(5)
    w = (1.0 + 0.2 * rng.standard_normal(D)).astype(np.float32)
    return synth.bf16_to_f32(synth.f32_to_bf16(w))  # values a bf16 checkpoint would hold


def block_inputs(layer, w, T, seed, O=None, sd=2.0, min_margin=workloads.MIN_MARGIN):
    """Residual rows h ~ N(0, sd^2) bf16 whose normalised rows keep the
    oracle's top-8/top-9 margin (tokens below it are redrawn)."""
    O = O or oracle.get()
    redraw = np.zeros(T, dtype=np.uint32)
    h = synth.x_rows(seed, T, D, redraw, sd=sd)
    for _ in range(64):
        xn = np.stack([O.rmsnorm_bf16(h[t], w, EPS) for t in range(T)])
        bad = np.nonzero(O.route(layer, xn)["margin"] < min_margin)[0]
        if bad.size == 0:
            return h
        redraw[bad] += 1
        h = synth.x_rows(seed, T, D, redraw, sd=sd)
    raise RuntimeError("could not enforce the routing margin")


def run_block(gpu, layer, h, w, path=0, in_place=False):
    import sparse_moe_ffn_fp32_amd as moe
    torch = gpu.torch
    T = h.shape[0]
    dl = gpu.device_layer(layer)
    hd = torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).cuda()
    wd = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).cuda()
    y = hd if in_place else torch.full((T, D), -1, dtype=torch.int16, device="cuda")
    idx = torch.full((T, 8), -1, dtype=torch.int32, device="cuda")
    wt = torch.full((T, 8), float("nan"), dtype=torch.float32, device="cuda")
    ws = moe.alloc_workspace(T, block=True)
    ws.fill_(0xFF)  # nothing may read unwritten workspace
    moe.moe_ffn_block_forward_traced(hd, wd, EPS, dl, y, ws, idx, wt, path=path)
    torch.cuda.synchronize()
    # the normalised rows of the (only) pass sit after the FFN's workspace
    off = (moe.moe_ffn_workspace_size(T) + 255) // 256 * 256
    xn = ws[off: off + T * D * 2].cpu().numpy().view(np.uint16).reshape(T, D).copy()
    return y.cpu().numpy().view(np.uint16).copy(), idx.cpu().numpy(), wt.cpu().numpy(), xn


def check(layer, h, w, y, idx, wt, xn, O=None):
    O = O or oracle.get()
    ref = O.block_forward(layer, h, w, EPS)
    # the normalised rows: computed in double on both sides and rounded once,
    # so equal unless a product lies within a few double ulps of a bf16
    # halfway point (then one bf16 ulp apart)
    diff = xn != ref["xn"]
    assert diff.sum() <= max(1, xn.size // 100000), f"{int(diff.sum())} normalised values differ"
    d = np.abs(xn[diff].astype(np.int32) - ref["xn"][diff].astype(np.int32))
    assert np.all(d <= 1)
    assert np.array_equal(idx, ref["idx"]), "experts differ from the oracle's"
    assert np.abs(wt.astype(np.float64) - ref["w"]).max() <= W_ABS
    got = bf16_to_f64(y)
    err = np.linalg.norm(got - ref["y"], axis=1) / np.linalg.norm(ref["y"], axis=1)
    assert err.max() <= Y_REL_L2, f"rel L2 {err.max():.3e} on token {int(err.argmax())}"
    return float(err.max())


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 8, 9, 37, 64, 300])
def test_block_forward(gpu, layer0, norm_w, T):
    h = block_inputs(layer0, norm_w, T, 400 + T)
    _say(f"block T={T}")
    y, idx, wt, xn = run_block(gpu, layer0, h, norm_w)
    _say("max rel L2", check(layer0, h, norm_w, y, idx, wt, xn))


@pytest.mark.parametrize("path", [1, 2])
def test_block_forced_paths(gpu, layer0, norm_w, path):
    h = block_inputs(layer0, norm_w, 37, 77)
    _say(f"block T=37 path={path}")
    y, idx, wt, xn = run_block(gpu, layer0, h, norm_w, path=path)
    check(layer0, h, norm_w, y, idx, wt, xn)


@pytest.mark.parametrize("T", [2, 5, 300])
def test_block_in_place(gpu, layer0, norm_w, T):
    """y written over h itself gives the out-of-place result, bit for bit."""
    h = block_inputs(layer0, norm_w, T, 90 + T)
    _say(f"block in place T={T}")
    a = run_block(gpu, layer0, h, norm_w)
    b = run_block(gpu, layer0, h, norm_w, in_place=True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("T", [1, 3, 100])
def test_block_zero_ffn_returns_h(gpu, norm_w, T):
    """Every routed scale and bias zero and no shared expert: the FFN is
    exactly 0, so y = h bit for bit on both paths."""
    lay = copy.deepcopy(workloads.layer_for(0))
    for q in (lay.gate, lay.up, lay.down):
        q.scales[:] = 0
        q.biases[:] = 0
    lay.sh_gate_inp = lay.sh_gate = lay.sh_up = lay.sh_down = None
    h = synth.x_rows(31, T, D, sd=2.0)
    _say(f"block zero FFN T={T}")
    y = run_block(gpu, lay, h, norm_w)[0]
    assert np.array_equal(y, h)
    ref = oracle.get().block_forward(lay, h, norm_w, EPS)["y"]  # h + 0, exact in fp64
    assert np.array_equal(bf16_to_f64(y), ref)


def test_block_prefill_in_slices(gpu, layer0, norm_w):
    """The block entry point over 32768 + 7 tokens runs in two slices inside
    one slice's workspace (each slice normalised into the same buffer, its
    residual rows offset): the result equals, bit for bit, two separate calls
    on the slices, and the oracle's block result on a sample that includes
    the slice boundary and the ragged tail."""
    import sparse_moe_ffn_fp32_amd as moe
    torch = gpu.torch
    chunk, tail = 32768, 7
    T = chunk + tail
    h = synth.x_rows(4242, T, D, sd=2.0)
    dl = gpu.device_layer(layer0)
    hd = torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).cuda()
    wd = torch.from_numpy(np.ascontiguousarray(norm_w, dtype=np.float32)).cuda()
    ws = moe.alloc_workspace(T, block=True)
    assert ws.numel() == moe.moe_ffn_block_workspace_size(chunk)

    def call(lo, hi):
        y = torch.empty((hi - lo, D), dtype=torch.int16, device="cuda")
        idx = torch.empty((hi - lo, 8), dtype=torch.int32, device="cuda")
        wt = torch.empty((hi - lo, 8), dtype=torch.float32, device="cuda")
        moe.moe_ffn_block_forward_traced(hd[lo:hi], wd, EPS, dl, y, ws, idx, wt, path=2)
        torch.cuda.synchronize()
        return y.cpu().numpy().view(np.uint16), idx.cpu().numpy(), wt.cpu().numpy()

    _say(f"block prefill in slices T={T}")
    whole = call(0, T)
    parts = [call(0, chunk), call(chunk, T)]
    for u, a, b in zip(whole, parts[0], parts[1]):
        assert np.array_equal(u, np.concatenate([a, b])), "sliced block pass differs from separate calls"
    sample = np.unique(np.concatenate([np.arange(0, T, 1024), np.arange(chunk - 4, T)]))
    ref = oracle.get().block_forward(layer0, h, norm_w, EPS, tokens=sample)
    ok = ref["margin"] >= workloads.MIN_MARGIN  # tokens whose experts are decided beyond rounding
    assert ok.sum() >= 0.9 * sample.size
    y, idx, wt = whole[0][sample], whole[1][sample], whole[2][sample]
    assert np.array_equal(idx[ok], ref["idx"][ok]), "experts differ from the oracle's"
    assert np.abs(wt[ok].astype(np.float64) - ref["w"][ok]).max() <= W_ABS
    got = bf16_to_f64(y[ok])
    err = np.linalg.norm(got - ref["y"][ok], axis=1) / np.linalg.norm(ref["y"][ok], axis=1)
    assert err.max() <= Y_REL_L2, f"rel L2 {err.max():.3e}"
    _say(f"{int(ok.sum())} of {sample.size} sampled tokens checked, max rel L2 {err.max():.3e}")
