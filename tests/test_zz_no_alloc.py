"""moe_ffn_forward_noalloc on the GPU through the C ABI.

The entry point that allocates nothing runs the decode path in the library's
static per-GPU scratch.  Its outputs (y, expert indices, routing weights)
must equal moe_ffn_forward's with a caller workspace bit for bit (the same
kernels run on the same inputs), on consecutive no-allocation calls whose
token counts fall, so that nothing a larger call left in the shared scratch
reaches a smaller one; the first call is also checked against the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads
from gpu_common import output_check, routing_check

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_noalloc_matches_workspace_entry_point():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_ffn_fp32_amd as moe

    layer = workloads.layer_for(0)
    dl = moe.DeviceLayer.from_host(layer)
    sizes = (64, 37, 8, 3)
    xs, refs = {}, {}

    def outputs(T):
        return (torch.full((T, 2048), -1, dtype=torch.int16, device="cuda"),
                torch.full((T, 8), -1, dtype=torch.int32, device="cuda"),
                torch.full((T, 8), float("nan"), dtype=torch.float32, device="cuda"))

    def host(o):
        return tuple(t.cpu().numpy().copy() for t in o)

    for T in sizes:
        x, _, _ = workloads.enforce_margin(layer, T, 500 + T)
        xs[T] = torch.from_numpy(x.view(np.int16)).cuda()
        o = outputs(T)
        moe.moe_ffn_forward(xs[T], dl, o[0], moe.alloc_workspace(T), o[1], o[2])
        torch.cuda.synchronize()
        refs[T] = host(o)
    # consecutive no-allocation calls, falling token counts
    got = {}
    for T in sizes:
        _say(f"noalloc T={T}")
        o = outputs(T)
        moe.moe_ffn_forward_noalloc(xs[T], dl, o[0], o[1], o[2])
        got[T] = o
    torch.cuda.synchronize()
    for T in sizes:
        g = host(got[T])
        for a, b, name in zip(g, refs[T], ("y", "topk_idx", "topk_weight")):
            assert np.array_equal(a, b), f"T={T}: {name} differs from moe_ffn_forward"
    x64 = xs[64].cpu().numpy().view(np.uint16)
    y64, i64, w64 = host(got[64])
    routing_check(layer, x64, i64, w64)
    _say(output_check(layer, x64, y64.view(np.uint16)))
    # above the maximum: a status, nothing launched
    big = torch.zeros((65, 2048), dtype=torch.int16, device="cuda")
    yb = torch.full((65, 2048), 7, dtype=torch.int16, device="cuda")
    st = moe.moe_ffn_forward_noalloc(big, dl, yb, check=False)
    torch.cuda.synchronize()
    assert st == moe.MOE_FFN_ETOOBIG and bool((yb == 7).all())
