"""GPU tests of the layout and router variants.  The fused gate/up layout (SSD Streaming Expert Layers,
section Quantized Layout: gate and up of an expert stored as one tensor,
its gate rows on top of its up rows): bit-for-bit agreement with separate
tensors on every path, agreement with the oracle, and detection of the
whole-layer concatenation that mixes up the experts' rows.
expert_weights_scale: routing unchanged, weights and routed output scaled,
checked against the oracle of the scaled layer.  sqrt-softplus gating: the
same selection, weights and output against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth
import workloads
from gpu_common import GpuRunner, output_check, bf16_to_f64, Y_REL_L2

pytestmark = pytest.mark.gpu
PATHS = {"auto": 0, "decode": 1, "prefill": 2}


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
def fused0(gpu, layer0):
    import sparse_moe_ffn_fp32_amd as moe
    return moe.DeviceLayer.from_host(layer0, fused=True)


@pytest.mark.parametrize("T,path", [(1, "auto"), (3, "auto"), (4, "auto"), (6, "auto"), (37, "decode"), (64, "auto"),
                                    (37, "prefill"), (300, "auto")])
def test_fused_gate_up_equals_separate(gpu, layer0, fused0, T, path):
    x, _, _ = workloads.enforce_margin(layer0, T, 900 + T)
    _say(f"fused gate/up T={T} path={path}")
    a = gpu.run(layer0, x, path=PATHS[path])
    b = gpu.run(layer0, x, path=PATHS[path], dl=fused0)
    for u, v in zip(a, b):
        assert np.array_equal(u, v), "fused layout differs from separate tensors"
    _say(output_check(layer0, x, b[0]))


def test_fused_gate_up_large_tiles(gpu, layer0, fused0):
    """A pass of 16384 tokens (the gate/up and down kernels over some 1,100
    tiles): the same bit for bit (inputs without a routing margin: only the two layouts are
    compared)."""
    T = 16384
    x = synth.x_rows(55, T, 2048)
    _say(f"fused gate/up T={T}")
    a = gpu.run(layer0, x)
    b = gpu.run(layer0, x, dl=fused0)
    for u, v in zip(a, b):
        assert np.array_equal(u, v), "fused layout differs from separate tensors"


def test_whole_layer_concatenation_is_detected(gpu, layer0):
    """All experts' gate rows followed by all experts' up rows is not the
    fused layout: passed as one, expert e >= 1 reads other experts' rows and
    the output leaves the tolerance on (nearly) every token."""
    import sparse_moe_ffn_fp32_amd as moe
    torch = gpu.torch
    dl = moe.DeviceLayer.from_host(layer0)
    wrong = moe.DeviceLayer.from_host(layer0)
    wrong.gate = tuple(torch.cat([g.reshape(-1), u.reshape(-1)]) for g, u in zip(dl.gate, dl.up))
    wrong.up = (None, None, None)
    wrong.gate_up_fused = True
    T = 37
    x, _, _ = workloads.enforce_margin(layer0, T, 4242)
    y = gpu.run(layer0, x, dl=wrong)[0]
    ref = oracle.get().forward(layer0, x)["y"]
    rel = np.linalg.norm(bf16_to_f64(y) - ref, axis=1) / np.linalg.norm(ref, axis=1)
    _say(f"whole-layer concatenation: rel L2 min {rel.min():.3e}")
    assert np.mean(rel > 10 * Y_REL_L2) > 0.9


@pytest.mark.parametrize("T,path", [(1, "auto"), (4, "auto"), (37, "decode"), (37, "prefill"), (300, "auto")])
def test_weights_scale(gpu, layer0, T, path):
    """expert_weights_scale 2.5 (qwen35moe Forward-Pass Design, "Shared-expert
    MoE FFN"): the same experts, weights 2.5 times the unscaled ones, y
    against the oracle of the scaled layer; 0 gives the unscaled result bit
    for bit."""
    import copy
    import sparse_moe_ffn_fp32_amd as moe
    from gpu_common import W_ABS
    x, _, _ = workloads.enforce_margin(layer0, T, 700 + T)
    lay = copy.copy(layer0)
    lay.weights_scale = 2.5
    _say(f"weights_scale 2.5 T={T} path={path}")
    base = gpu.run(layer0, x, path=PATHS[path])
    got = gpu.run(lay, x, path=PATHS[path], dl=moe.DeviceLayer.from_host(lay))
    assert np.array_equal(got[1], base[1]), "the scale moved the routing"
    ref = oracle.get().forward(lay, x)
    assert np.array_equal(got[1], ref["idx"])
    assert np.abs(got[2].astype(np.float64) - ref["w"]).max() <= 2.5 * W_ABS
    _say(output_check(lay, x, got[0]))
    zero = copy.copy(layer0)
    zero.weights_scale = 0.0
    z = gpu.run(zero, x, path=PATHS[path], dl=moe.DeviceLayer.from_host(zero))
    for u, v in zip(z, base):
        assert np.array_equal(u, v), "weights_scale 0 must be the unscaled default"


@pytest.mark.parametrize("T,path,offset", [(1, "auto", 0.0), (4, "auto", 0.0), (37, "decode", 0.0),
                                           (37, "prefill", 0.0), (300, "auto", 0.0), (4, "auto", 25.0),
                                           (300, "auto", -25.0), (1, "auto", -150.0), (37, "decode", -150.0),
                                           (300, "auto", -600.0)])
def test_sqrt_softplus_gating(gpu, layer0, T, path, offset):
    """sqrt(softplus(logit)) scores (ds4.c study notes Part 3, MoE trace 3):
    the same experts as the softmax gate, weights and y against the oracle;
    a constant router-bias offset of +-25 moves every logit into the large
    and small softplus branches, offsets of -150 and -600 put every selected
    score below the fp32 (and, at -600, near the fp64) underflow."""
    import copy
    import sparse_moe_ffn_fp32_amd as moe
    from gpu_common import W_ABS
    lay = copy.copy(layer0)
    if offset:
        lay.router_b = np.full(layer0.dims.n_experts, offset, dtype=np.float32)
    x, _, _ = workloads.enforce_margin(lay, T, 600 + T)
    soft = copy.copy(lay)
    lay.gating = moe.GATING_SQRT_SOFTPLUS
    _say(f"sqrt-softplus gating T={T} path={path} offset={offset}")
    base = gpu.run(soft, x, path=PATHS[path], dl=moe.DeviceLayer.from_host(soft))
    got = gpu.run(lay, x, path=PATHS[path], dl=moe.DeviceLayer.from_host(lay))
    assert np.array_equal(got[1], base[1]), "the gating changed the selection"
    ref = oracle.get().forward(lay, x)
    assert np.array_equal(got[1], ref["idx"])
    assert np.abs(got[2].astype(np.float64) - ref["w"]).max() <= W_ABS
    _say(output_check(lay, x, got[0]))


def _hash_layer(base, n_vocab, seed, dup):
    """base with a seeded hash table [8, n_vocab] of experts (with dup, rank 1
    repeats rank 0's expert in every column)."""
    import copy
    lay = copy.copy(base)
    tab = np.random.default_rng(seed).integers(0, base.dims.n_experts, size=(base.dims.top_k, n_vocab))
    tab = tab.astype(np.int32)
    if dup:
        tab[1] = tab[0]
    lay.tid2eid = tab
    return lay


@pytest.mark.parametrize("T,path,gating,dup", [(1, "auto", 0, False), (4, "auto", 1, True), (8, "auto", 0, False),
                                               (37, "decode", 0, False),
                                               (37, "prefill", 1, False), (300, "auto", 0, True),
                                               (300, "auto", 1, False)])
def test_hash_routing(gpu, layer0, T, path, gating, dup):
    """Hash routing (ds4.c study notes Part 3, MoE trace 3): token t's experts
    are column token_ids[t] of the [8, n_vocab] table, exactly and in table
    order, on every path; the weights (the gating's scores of those experts,
    renormalised) and y against the oracle.  No routing margin is needed:
    the choice does not depend on the logits."""
    import sparse_moe_ffn_fp32_amd as moe
    from gpu_common import W_ABS
    lay = _hash_layer(layer0, 1000, 40 + T, dup)
    lay.gating = gating
    tid = np.random.default_rng(T).integers(0, 1000, size=T).astype(np.int32)
    x = synth.x_rows(700 + T, T, 2048)
    _say(f"hash routing T={T} path={path} gating={gating} dup={dup}")
    y, idx, w = gpu.run(lay, x, path=PATHS[path], dl=moe.DeviceLayer.from_host(lay), token_ids=tid)
    assert np.array_equal(idx, lay.tid2eid[:, tid].T), "experts differ from the table lookup"
    ref = oracle.get().forward(lay, x, token_ids=tid)
    assert np.abs(w.astype(np.float64) - ref["w"]).max() <= W_ABS
    _say(output_check(lay, x, y, token_ids=tid))
