"""Pins of the fp64 oracle against facts fixed outside it.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with the fact it checks.  ``test_oracle_pins.py`` runs them
on the real oracle; ``test_oracle_mutants.py`` runs them on copies of the
oracle with planted mistakes and requires that some pin fails for each.

The pages print no worked example for this path, so the pins are closed
forms, invariants, special cases that reduce to a library routine, and brute
force against an independent numpy reference on tiny shapes.
"""
from __future__ import annotations

import copy

import numpy as np

import synth
import np_reference as npr

TINY = synth.Dims(d_model=128, n_experts=16, top_k=4, d_ff=64, d_ff_shared=64, group_size=64)

_cache = {}


def tiny_layer(seed=11, **kw) -> synth.Layer:
    key = (seed, tuple(sorted(kw.items())))
    if key not in _cache:
        _cache[key] = synth.make_layer(seed, TINY, w_sd=0.05, nthreads=1, **kw)
    return copy.deepcopy(_cache[key])


def tiny_x(seed=3, T=6):
    return synth.x_rows(seed, T, TINY.d_model, nthreads=1)


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ----------------------------------------------------------------- bf16
def pin_bf16_exhaustive(O):
    """bf16 -> fp32 is the 16-bit left shift of the bit pattern, for all
    65,536 patterns (NaNs compared by bits)."""
    bits = np.arange(65536, dtype=np.uint32)
    want = (bits << 16).view(np.float32)
    # through the oracle's dequant with s=1 would lose NaN payloads; call directly
    got = np.array([O.bf16_to_f32(int(b)) for b in bits[::1]], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32)[~np.isnan(want)], want.view(np.uint32)[~np.isnan(want)])
    assert np.isnan(got[np.isnan(want)]).all()


# ----------------------------------------------------------------- dequant
def _q4_one_row(words, scales, biases):
    return synth.Q4(np.asarray(words, dtype=np.uint32).reshape(1, 1, -1),
                    np.asarray(scales, dtype=np.uint16).reshape(1, 1, -1),
                    np.asarray(biases, dtype=np.uint16).reshape(1, 1, -1))


def pin_dequant_handpacked(O):
    """Nibble k of word j is element 8j+k ("low first"); one bf16 scale and
    bias per group of 64.  Words 0x76543210, 0xFEDCBA98 give q = 0..15."""
    one, zero, half, m1, two, three = 0x3F80, 0x0000, 0x3F00, 0xBF80, 0x4000, 0x4040
    words = [0x76543210, 0xFEDCBA98] + [0] * 6 + [0x76543210, 0xFEDCBA98] + [0] * 6
    q = np.array(list(range(16)) + [0] * 48, dtype=np.float32)
    # group 0: (s, b) = (1, 0); group 1: (0.5, -1)
    got = O.dequant_row(_q4_one_row(words, [one, half], [zero, m1]), 0, 1, 128, 64, 0)
    assert np.array_equal(got[:64], q)
    assert np.array_equal(got[64:], 0.5 * q - 1.0)
    # group 0: (2, 3): W = 2q + 3
    got = O.dequant_row(_q4_one_row(words[:8], [two], [three]), 0, 1, 64, 64, 0)
    assert np.array_equal(got, 2.0 * q + 3.0)


def pin_dequant_quantizer_bound(O):
    """The generator's encoding decodes to within s/2 (plus the bf16 rounding
    of s and b) of the fp32 weights it encoded."""
    rows, cols, g = 4, 256, 64
    qw, sc, bi = synth.q4_matrix(5, 99, 1, rows, cols, g, 0.02, nthreads=1)
    w = synth.normal_f32(5, 99, rows * cols, 0.02, nthreads=1).reshape(rows, cols)
    q4 = synth.Q4(qw, sc, bi)
    s = np.repeat(synth.bf16_to_f32(sc[0]), g, axis=1)
    b = np.repeat(synth.bf16_to_f32(bi[0]), g, axis=1)
    mn = np.repeat(w.reshape(rows, -1, g).min(axis=2), g, axis=1)
    for r in range(rows):
        got = O.dequant_row(q4, 0, rows, cols, g, r)
        slack = 0.5 * s[r] + np.abs(b[r] - mn[r]) + 1e-7
        assert np.all(np.abs(got - w[r]) <= slack + 0.01 * s[r])


# ----------------------------------------------------------------- router
def pin_router_onehot(O):
    """x = e_j gives logits = Wr[:, j] (+ bias) exactly."""
    lay = tiny_layer(zipf_s=1.0)
    for j in (0, 5, 127):
        x = np.zeros(TINY.d_model, dtype=np.uint16)
        x[j] = 0x3F80  # 1.0
        got = O.router_logits(lay, x)
        want = lay.router_w[:, j].astype(np.float64) + lay.router_b.astype(np.float64)
        assert np.array_equal(got, want)


def pin_router_bruteforce(O):
    lay = tiny_layer(zipf_s=1.0)
    x = tiny_x()
    want = npr.bf16(x).astype(np.float64) @ lay.router_w.astype(np.float64).T + lay.router_b.astype(np.float64)
    for t in range(x.shape[0]):
        got = O.router_logits(lay, x[t])
        assert np.max(np.abs(got - want[t])) <= 1e-12 * np.max(np.abs(want[t]))


# ----------------------------------------------------------------- select
def pin_select_random(O):
    """Selected set and order equal a stable argsort of -logits; weights are
    the renormalised softmax; they sum to 1; margin is l(k) - l(k+1)."""
    rng = np.random.default_rng(7)
    for _ in range(50):
        E, k = 32, 8
        lg = rng.standard_normal(E)
        sel, w, m = O.select(lg, k)
        order = np.argsort(-lg, kind="stable")
        assert np.array_equal(sel, order[:k])
        p = np.exp(lg - lg.max())
        p /= p.sum()
        assert np.allclose(w, p[order[:k]] / p[order[:k]].sum(), rtol=1e-13, atol=0)
        assert abs(w.sum() - 1.0) <= 1e-15 * 4
        assert abs(m - (lg[order[k - 1]] - lg[order[k]])) <= 1e-15
        assert np.all(np.diff(w) <= 0)


def pin_select_ties(O):
    """Equal logits: lower index first, for membership and order; all-equal
    logits select 0..k-1 with weight exactly 1/k."""
    sel, w, m = O.select(np.zeros(256), 8)
    assert list(sel) == list(range(8)) and np.all(w == 0.125) and m == 0.0
    lg = np.array([0.0, 3.0, 1.0, 3.0, 2.0, 1.0, 2.0, -1.0])
    sel, w, m = O.select(lg, 4)
    assert list(sel) == [1, 3, 4, 6]
    sel, w, m = O.select(lg, 5)
    assert list(sel) == [1, 3, 4, 6, 2] and m == 0.0  # 2 beats 5 at logit 1.0


# ----------------------------------------------------------------- experts
def pin_identical_experts_dense(O):
    """When every expert holds the same bytes the routed sum is one dense
    SwiGLU (the weights sum to 1), computed here by numpy matmuls on the
    dequantised matrices."""
    lay = tiny_layer(shared=False)
    for q in (lay.gate, lay.up, lay.down):
        for a in (q.qweight, q.scales, q.biases):
            a[:] = a[2][None]
    x = tiny_x()
    r = O.forward(lay, x, nthreads=1)
    mats = [npr.dequant(q, 0, TINY.group_size).astype(np.float64) for q in (lay.gate, lay.up, lay.down)]
    for t in range(x.shape[0]):
        want = npr.swiglu(*mats, npr.bf16(x[t]).astype(np.float64))
        assert rel(r["y"][t], want) <= 1e-13


def pin_dominant_expert(O):
    """A router offset of +100 on expert e gives it weight 1 - O(e^-90), so
    the output is that expert's dense SwiGLU."""
    lay = tiny_layer(shared=False)
    lay.router_b = np.zeros(TINY.n_experts, dtype=np.float32)
    e = 9
    lay.router_b[e] = 100.0
    x = tiny_x()
    r = O.forward(lay, x, nthreads=1)
    mats = [npr.dequant(q, e, TINY.group_size).astype(np.float64) for q in (lay.gate, lay.up, lay.down)]
    assert np.all(r["idx"][:, 0] == e) and np.all(r["w"][:, 0] >= 1.0 - 1e-15)
    for t in range(x.shape[0]):
        want = npr.swiglu(*mats, npr.bf16(x[t]).astype(np.float64))
        assert rel(r["y"][t], want) <= 1e-13


def pin_expert_direct(O):
    """moe_oracle_expert equals the dense numpy SwiGLU of that expert."""
    lay = tiny_layer()
    xd = npr.bf16(tiny_x()[0]).astype(np.float64)
    for e in (0, 7, 15):
        mats = [npr.dequant(q, e, TINY.group_size).astype(np.float64) for q in (lay.gate, lay.up, lay.down)]
        assert rel(O.expert(lay, e, xd), npr.swiglu(*mats, xd)) <= 1e-13


# ----------------------------------------------------------------- shared / combine
def pin_shared_terms(O):
    """No shared expert => y = routed.  No gate vector => sgate = 1.  The
    shared expert equals the dense numpy SwiGLU of its bf16 matrices and
    sgate = sigmoid(w . x)."""
    lay = tiny_layer()
    x = tiny_x()
    full = O.forward(lay, x, nthreads=1)["y"]
    no_sh = copy.deepcopy(lay)
    no_sh.sh_gate = no_sh.sh_up = no_sh.sh_down = no_sh.sh_gate_inp = None
    routed = O.forward(no_sh, x, nthreads=1)["y"]
    no_gate = copy.deepcopy(lay)
    no_gate.sh_gate_inp = None
    ungated = O.forward(no_gate, x, nthreads=1)["y"]
    wg, wu, wd = (npr.bf16(m).astype(np.float64) for m in (lay.sh_gate, lay.sh_up, lay.sh_down))
    for t in range(x.shape[0]):
        xd = npr.bf16(x[t]).astype(np.float64)
        ys = npr.swiglu(wg, wu, wd, xd)
        sg = 1.0 / (1.0 + np.exp(-(npr.bf16(lay.sh_gate_inp).astype(np.float64) @ xd)))
        assert rel(ungated[t] - routed[t], ys) <= 1e-12
        assert rel(full[t] - routed[t], sg * ys) <= 1e-12
        out, s = O.shared(lay, xd)
        assert rel(out, ys) <= 1e-13 and abs(s - sg) <= 1e-15


def pin_zero_input(O):
    """x = 0 gives y = 0 exactly (silu(0) = 0), and uniform routing."""
    lay = tiny_layer()
    x = np.zeros((3, TINY.d_model), dtype=np.uint16)
    r = O.forward(lay, x, nthreads=1)
    assert np.all(r["y"] == 0.0)
    assert np.all(r["idx"] == np.arange(TINY.top_k)[None, :]) and np.all(r["w"] == 1.0 / TINY.top_k)


# ----------------------------------------------------------------- invariants
def pin_permutation_invariance(O):
    lay = tiny_layer(zipf_s=1.5)
    x = tiny_x(T=9)
    perm = np.array([4, 0, 8, 2, 7, 1, 3, 6, 5])
    a = O.forward(lay, x, nthreads=3)
    b = O.forward(lay, x[perm], nthreads=2)
    for key in ("y", "idx", "w", "margin"):
        assert np.array_equal(b[key], a[key][perm])
    c = O.forward(lay, x, tokens=perm, nthreads=1)
    for key in ("y", "idx", "w", "margin"):
        assert np.array_equal(c[key], a[key][perm])


def pin_down_halving(O):
    """Halving every down scale and bias (exact in bf16) halves the routed
    output exactly."""
    lay = tiny_layer(shared=False)
    x = tiny_x()
    a = O.forward(lay, x, nthreads=1)["y"]
    half = copy.deepcopy(lay)
    for arr in (half.down.scales, half.down.biases):
        f = synth.bf16_to_f32(arr) * np.float32(0.5)
        arr[:] = synth.f32_to_bf16(f)
        assert np.array_equal(synth.bf16_to_f32(arr), f)
    b = O.forward(half, x, nthreads=1)["y"]
    assert np.array_equal(b, 0.5 * a)


def pin_bruteforce_tiny(O):
    """Whole forward equals the independent numpy reference on tiny shapes,
    with and without router offsets, shared expert and shared gate."""
    x = tiny_x(T=7)
    for kw in (dict(), dict(zipf_s=1.0), dict(shared=False), dict(gate_inp=False)):
        lay = tiny_layer(**kw)
        got = O.forward(lay, x, nthreads=2)
        want = npr.forward(lay, x)
        assert np.array_equal(got["idx"], want["idx"])
        assert np.allclose(got["w"], want["w"], rtol=1e-13, atol=0)
        for t in range(x.shape[0]):
            assert rel(got["y"][t], want["y"][t]) <= 1e-12


def pin_gate_up_order(O):
    """Swapping gate and up changes the output completely (the math contract
    is silu(gate) * up, not silu(up) * gate)."""
    lay = tiny_layer()
    x = tiny_x()
    a = O.forward(lay, x, nthreads=1)["y"]
    sw = copy.deepcopy(lay)
    sw.gate, sw.up = sw.up, sw.gate
    b = O.forward(sw, x, nthreads=1)["y"]
    want = npr.forward(lay, x)["y"]
    assert all(rel(a[t], want[t]) <= 1e-12 for t in range(x.shape[0]))
    assert all(rel(b[t], a[t]) > 0.2 for t in range(x.shape[0]))


# ----------------------------------------------------------------- block boundary
def _bf(v: float) -> int:
    """bf16 bits of a value that bf16 holds exactly."""
    f = np.array([v], dtype=np.float32)
    b = int(f.view(np.uint32)[0])
    assert b & 0xFFFF == 0, v
    return b >> 16


def pin_rmsnorm_one_hot(O):
    """A one-hot row a*e_j of n = 64 values has mean(x^2) = a^2/64, so with
    eps = 0 the scale is 8/|a| and only entry j is non-zero: sign(a) * 8 *
    w_j, exact in bf16 for these weights; with eps = 3 and a = 8 the mean is
    1, sqrt(1 + 3) = 2 and the entry is 4 * w_j."""
    n = 64
    w = np.linspace(0.25, 2.0, n, dtype=np.float32) * np.float32(0.5)  # distinct, exact in bf16 x 8
    w = synth.bf16_to_f32(synth.f32_to_bf16(w))
    for j, a, eps, want in ((5, 3.0, 0.0, 8.0), (40, -0.75, 0.0, -8.0), (17, 8.0, 3.0, 4.0)):
        x = np.zeros(n, dtype=np.uint16)
        x[j] = _bf(a)
        out = O.rmsnorm_bf16(x, w, eps)
        assert np.count_nonzero(out) == 1, (j, a)
        assert out[j] == _bf(float(np.float32(want) * w[j])), (j, hex(out[j]))


def pin_rmsnorm_constant_row(O):
    """A constant row c: mean(x^2) = c^2.  eps = 0 gives sign(c) * w exactly;
    eps = 3c^2 gives sqrt(4c^2) = 2|c|, so sign(c) * w / 2 exactly."""
    n = 2048
    w = synth.bf16_to_f32(synth.f32_to_bf16(np.linspace(0.5, 1.5, n, dtype=np.float32)))
    for c in (2.0, -0.375, 1.5):
        x = np.full(n, _bf(c), dtype=np.uint16)
        out = synth.bf16_to_f32(O.rmsnorm_bf16(x, w, 0.0))
        assert np.array_equal(out, np.sign(c) * w), c
        out = synth.bf16_to_f32(O.rmsnorm_bf16(x, w, 3.0 * c * c))
        assert np.array_equal(out, np.sign(c) * w * np.float32(0.5)), c


def pin_rmsnorm_ties_to_even(O):
    """The normalised value is rounded once to bf16, halfway cases to even:
    one-hot rows of n = 64 (scale 8/a) with weights putting 8 * w exactly
    halfway between two bf16 values (1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6)."""
    n = 64
    for wv, want in ((1.0 + 2.0 ** -8, 1.0), (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6), (1.0 + 2.0 ** -9, 1.0)):
        w = np.full(n, np.float32(wv / 8.0), dtype=np.float32)
        assert float(w[0]) * 8.0 == wv
        x = np.zeros(n, dtype=np.uint16)
        x[9] = _bf(1.0)
        assert O.rmsnorm_bf16(x, w, 0.0)[9] == _bf(want), wv


def pin_rmsnorm_invariants(O):
    """With eps = 0 the normalisation ignores power-of-two scalings of the
    row (exact in binary) and is odd in x."""
    x = synth.x_rows(21, 1, 2048, nthreads=1)[0]
    w = synth.bf16_to_f32(synth.f32_to_bf16(np.linspace(0.8, 1.2, 2048, dtype=np.float32)))
    base = O.rmsnorm_bf16(x, w, 0.0)
    for k in (-3, 1, 4):
        xs = synth.f32_to_bf16(synth.bf16_to_f32(x) * np.float32(2.0 ** k))
        assert np.array_equal(O.rmsnorm_bf16(xs, w, 0.0), base), k
    neg = (x ^ np.uint16(0x8000)).astype(np.uint16)
    got = O.rmsnorm_bf16(neg, w, 0.0)
    nz = synth.bf16_to_f32(base) != 0
    assert np.array_equal(got[nz], (base ^ np.uint16(0x8000))[nz])


def pin_block_residual(O):
    """The block adds the un-normalised input: with every routed scale and
    bias zero and no shared expert the FFN is 0 and y = h exactly; in
    general the FFN part is the forward of the normalised rows."""
    lay = tiny_layer(shared=False)
    for arr in (lay.gate.scales, lay.gate.biases, lay.up.scales, lay.up.biases, lay.down.scales, lay.down.biases):
        arr[:] = 0
    h = tiny_x(seed=8, T=5)
    w = synth.bf16_to_f32(synth.f32_to_bf16(np.linspace(0.5, 1.5, TINY.d_model, dtype=np.float32)))
    r = O.block_forward(lay, h, w, 1e-6, nthreads=1)
    assert np.array_equal(r["y"], synth.bf16_to_f32(h).astype(np.float64))
    lay = tiny_layer()
    r = O.block_forward(lay, h, w, 1e-6, nthreads=2)
    for t in range(h.shape[0]):
        assert np.array_equal(r["xn"][t], O.rmsnorm_bf16(h[t], w, 1e-6))
    f = O.forward(lay, r["xn"], nthreads=1)
    assert np.array_equal(r["idx"], f["idx"]) and np.array_equal(r["w"], f["w"])
    ffn = r["y"] - synth.bf16_to_f32(h).astype(np.float64)
    for t in range(h.shape[0]):
        assert rel(ffn[t], f["y"][t]) <= 1e-12
    r2 = O.block_forward(lay, h, w, 1e-6, tokens=np.array([3, 0]), nthreads=1)
    assert np.array_equal(r2["y"], r["y"][[3, 0]])


def pin_weights_scale(O):
    """expert_weights_scale multiplies the renormalised weights and nothing
    else: the routing is unchanged, the reported weights are the unscaled
    ones times the factor, and without a shared expert a factor of 2 doubles
    y exactly (a power of two commutes with every rounding of the double
    sums); 0 stands for the unscaled default; with the shared expert only the
    routed part scales (factor 0.3, to double rounding)."""
    import copy
    lay = tiny_layer(shared=False)
    x = tiny_x(seed=12, T=6)
    base = O.forward(lay, x, nthreads=1)
    two = copy.copy(lay)
    two.weights_scale = 2.0
    r2 = O.forward(two, x, nthreads=1)
    assert np.array_equal(r2["idx"], base["idx"])
    assert np.array_equal(r2["w"], 2.0 * base["w"])
    assert np.array_equal(r2["y"], 2.0 * base["y"])
    assert np.array_equal(O.route(two, x)["w"], 2.0 * O.route(lay, x)["w"])
    zero = copy.copy(lay)
    zero.weights_scale = 0.0
    r0 = O.forward(zero, x, nthreads=1)
    assert np.array_equal(r0["y"], base["y"]) and np.array_equal(r0["w"], base["w"])
    sh = tiny_layer()
    no_routed = copy.deepcopy(sh)
    for arr in (no_routed.down.scales, no_routed.down.biases):
        arr[:] = 0
    shared_part = O.forward(no_routed, x, nthreads=1)["y"]
    s3 = copy.copy(sh)
    s3.weights_scale = 0.3
    a = O.forward(sh, x, nthreads=1)["y"] - shared_part
    b = O.forward(s3, x, nthreads=1)["y"] - shared_part
    for t in range(x.shape[0]):
        assert rel(b[t], 0.3 * a[t]) <= 1e-12


def pin_sqrt_softplus_gating(O):
    """sqrt(softplus) scores on logits set exactly through the router bias
    (zero router weights): for logits >= 100, softplus is the logit itself
    in double, so logits 6400, 1600, 400, 100 weigh 80:40:20:10 / 150; for
    logits <= -40 softplus is e^z to double precision, so logits -40 and -42
    weigh in the ratio e^1; the selection is the softmax gate's."""
    import copy
    lay = tiny_layer(shared=False)
    E, k = lay.dims.n_experts, lay.dims.top_k
    assert k == 4
    lay.router_w = np.zeros_like(lay.router_w)
    bias = np.full(E, -1000.0, dtype=np.float32)
    bias[[5, 2, 9, 0]] = [6400.0, 1600.0, 400.0, 100.0]
    lay.router_b = bias
    lay.gating = 1
    x = tiny_x(seed=4, T=3)
    r = O.route(lay, x)
    assert np.array_equal(r["idx"], np.tile([5, 2, 9, 0], (3, 1)))
    want = np.array([80.0, 40.0, 20.0, 10.0]) / 150.0
    assert np.abs(r["w"] - want).max() <= 1e-15
    bias = np.full(E, -1000.0, dtype=np.float32)
    bias[[1, 3, 6, 7]] = [-40.0, -42.0, -44.0, -46.0]
    lay.router_b = bias
    r = O.route(lay, x)
    assert np.array_equal(r["idx"], np.tile([1, 3, 6, 7], (3, 1)))
    w = r["w"][0]
    for a in range(3):
        assert abs(w[a] / w[a + 1] - np.e) <= 1e-12 * np.e
    soft = copy.copy(lay)
    soft.gating = 0
    lay2 = tiny_layer()
    lay2.gating = 1
    x2 = tiny_x(seed=9, T=5)
    assert np.array_equal(O.route(lay2, x2)["idx"], O.route(tiny_layer(), x2)["idx"])
    assert abs(O.forward(lay2, x2, nthreads=1)["w"].sum(axis=1) - 1.0).max() <= 1e-14


def pin_sqrt_softplus_extremes(O):
    """sqrt(softplus) scores where they are closed forms: a logit of 0 has
    softplus ln 2, logits <= -40 have softplus e^z (to double precision), so
    logits 0, -40, -42, -44 weigh sqrt(ln 2) e^20 : 1 : e^-1 : e^-2; and
    logits -1000, -1002, -1004, -1006 (every score far below the smallest
    double) still weigh 1 : e^-1 : e^-2 : e^-3, each normalised to sum 1."""
    lay = tiny_layer(shared=False)
    E = lay.dims.n_experts
    lay.router_w = np.zeros_like(lay.router_w)
    lay.gating = 1
    x = tiny_x(seed=5, T=2)
    bias = np.full(E, -5000.0, dtype=np.float32)
    bias[[4, 7, 1, 12]] = [0.0, -40.0, -42.0, -44.0]
    lay.router_b = bias
    r = O.route(lay, x)
    assert np.array_equal(r["idx"], np.tile([4, 7, 1, 12], (2, 1)))
    raw = np.array([np.sqrt(np.log(2.0)) * np.exp(20.0), 1.0, np.exp(-1.0), np.exp(-2.0)])
    assert np.abs(r["w"] - raw / raw.sum()).max() <= 1e-15
    bias = np.full(E, -5000.0, dtype=np.float32)
    bias[[3, 9, 0, 6]] = [-1000.0, -1002.0, -1004.0, -1006.0]
    lay.router_b = bias
    r = O.route(lay, x)
    assert np.array_equal(r["idx"], np.tile([3, 9, 0, 6], (2, 1)))
    raw = np.exp(-np.arange(4.0))
    assert np.isfinite(r["w"]).all() and np.abs(r["w"] - raw / raw.sum()).max() <= 1e-15


def _hash_table(k, n_vocab, E):
    """Column v of the table lists experts (3v + 5r + 1) mod E, r < k:
    distinct within a column for k <= 3 (and for r = 0..3 with E = 16)."""
    r = np.arange(k)[:, None]
    v = np.arange(n_vocab)[None, :]
    return ((3 * v + 5 * r + 1) % E).astype(np.int32)


def pin_hash_routing(O):
    """Hash routing (ds4.c notes Part 3, MoE trace 3): the experts of token t
    are column token_ids[t] of the [k, n_vocab] table, in table order, for
    any x; with zero router weights the logits are the bias exactly, so the
    softmax weights are e^b / sum e^b over the looked-up experts (a repeated
    expert gets its share once per rank), sqrt-softplus weights of logits
    >= 100 are sqrt(b) / sum sqrt(b), and expert_weights_scale multiplies
    them; the whole forward is sum_r w_r SwiGLU_e_r(x) from dense numpy."""
    import copy
    lay = tiny_layer(shared=False)
    E, k = lay.dims.n_experts, lay.dims.top_k
    nv = 10
    lay.tid2eid = _hash_table(k, nv, E)
    tid = np.array([0, 9, 3, 3, 7, 1], dtype=np.int32)
    x = tiny_x(seed=6, T=6)
    r = O.route(lay, x, token_ids=tid)
    want_idx = lay.tid2eid[:, tid].T
    assert np.array_equal(r["idx"], want_idx) and np.isinf(r["margin"]).all()
    assert np.array_equal(O.route(lay, tiny_x(seed=7, T=6), token_ids=tid)["idx"], want_idx)
    flat = copy.deepcopy(lay)
    flat.router_w = np.zeros_like(lay.router_w)
    flat.router_b = (np.arange(E) % 5).astype(np.float32)
    w = O.route(flat, x, token_ids=tid)["w"]
    eb = np.exp(flat.router_b.astype(np.float64)[want_idx])
    assert np.abs(w - eb / eb.sum(axis=1, keepdims=True)).max() <= 1e-15
    dup = copy.deepcopy(flat)
    dup.tid2eid = dup.tid2eid.copy()
    dup.tid2eid[1] = dup.tid2eid[0]  # rank 1 repeats rank 0's expert
    wd = O.route(dup, x, token_ids=tid)["w"]
    eb2 = np.exp(flat.router_b.astype(np.float64)[dup.tid2eid[:, tid].T])
    assert np.abs(wd - eb2 / eb2.sum(axis=1, keepdims=True)).max() <= 1e-15 and np.all(wd[:, 0] == wd[:, 1])
    sp = copy.deepcopy(flat)
    sp.router_b = (100.0 * (np.arange(E) + 1) ** 2).astype(np.float32)
    sp.gating = 1
    sp.weights_scale = 2.0
    ws = O.route(sp, x, token_ids=tid)["w"]
    sq = 10.0 * (want_idx + 1).astype(np.float64)
    assert np.abs(ws - 2.0 * sq / sq.sum(axis=1, keepdims=True)).max() <= 1e-14
    out = O.forward(flat, x, token_ids=tid, nthreads=1)
    g = flat.dims.group_size
    xd = npr.bf16(x).astype(np.float64)
    for t in range(x.shape[0]):
        y = np.zeros(flat.dims.d_model)
        for rr in range(k):
            e = int(want_idx[t, rr])
            y += out["w"][t, rr] * npr.swiglu(npr.dequant(flat.gate, e, g).astype(np.float64),
                                              npr.dequant(flat.up, e, g).astype(np.float64),
                                              npr.dequant(flat.down, e, g).astype(np.float64), xd[t])
        assert rel(out["y"][t], y) <= 1e-12


def pin_hash_table_validated(O):
    """Table entries outside [0, E) and token ids outside [0, n_vocab) are
    refused rather than read out of range."""
    lay = tiny_layer(shared=False)
    E, k = lay.dims.n_experts, lay.dims.top_k
    lay.tid2eid = _hash_table(k, 4, E)
    x = tiny_x(seed=6, T=2)
    for bad_ids in (np.array([0, 4], dtype=np.int32), np.array([-1, 0], dtype=np.int32)):
        try:
            O.route(lay, x, token_ids=bad_ids)
        except ValueError:
            pass
        else:
            raise AssertionError("out-of-range token id accepted")
    lay.tid2eid[2, 1] = E
    try:
        O.route(lay, x, token_ids=np.array([0, 1], dtype=np.int32))
    except ValueError:
        pass
    else:
        raise AssertionError("out-of-range table entry accepted")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
