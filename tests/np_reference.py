"""Independent numpy fp64 reference for tiny shapes (brute-force pin of the
oracle).  Written separately from the C oracle: vectorised numpy, library
matmul/argsort/exp, no shared helpers.

qwen35moe Forward-Pass Design (Pantheon port), "Shared-expert MoE FFN":
softmax router, top-k, norm_topk_prob, SwiGLU experts, sigmoid-gated shared
expert.  Packed layout: SSD Streaming Expert Layers (edge0), "Quantized
Layout".
"""
import numpy as np


def bf16(a):
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def dequant(q4, e, group):
    """[out, in] float32 matrix of expert e."""
    qw = q4.qweight[e]
    shifts = (4 * np.arange(8, dtype=np.uint32))[None, None, :]
    q = ((qw[:, :, None] >> shifts) & np.uint32(15)).reshape(qw.shape[0], -1).astype(np.float32)
    s = np.repeat(bf16(q4.scales[e]), group, axis=1)
    b = np.repeat(bf16(q4.biases[e]), group, axis=1)
    return (s * q + b).astype(np.float32)  # s*q exact in fp32, one rounding on +b


def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu(wg, wu, wd, xd):
    return wd @ (silu(wg @ xd) * (wu @ xd))


def forward(lay, x):
    d = lay.dims
    xd = bf16(x).astype(np.float64)                                   # [T, D]
    logits = xd @ lay.router_w.astype(np.float64).T
    if lay.router_b is not None:
        logits = logits + lay.router_b.astype(np.float64)[None, :]
    order = np.argsort(-logits, axis=1, kind="stable")
    sel = order[:, : d.top_k]
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    ps = np.take_along_axis(p, sel, axis=1)
    w = ps / ps.sum(axis=1, keepdims=True)
    mats = {}
    y = np.zeros_like(xd)
    for t in range(xd.shape[0]):
        for r in range(d.top_k):
            e = int(sel[t, r])
            if e not in mats:
                mats[e] = [dequant(q, e, d.group_size).astype(np.float64) for q in (lay.gate, lay.up, lay.down)]
            y[t] += w[t, r] * swiglu(*mats[e], xd[t])
    if lay.sh_gate is not None:
        wg, wu, wd = (bf16(m).astype(np.float64) for m in (lay.sh_gate, lay.sh_up, lay.sh_down))
        sg = np.ones(xd.shape[0])
        if lay.sh_gate_inp is not None:
            sg = 1.0 / (1.0 + np.exp(-(xd @ bf16(lay.sh_gate_inp).astype(np.float64))))
        for t in range(xd.shape[0]):
            y[t] += sg[t] * swiglu(wg, wu, wd, xd[t])
    return dict(y=y, idx=sel.astype(np.int32), w=w, logits=logits)
