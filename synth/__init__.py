"""Seeded synthetic inputs for the sparse shared-expert MoE FFN.

A module of its own: it draws and encodes inputs (activations, fp32 router,
4-bit affine expert matrices, bf16 shared expert, Zipf router offsets) and
holds none of the FFN's arithmetic.  The fp64 oracle and the GPU library both
consume what it produces.  The C source (``moe_synth.c``) documents the
generator; this file is marshalling only.

Workload recipes follow the configurations the shared-expert MoE FFN is
measured on (n_embd 2048, 256 experts, top-8, FF 512, shared FF 512, 4-bit
affine group 64 with bf16 scales/biases, u32 [E, out, in/8] packing as on the
edge0 streaming page, "Quantized Layout").
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_synth.c")
_LIB = os.path.join(_HERE, "libmoe_synth.so")

# tensor ids of the counter-based streams
T_X, T_ROUTER, T_RBIAS, T_GATE, T_UP, T_DOWN, T_SH_GATE, T_SH_UP, T_SH_DOWN, T_SH_GATE_INP = range(1, 11)


def build_lib() -> str:
    cmd = ["gcc", "-O3", "-fno-math-errno", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra", "-o", _LIB, _SRC, "-lm", "-lpthread"]
    subprocess.check_call(cmd)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_lib()
        L = ctypes.CDLL(_LIB)
        u64, u32, i64, dbl, vp, i32 = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_double,
                                       ctypes.c_void_p, ctypes.c_int)
        L.synth_key.argtypes = [u64, u32, u32]
        L.synth_key.restype = u64
        L.synth_draw.argtypes = [u64, u64]
        L.synth_draw.restype = u64
        L.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        L.synth_f32_to_bf16.restype = ctypes.c_uint16
        L.synth_normal_bf16.argtypes = [u64, u32, u32, u64, i64, dbl, vp, i32]
        L.synth_normal_f32.argtypes = [u64, u32, u32, u64, i64, dbl, vp, i32]
        L.synth_x_rows.argtypes = [u64, u32, i64, i64, vp, dbl, vp, i32]
        L.synth_q4_matrix.argtypes = [u64, u32, i64, i64, i64, i64, dbl, vp, vp, vp, i32]
        L.synth_zipf_bias.argtypes = [u64, u32, i64, dbl, dbl, vp]
        for f in ("synth_normal_bf16", "synth_normal_f32", "synth_x_rows", "synth_q4_matrix", "synth_zipf_bias"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- primitives
def normal_bf16(seed: int, tensor: int, n: int, sd: float, stream: int = 0, start: int = 0, nthreads=None):
    out = np.empty(n, dtype=np.uint16)
    lib().synth_normal_bf16(seed, tensor, stream, start, n, sd, _p(out), nthreads or default_threads())
    return out


def normal_f32(seed: int, tensor: int, n: int, sd: float, stream: int = 0, start: int = 0, nthreads=None):
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(seed, tensor, stream, start, n, sd, _p(out), nthreads or default_threads())
    return out


def x_rows(seed: int, T: int, D: int, redraw: Optional[np.ndarray] = None, sd: float = 1.0, nthreads=None):
    x = np.empty((T, D), dtype=np.uint16)
    rd = None
    if redraw is not None:
        rd = np.ascontiguousarray(redraw, dtype=np.uint32)
        assert rd.shape == (T,)
    lib().synth_x_rows(seed, T_X, T, D, _p(rd) if rd is not None else None, sd, _p(x), nthreads or default_threads())
    return x


def q4_matrix(seed: int, tensor: int, nmat: int, rows: int, cols: int, group: int, sd: float, nthreads=None):
    assert cols % group == 0 and group % 8 == 0
    qw = np.empty((nmat, rows, cols // 8), dtype=np.uint32)
    sc = np.empty((nmat, rows, cols // group), dtype=np.uint16)
    bi = np.empty((nmat, rows, cols // group), dtype=np.uint16)
    lib().synth_q4_matrix(seed, tensor, nmat, rows, cols, group, sd, _p(qw), _p(sc), _p(bi),
                          nthreads or default_threads())
    return qw, sc, bi


def zipf_bias(seed: int, E: int, s: float, coef: float = 1.2):
    out = np.empty(E, dtype=np.float32)
    lib().synth_zipf_bias(seed, T_RBIAS, E, s, coef, _p(out))
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bits (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# ---------------------------------------------------------------- workloads
@dataclass
class Dims:
    d_model: int = 2048
    n_experts: int = 256
    top_k: int = 8
    d_ff: int = 512
    d_ff_shared: int = 512
    group_size: int = 64


@dataclass
class Q4:
    qweight: np.ndarray  # u32 [E, out, in/8]
    scales: np.ndarray   # bf16 bits [E, out, in/g]
    biases: np.ndarray   # bf16 bits [E, out, in/g]


@dataclass
class Layer:
    dims: Dims
    router_w: np.ndarray                 # f32 [E, D]
    router_b: Optional[np.ndarray]       # f32 [E] or None
    gate: Q4
    up: Q4
    down: Q4
    sh_gate_inp: Optional[np.ndarray]    # bf16 [D] or None
    sh_gate: Optional[np.ndarray]        # bf16 [Fs, D] or None (no shared expert)
    sh_up: Optional[np.ndarray]          # bf16 [Fs, D]
    sh_down: Optional[np.ndarray]        # bf16 [D, Fs]
    meta: dict = field(default_factory=dict)
    weights_scale: float = 1.0           # expert_weights_scale of the routed MoE call
    gating: int = 0                      # 0: softmax scores; 1: sqrt(softplus(logit)) scores
    tid2eid: Optional[np.ndarray] = None  # hash routing table int32 [top_k, n_vocab], or None


def make_layer(seed: int, dims: Dims = Dims(), *, w_sd: float = 0.02, zipf_s: Optional[float] = None,
               zipf_coef: float = 1.2, shared: bool = True, gate_inp: bool = True, nthreads=None) -> Layer:
    """Weights of one MoE FFN layer, all ~N(0, w_sd) before encoding.

    Router fp32; routed experts 4-bit affine; shared expert bf16; optional
    shared-expert gate vector bf16; optional Zipf router offsets."""
    D, E, F, Fs, g = dims.d_model, dims.n_experts, dims.d_ff, dims.d_ff_shared, dims.group_size
    nt = nthreads or default_threads()
    router_w = normal_f32(seed, T_ROUTER, E * D, w_sd, nthreads=nt).reshape(E, D)
    router_b = zipf_bias(seed, E, zipf_s, zipf_coef) if zipf_s is not None else None
    gate = Q4(*q4_matrix(seed, T_GATE, E, F, D, g, w_sd, nt))
    up = Q4(*q4_matrix(seed, T_UP, E, F, D, g, w_sd, nt))
    down = Q4(*q4_matrix(seed, T_DOWN, E, D, F, g, w_sd, nt))
    if shared:
        sh_gate = normal_bf16(seed, T_SH_GATE, Fs * D, w_sd, nthreads=nt).reshape(Fs, D)
        sh_up = normal_bf16(seed, T_SH_UP, Fs * D, w_sd, nthreads=nt).reshape(Fs, D)
        sh_down = normal_bf16(seed, T_SH_DOWN, D * Fs, w_sd, nthreads=nt).reshape(D, Fs)
        sgi = normal_bf16(seed, T_SH_GATE_INP, D, w_sd, nthreads=nt) if gate_inp else None
    else:
        sh_gate = sh_up = sh_down = sgi = None
    return Layer(dims, router_w, router_b, gate, up, down, sgi, sh_gate, sh_up, sh_down,
                 meta={"seed": seed, "w_sd": w_sd, "zipf_s": zipf_s, "zipf_coef": zipf_coef})


# The five measured configurations (T, router offsets).  Config 1 is 40
# independent layers with seeds 0..39 at T=1.
CONFIGS = {
    0: dict(name="layer_T4", T=4, layers=1, zipf_s=None),
    1: dict(name="decode_T1_40layers", T=1, layers=40, zipf_s=None),
    2: dict(name="decode_T64", T=64, layers=1, zipf_s=None),
    3: dict(name="prefill_T4096_zipf1.0", T=4096, layers=1, zipf_s=1.0),
    4: dict(name="prefill_T32768_zipf1.5_ties", T=32768, layers=1, zipf_s=1.5),
}
