"""ctypes binding of the fp64 CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU library never
imports or links this package.  Marshalling only; all arithmetic is in C.

Layer objects are duck-typed: anything with the attributes ``dims``
(d_model, n_experts, top_k, d_ff, d_ff_shared, group_size), ``router_w``,
``router_b``, ``gate``/``up``/``down`` (qweight, scales, biases),
``sh_gate_inp``, ``sh_gate``, ``sh_up``, ``sh_down`` (numpy arrays or None).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "moe_oracle.c")
LIB = os.path.join(_HERE, "libmoe_oracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB) -> str:
    subprocess.check_call(["gcc", *CFLAGS, "-I", _HERE, "-o", out, src, "-lm", "-lpthread"])
    return out


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("d_model", "n_experts", "top_k", "d_ff", "d_ff_shared", "group_size")]


class _Q4(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class _Layer(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("gate", _Q4), ("up", _Q4), ("down", _Q4),
                ("sh_gate_inp", ctypes.c_void_p), ("sh_gate", ctypes.c_void_p),
                ("sh_up", ctypes.c_void_p), ("sh_down", ctypes.c_void_p), ("weights_scale", ctypes.c_double),
                ("gating", ctypes.c_int32), ("tid2eid", ctypes.c_void_p), ("n_vocab", ctypes.c_int64),
                ("token_ids", ctypes.c_void_p)]


def _ptr(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "arrays must be C-contiguous numpy arrays"
    return a.ctypes.data


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


class Oracle:
    def __init__(self, lib_path: str = LIB):
        if not os.path.exists(lib_path):
            if lib_path != LIB:
                raise FileNotFoundError(lib_path)
            build()
        L = ctypes.CDLL(lib_path)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.moe_oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.moe_oracle_bf16_to_f32.restype = ctypes.c_float
        L.moe_oracle_dequant_row.argtypes = [ctypes.POINTER(_Q4), i64, i64, i64, i64, i64, vp]
        L.moe_oracle_dequant_row.restype = None
        L.moe_oracle_router_logits.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Layer), vp, vp]
        L.moe_oracle_router_logits.restype = None
        L.moe_oracle_select.argtypes = [vp, i64, i64, vp, vp, vp]
        L.moe_oracle_select.restype = ctypes.c_int
        L.moe_oracle_expert.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Layer), i64, vp, vp]
        L.moe_oracle_expert.restype = None
        L.moe_oracle_shared.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Layer), vp, vp, vp]
        L.moe_oracle_shared.restype = None
        L.moe_oracle_forward.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Layer), i64, vp, vp, i64,
                                         vp, vp, vp, vp, vp, ctypes.c_int]
        L.moe_oracle_forward.restype = ctypes.c_int
        L.moe_oracle_route.argtypes = L.moe_oracle_forward.argtypes[:6] + [vp, vp, vp, vp, ctypes.c_int]
        L.moe_oracle_rmsnorm_bf16.argtypes = [vp, vp, i64, ctypes.c_double, vp]
        L.moe_oracle_rmsnorm_bf16.restype = None
        L.moe_oracle_block_forward.argtypes = [ctypes.POINTER(_Dims), ctypes.POINTER(_Layer), i64, vp, vp,
                                               ctypes.c_double, vp, i64, vp, vp, vp, vp, vp, vp, ctypes.c_int]
        L.moe_oracle_route.restype = ctypes.c_int
        self.L = L
        self.path = lib_path

    # ----------------------------------------------------------- marshalling
    @staticmethod
    def _dims(d) -> _Dims:
        return _Dims(d.d_model, d.n_experts, d.top_k, d.d_ff, d.d_ff_shared, d.group_size)

    @staticmethod
    def _q4(q) -> _Q4:
        return _Q4(_ptr(q.qweight), _ptr(q.scales), _ptr(q.biases))

    def _layer(self, lay, token_ids=None) -> _Layer:
        """The layer struct; with a hash table (lay.tid2eid, int32 [k,
        n_vocab]) the call's token ids (int32 [T]) are required."""
        tab = getattr(lay, "tid2eid", None)
        if tab is not None:
            assert tab.dtype == np.int32 and tab.ndim == 2 and tab.shape[0] == lay.dims.top_k
            assert token_ids is not None and token_ids.dtype == np.int32, "hash routing needs the token ids"
        return _Layer(_ptr(lay.router_w), _ptr(lay.router_b), self._q4(lay.gate), self._q4(lay.up),
                      self._q4(lay.down), _ptr(lay.sh_gate_inp), _ptr(lay.sh_gate), _ptr(lay.sh_up),
                      _ptr(lay.sh_down), float(lay.weights_scale), int(lay.gating), _ptr(tab),
                      0 if tab is None else tab.shape[1], _ptr(token_ids) if tab is not None else None)

    # ----------------------------------------------------------------- steps
    def bf16_to_f32(self, bits: int) -> float:
        return self.L.moe_oracle_bf16_to_f32(bits)

    def dequant_row(self, q4, expert: int, out_dim: int, in_dim: int, group: int, row: int) -> np.ndarray:
        out = np.empty(in_dim, dtype=np.float32)
        q = self._q4(q4)
        self.L.moe_oracle_dequant_row(ctypes.byref(q), expert, out_dim, in_dim, group, row, out.ctypes.data)
        return out

    def router_logits(self, lay, x_row: np.ndarray) -> np.ndarray:
        x_row = np.ascontiguousarray(x_row, dtype=np.uint16)
        out = np.empty(lay.dims.n_experts, dtype=np.float64)
        d, l = self._dims(lay.dims), self._layer(lay)
        self.L.moe_oracle_router_logits(ctypes.byref(d), ctypes.byref(l), x_row.ctypes.data, out.ctypes.data)
        return out

    def select(self, logits: np.ndarray, k: int):
        lg = np.ascontiguousarray(logits, dtype=np.float64)
        sel = np.empty(k, dtype=np.int32)
        w = np.empty(k, dtype=np.float64)
        m = np.empty(1, dtype=np.float64)
        st = self.L.moe_oracle_select(lg.ctypes.data, lg.size, k, sel.ctypes.data, w.ctypes.data, m.ctypes.data)
        if st != 0:
            raise ValueError(f"moe_oracle_select failed: {st}")
        return sel, w, float(m[0])

    def expert(self, lay, e: int, xd: np.ndarray) -> np.ndarray:
        xd = np.ascontiguousarray(xd, dtype=np.float64)
        out = np.empty(lay.dims.d_model, dtype=np.float64)
        d, l = self._dims(lay.dims), self._layer(lay)
        self.L.moe_oracle_expert(ctypes.byref(d), ctypes.byref(l), e, xd.ctypes.data, out.ctypes.data)
        return out

    def shared(self, lay, xd: np.ndarray):
        xd = np.ascontiguousarray(xd, dtype=np.float64)
        out = np.empty(lay.dims.d_model, dtype=np.float64)
        sg = np.empty(1, dtype=np.float64)
        d, l = self._dims(lay.dims), self._layer(lay)
        self.L.moe_oracle_shared(ctypes.byref(d), ctypes.byref(l), xd.ctypes.data, out.ctypes.data,
                                 sg.ctypes.data)
        return out, float(sg[0])

    def forward(self, lay, x: np.ndarray, tokens=None, nthreads=None, want_logits=False, token_ids=None) -> dict:
        x = np.ascontiguousarray(x, dtype=np.uint16)
        T, D = x.shape
        assert D == lay.dims.d_model
        tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
        n = T if tok is None else tok.size
        k, E = lay.dims.top_k, lay.dims.n_experts
        y = np.empty((n, D), dtype=np.float64)
        idx = np.empty((n, k), dtype=np.int32)
        w = np.empty((n, k), dtype=np.float64)
        margin = np.empty(n, dtype=np.float64)
        logits = np.empty((n, E), dtype=np.float64) if want_logits else None
        tid = None if token_ids is None else np.ascontiguousarray(token_ids, dtype=np.int32)
        d, l = self._dims(lay.dims), self._layer(lay, tid)
        st = self.L.moe_oracle_forward(ctypes.byref(d), ctypes.byref(l), T, x.ctypes.data,
                                       None if tok is None else tok.ctypes.data, n, y.ctypes.data,
                                       idx.ctypes.data, w.ctypes.data, margin.ctypes.data,
                                       None if logits is None else logits.ctypes.data,
                                       nthreads or default_threads())
        if st != 0:
            raise ValueError(f"moe_oracle_forward failed: {st}")
        out = dict(y=y, idx=idx, w=w, margin=margin)
        if want_logits:
            out["logits"] = logits
        return out


    def rmsnorm_bf16(self, x_row: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
        """One row: bf16 bits -> bf16 bits of x / sqrt(mean(x^2) + eps) * weight."""
        x = np.ascontiguousarray(x_row, dtype=np.uint16)
        wv = np.ascontiguousarray(weight, dtype=np.float32)
        assert wv.shape == x.shape
        out = np.empty_like(x)
        self.L.moe_oracle_rmsnorm_bf16(x.ctypes.data, wv.ctypes.data, x.size, float(eps), out.ctypes.data)
        return out

    def block_forward(self, lay, h: np.ndarray, norm_w: np.ndarray, eps: float, tokens=None, nthreads=None,
                      want_logits=False, token_ids=None) -> dict:
        """y = h + FFN(RMSNorm(h) * norm_w) in double; also the bf16 rows xn."""
        h = np.ascontiguousarray(h, dtype=np.uint16)
        nw = np.ascontiguousarray(norm_w, dtype=np.float32)
        T, D = h.shape
        assert nw.shape == (D,)
        tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
        n = T if tok is None else tok.size
        k, E = lay.dims.top_k, lay.dims.n_experts
        xn = np.empty((T, D), dtype=np.uint16)
        y = np.empty((n, D), dtype=np.float64)
        idx = np.empty((n, k), dtype=np.int32)
        w = np.empty((n, k), dtype=np.float64)
        margin = np.empty(n, dtype=np.float64)
        logits = np.empty((n, E), dtype=np.float64) if want_logits else None
        tid = None if token_ids is None else np.ascontiguousarray(token_ids, dtype=np.int32)
        d, l = self._dims(lay.dims), self._layer(lay, tid)
        st = self.L.moe_oracle_block_forward(ctypes.byref(d), ctypes.byref(l), T, h.ctypes.data, nw.ctypes.data,
                                             float(eps), None if tok is None else tok.ctypes.data, n,
                                             xn.ctypes.data, y.ctypes.data, idx.ctypes.data, w.ctypes.data,
                                             margin.ctypes.data, None if logits is None else logits.ctypes.data,
                                             nthreads or default_threads())
        if st != 0:
            raise ValueError(f"moe_oracle_block_forward failed: {st}")
        out = dict(y=y, idx=idx, w=w, margin=margin, xn=xn)
        if want_logits:
            out["logits"] = logits
        return out

    def route(self, lay, x: np.ndarray, tokens=None, nthreads=None, want_logits=False, token_ids=None) -> dict:
        x = np.ascontiguousarray(x, dtype=np.uint16)
        T, D = x.shape
        tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
        n = T if tok is None else tok.size
        k, E = lay.dims.top_k, lay.dims.n_experts
        idx = np.empty((n, k), dtype=np.int32)
        w = np.empty((n, k), dtype=np.float64)
        margin = np.empty(n, dtype=np.float64)
        logits = np.empty((n, E), dtype=np.float64) if want_logits else None
        tid = None if token_ids is None else np.ascontiguousarray(token_ids, dtype=np.int32)
        d, l = self._dims(lay.dims), self._layer(lay, tid)
        st = self.L.moe_oracle_route(ctypes.byref(d), ctypes.byref(l), T, x.ctypes.data,
                                     None if tok is None else tok.ctypes.data, n, idx.ctypes.data, w.ctypes.data,
                                     margin.ctypes.data, None if logits is None else logits.ctypes.data,
                                     nthreads or default_threads())
        if st != 0:
            raise ValueError(f"moe_oracle_route failed: {st}")
        out = dict(idx=idx, w=w, margin=margin)
        if want_logits:
            out["logits"] = logits
        return out


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
