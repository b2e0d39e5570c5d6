"""Python binding of libmoe_ffn.so, the MI355X (gfx950) sparse shared-expert
MoE FFN.

Marshalling only: every step of the FFN runs in the library's HIP kernels.
PyTorch provides device memory and streams.  The functions carry the C
entry points' names; see include/moe_ffn.h for the contract.  There is no
CPU fallback: if the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; MOE_FFN_LIB names another build of the same library
LIB_PATH = os.environ.get("MOE_FFN_LIB") or os.path.join(HERE, "libmoe_ffn.so")

MOE_FFN_OK = 0
MOE_FFN_EINVAL = -1
MOE_FFN_EUNSUPPORTED = -2
MOE_FFN_EALIGN = -3
MOE_FFN_EWORKSPACE = -4
MOE_FFN_EHIP = -5
MOE_FFN_ETOOBIG = -6
NOALLOC_MAX_T = 64
PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2
GATING_SOFTMAX, GATING_SQRT_SOFTPLUS = 0, 1
DECODE_MAX_T = 64

EXPORTED = ("moe_ffn_workspace_size", "moe_ffn_forward", "moe_ffn_forward_path", "moe_ffn_forward_traced",
            "moe_ffn_block_workspace_size", "moe_ffn_block_forward", "moe_ffn_block_forward_traced",
            "moe_ffn_forward_noalloc", "moe_ffn_status_string")
KERNEL_ROUTER, KERNEL_EXPERT_GU, KERNEL_EXPERT_DOWN, KERNEL_COMBINE = 1, 2, 3, 4


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("d_model", "n_experts", "top_k", "d_ff", "d_ff_shared", "group_size")]


DIMS = Dims(2048, 256, 8, 512, 512, 64)


class Q4Tensor(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class Experts(ctypes.Structure):
    _fields_ = [("gate", Q4Tensor), ("up", Q4Tensor), ("down", Q4Tensor), ("gate_up_fused", ctypes.c_int32)]


class Router(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("weights_scale", ctypes.c_float),
                ("gating", ctypes.c_int32), ("tid2eid", ctypes.c_void_p), ("token_ids", ctypes.c_void_p),
                ("n_vocab", ctypes.c_int32)]


class Shared(ctypes.Structure):
    _fields_ = [("gate_inp", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p),
                ("down", ctypes.c_void_p)]


class Trace(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("start", ctypes.c_void_p), ("stop", ctypes.c_void_p)]


class MoeFfnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def lib(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m sparse_moe_ffn_fp32_amd.build` "
                               "(or __graft_entry__.build())")
        L = ctypes.CDLL(path)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.moe_ffn_workspace_size.argtypes = [ctypes.POINTER(Dims), i64]
        L.moe_ffn_workspace_size.restype = ctypes.c_size_t
        fwd = [ctypes.POINTER(Dims), i64, vp, ctypes.POINTER(Router), ctypes.POINTER(Experts),
               ctypes.POINTER(Shared), vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_ffn_forward.argtypes = fwd
        L.moe_ffn_forward.restype = ctypes.c_int
        L.moe_ffn_forward_path.argtypes = fwd + [ctypes.c_int]
        L.moe_ffn_forward_path.restype = ctypes.c_int
        L.moe_ffn_forward_traced.argtypes = fwd + [ctypes.c_int, ctypes.POINTER(Trace)]
        L.moe_ffn_forward_traced.restype = ctypes.c_int
        L.moe_ffn_block_workspace_size.argtypes = [ctypes.POINTER(Dims), i64]
        L.moe_ffn_block_workspace_size.restype = ctypes.c_size_t
        blk = [ctypes.POINTER(Dims), i64, vp, vp, ctypes.c_float, ctypes.POINTER(Router), ctypes.POINTER(Experts),
               ctypes.POINTER(Shared), vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.moe_ffn_block_forward.argtypes = blk
        L.moe_ffn_block_forward.restype = ctypes.c_int
        L.moe_ffn_block_forward_traced.argtypes = blk + [ctypes.c_int, ctypes.POINTER(Trace)]
        L.moe_ffn_block_forward_traced.restype = ctypes.c_int
        L.moe_ffn_forward_noalloc.argtypes = fwd[:9] + [vp]
        L.moe_ffn_forward_noalloc.restype = ctypes.c_int
        L.moe_ffn_status_string.argtypes = [ctypes.c_int]
        L.moe_ffn_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _check(t, name: str, dtypes, rows: Optional[int] = None, cols: Optional[int] = None):
    """Refuse a torch tensor the kernels would misread: not on a GPU, not
    contiguous, of another element type, or too small for `rows` x `cols`.
    Objects that are not torch tensors (raw pointers) pass unchecked."""
    if t is None:
        return
    try:
        import torch
    except ImportError:  # pragma: no cover
        return
    if not isinstance(t, torch.Tensor):
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if rows is not None and cols is not None:
        if t.dim() != 2 or t.shape[0] < rows or t.shape[1] != cols:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected [>= {rows}, {cols}]")


def _check_call(x, y, topk_idx, topk_weight, T: int, dims):
    import torch
    _check(x, "x", (torch.int16, torch.uint16, torch.bfloat16), T, dims.d_model)
    _check(y, "y", (torch.int16, torch.uint16, torch.bfloat16), T, dims.d_model)
    _check(topk_idx, "topk_idx", (torch.int32,), T, dims.top_k)
    _check(topk_weight, "topk_weight", (torch.float32,), T, dims.top_k)


@dataclass
class DeviceLayer:
    """Device-resident weights of one layer (torch tensors; bf16 as int16 bits)."""
    router_w: object
    router_b: object
    gate: tuple
    up: tuple
    down: tuple
    sh_gate_inp: object
    sh_gate: object
    sh_up: object
    sh_down: object
    gate_up_fused: bool = False  # gate holds one [E, 2F, ...] tensor, up is empty
    weights_scale: float = 1.0   # expert_weights_scale (0 is read as 1)
    gating: int = 0              # GATING_SOFTMAX or GATING_SQRT_SOFTPLUS
    tid2eid: object = None       # hash routing table, int32 [top_k, n_vocab], or None

    @staticmethod
    def from_host(layer, device="cuda", fused: bool = False) -> "DeviceLayer":
        """fused: upload gate and up as one [E, 2F, ...] tensor, each
        expert's F gate rows followed by its F up rows."""
        import numpy as np
        import torch

        def t(a, dt):
            if a is None:
                return None
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)

        def q(q4):
            return (t(q4.qweight, np.int32), t(q4.scales, np.int16), t(q4.biases, np.int16))

        if fused:
            E = layer.dims.n_experts
            cat = lambda a, b: np.concatenate([a.reshape(E, -1), b.reshape(E, -1)], axis=1)
            gate = (t(cat(layer.gate.qweight, layer.up.qweight), np.int32),
                    t(cat(layer.gate.scales, layer.up.scales), np.int16),
                    t(cat(layer.gate.biases, layer.up.biases), np.int16))
            up = (None, None, None)
        else:
            gate, up = q(layer.gate), q(layer.up)
        return DeviceLayer(t(layer.router_w, np.float32), t(layer.router_b, np.float32), gate, up, q(layer.down),
                           t(layer.sh_gate_inp, np.int16), t(layer.sh_gate, np.int16), t(layer.sh_up, np.int16),
                           t(layer.sh_down, np.int16), fused, float(getattr(layer, "weights_scale", 1.0)),
                           int(getattr(layer, "gating", 0)), t(getattr(layer, "tid2eid", None), np.int32))

    def structs(self, token_ids=None):
        """The C structs; token_ids (int32 [T] on the GPU) are the call's,
        required with a hash table."""
        import torch
        f32, i32, i16 = (torch.float32,), (torch.int32,), (torch.int16, torch.uint16, torch.bfloat16)
        for name, t, dt in (("router_w", self.router_w, f32), ("router_b", self.router_b, f32),
                            ("sh_gate_inp", self.sh_gate_inp, i16), ("sh_gate", self.sh_gate, i16),
                            ("sh_up", self.sh_up, i16), ("sh_down", self.sh_down, i16)):
            _check(t, name, dt)
        for name, q in (("gate", self.gate), ("up", self.up), ("down", self.down)):
            for part, t, dt in zip(("qweight", "scales", "biases"), q, (i32, i16, i16)):
                _check(t, f"{name}.{part}", dt)
        _check(self.tid2eid, "tid2eid", i32)
        _check(token_ids, "token_ids", i32)
        if self.tid2eid is not None and token_ids is None:
            raise ValueError("hash routing needs the call's token_ids")
        n_vocab = int(self.tid2eid.shape[1]) if self.tid2eid is not None else 0
        r = Router(_ptr(self.router_w), _ptr(self.router_b), float(self.weights_scale), int(self.gating),
                   _ptr(self.tid2eid), _ptr(token_ids) if self.tid2eid is not None else None, n_vocab)
        ex = Experts(*(Q4Tensor(*(_ptr(a) for a in m)) for m in (self.gate, self.up, self.down)),
                     int(self.gate_up_fused))
        sh = None
        if self.sh_gate is not None:
            sh = Shared(_ptr(self.sh_gate_inp), _ptr(self.sh_gate), _ptr(self.sh_up), _ptr(self.sh_down))
        return r, ex, sh


def moe_ffn_status_string(status: int) -> str:
    return lib().moe_ffn_status_string(status).decode()


def moe_ffn_workspace_size(T: int, dims: Dims = DIMS) -> int:
    return int(lib().moe_ffn_workspace_size(ctypes.byref(dims), T))


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def moe_ffn_forward_path(x, layer: DeviceLayer, y, workspace, topk_idx=None, topk_weight=None, stream=None,
                         path: int = PATH_AUTO, dims: Dims = DIMS, T: Optional[int] = None,
                         workspace_bytes: Optional[int] = None, check: bool = True, token_ids=None) -> int:
    """Enqueue one FFN call on `stream` (default: torch's current stream).
    x, y: int16 tensors [T, d_model] holding bf16 bits.  Returns the status;
    raises MoeFfnError on a non-zero status when check is True."""
    r, ex, sh = layer.structs(token_ids)
    T = x.shape[0] if T is None else T
    _check_call(x, y, topk_idx, topk_weight, T, dims)
    wsb = (workspace.numel() * workspace.element_size()) if workspace is not None else 0
    if workspace_bytes is not None:
        wsb = workspace_bytes
    st = lib().moe_ffn_forward_path(ctypes.byref(dims), T, _ptr(x), ctypes.byref(r), ctypes.byref(ex),
                                    ctypes.byref(sh) if sh is not None else None, _ptr(y), _ptr(topk_idx),
                                    _ptr(topk_weight), _ptr(workspace), wsb, _stream_ptr(stream), path)
    if check and st != MOE_FFN_OK:
        raise MoeFfnError(st, moe_ffn_status_string(st))
    return st


def moe_ffn_forward_traced(x, layer: DeviceLayer, y, workspace, topk_idx=None, topk_weight=None, stream=None,
                           path: int = PATH_AUTO, trace: Optional[Trace] = None, dims: Dims = DIMS,
                           T: Optional[int] = None, check: bool = True, token_ids=None) -> int:
    """moe_ffn_forward_path plus an optional Trace (kernel id and two
    hipEvent_t handles as integers) bracketing one kernel of the call."""
    r, ex, sh = layer.structs(token_ids)
    T = x.shape[0] if T is None else T
    _check_call(x, y, topk_idx, topk_weight, T, dims)
    wsb = (workspace.numel() * workspace.element_size()) if workspace is not None else 0
    st = lib().moe_ffn_forward_traced(ctypes.byref(dims), T, _ptr(x), ctypes.byref(r), ctypes.byref(ex),
                                      ctypes.byref(sh) if sh is not None else None, _ptr(y), _ptr(topk_idx),
                                      _ptr(topk_weight), _ptr(workspace), wsb, _stream_ptr(stream), path,
                                      ctypes.byref(trace) if trace is not None else None)
    if check and st != MOE_FFN_OK:
        raise MoeFfnError(st, moe_ffn_status_string(st))
    return st


def moe_ffn_forward(x, layer: DeviceLayer, y, workspace, topk_idx=None, topk_weight=None, stream=None,
                    **kw) -> int:
    return moe_ffn_forward_path(x, layer, y, workspace, topk_idx, topk_weight, stream, PATH_AUTO, **kw)


def alloc_workspace(T: int, device="cuda", block: bool = False):
    """A workspace for calls with up to T tokens (uninitialised memory); with
    block=True, for the block entry point (moe_ffn_block_forward*)."""
    import torch
    n = moe_ffn_block_workspace_size(T) if block else moe_ffn_workspace_size(T)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_ffn_block_workspace_size(T: int, dims: Dims = DIMS) -> int:
    return int(lib().moe_ffn_block_workspace_size(ctypes.byref(dims), T))


def moe_ffn_block_forward_traced(h, norm_weight, eps: float, layer: DeviceLayer, y, workspace, topk_idx=None,
                                 topk_weight=None, stream=None, path: int = PATH_AUTO, trace: Optional[Trace] = None,
                                 dims: Dims = DIMS, T: Optional[int] = None, check: bool = True, token_ids=None) -> int:
    """y = h + FFN(RMSNorm(h) * norm_weight) (moe_ffn_block_forward_traced):
    h, y bf16 bits [T, D] (y may be h), norm_weight fp32 [D]."""
    r, ex, sh = layer.structs(token_ids)
    T = h.shape[0] if T is None else T
    _check_call(h, y, topk_idx, topk_weight, T, dims)
    _check(norm_weight, "norm_weight", (__import__("torch").float32,))
    wsb = (workspace.numel() * workspace.element_size()) if workspace is not None else 0
    st = lib().moe_ffn_block_forward_traced(ctypes.byref(dims), T, _ptr(h), _ptr(norm_weight), float(eps),
                                            ctypes.byref(r), ctypes.byref(ex),
                                            ctypes.byref(sh) if sh is not None else None, _ptr(y), _ptr(topk_idx),
                                            _ptr(topk_weight), _ptr(workspace), wsb, _stream_ptr(stream), path,
                                            ctypes.byref(trace) if trace is not None else None)
    if check and st != MOE_FFN_OK:
        raise MoeFfnError(st, moe_ffn_status_string(st))
    return st


def moe_ffn_block_forward(h, norm_weight, eps: float, layer: DeviceLayer, y, workspace, topk_idx=None,
                          topk_weight=None, stream=None, dims: Dims = DIMS, T: Optional[int] = None,
                          check: bool = True, token_ids=None) -> int:
    """moe_ffn_block_forward: the FFN sub-block with its boundary steps."""
    r, ex, sh = layer.structs(token_ids)
    T = h.shape[0] if T is None else T
    _check_call(h, y, topk_idx, topk_weight, T, dims)
    _check(norm_weight, "norm_weight", (__import__("torch").float32,))
    wsb = (workspace.numel() * workspace.element_size()) if workspace is not None else 0
    st = lib().moe_ffn_block_forward(ctypes.byref(dims), T, _ptr(h), _ptr(norm_weight), float(eps), ctypes.byref(r),
                                     ctypes.byref(ex), ctypes.byref(sh) if sh is not None else None, _ptr(y),
                                     _ptr(topk_idx), _ptr(topk_weight), _ptr(workspace), wsb, _stream_ptr(stream))
    if check and st != MOE_FFN_OK:
        raise MoeFfnError(st, moe_ffn_status_string(st))
    return st


def moe_ffn_forward_noalloc(x, layer: DeviceLayer, y, topk_idx=None, topk_weight=None, stream=None,
                            dims: Dims = DIMS, T: Optional[int] = None, check: bool = True, token_ids=None) -> int:
    """moe_ffn_forward_noalloc: T <= NOALLOC_MAX_T tokens with the library's
    own static device scratch (no workspace, no allocation anywhere)."""
    r, ex, sh = layer.structs(token_ids)
    T = x.shape[0] if T is None else T
    _check_call(x, y, topk_idx, topk_weight, T, dims)
    st = lib().moe_ffn_forward_noalloc(ctypes.byref(dims), T, _ptr(x), ctypes.byref(r), ctypes.byref(ex),
                                       ctypes.byref(sh) if sh is not None else None, _ptr(y), _ptr(topk_idx),
                                       _ptr(topk_weight), _stream_ptr(stream))
    if check and st != MOE_FFN_OK:
        raise MoeFfnError(st, moe_ffn_status_string(st))
    return st
