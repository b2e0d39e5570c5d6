"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, sizes workspaces, and rejects bad arguments before any
launch (no GPU needed: every call here returns from validation)."""
import ctypes
import os
import re

import pytest

import sparse_moe_ffn_fp32_amd as moe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_ffn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from sparse_moe_ffn_fp32_amd import build
        build.build()
    return moe.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_ffn_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(moe.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert moe.moe_ffn_status_string(st)
    assert moe.moe_ffn_status_string(-99) == "unknown status"


def test_workspace_size(L):
    assert moe.moe_ffn_workspace_size(0) == 0
    assert moe.moe_ffn_workspace_size(-1) == 0
    a, b = moe.moe_ffn_workspace_size(1), moe.moe_ffn_workspace_size(4096)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0
    bad = moe.Dims(2048, 128, 8, 512, 512, 64)
    assert L.moe_ffn_workspace_size(ctypes.byref(bad), 4) == 0


class _Fake:
    """Device pointers that are never dereferenced (validation fails first)."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr

    numel = staticmethod(lambda: 1 << 40)
    element_size = staticmethod(lambda: 1)


def _layer(base=0x10000000):
    f = lambda i: _Fake(base + 0x1000 * i)
    return moe.DeviceLayer(f(1), None, (f(2), f(3), f(4)), (f(5), f(6), f(7)), (f(8), f(9), f(10)), f(11),
                           f(12), f(13), f(14))


def _call(L, T=4, x=0x20000000, y=0x30000000, ws=0x40000000, wsb=None, layer=None, dims=moe.DIMS, path=0,
          idx=None, w=None):
    layer = layer or _layer()
    r, ex, sh = layer.structs()
    wsb = moe.moe_ffn_workspace_size(max(T, 1)) if wsb is None else wsb
    return L.moe_ffn_forward_path(ctypes.byref(dims), T, x, ctypes.byref(r), ctypes.byref(ex), ctypes.byref(sh),
                                  y, idx, w, ws, wsb, None, path)


def test_rejects_bad_arguments(L):
    assert _call(L, T=0) == moe.MOE_FFN_OK  # no launch for T == 0
    assert _call(L, T=-1) == moe.MOE_FFN_EINVAL
    assert _call(L, x=None) == moe.MOE_FFN_EINVAL
    assert _call(L, y=None) == moe.MOE_FFN_EINVAL
    assert _call(L, path=7) == moe.MOE_FFN_EINVAL
    assert _call(L, dims=moe.Dims(2048, 256, 8, 512, 512, 32)) == moe.MOE_FFN_EUNSUPPORTED
    assert _call(L, T=(1 << 20) + 1) == moe.MOE_FFN_EUNSUPPORTED
    assert _call(L, x=0x20000008) == moe.MOE_FFN_EALIGN
    assert _call(L, idx=0x50000004) == moe.MOE_FFN_EALIGN
    assert _call(L, ws=None) == moe.MOE_FFN_EWORKSPACE
    assert _call(L, wsb=1024) == moe.MOE_FFN_EWORKSPACE
    lay = _layer()
    lay.up = (lay.up[0], None, lay.up[2])
    assert _call(L, layer=lay) == moe.MOE_FFN_EINVAL
    lay = _layer()
    lay.sh_down = None
    assert _call(L, layer=lay) == moe.MOE_FFN_EINVAL
    lay = _layer()
    lay.down = (_Fake(0x60000002), lay.down[1], lay.down[2])
    assert _call(L, layer=lay) == moe.MOE_FFN_EALIGN
    assert L.moe_ffn_forward_path(None, 4, 1, None, None, None, 1, None, None, 1, 1, None, 0) == moe.MOE_FFN_EINVAL



def test_fused_gate_up_arguments(L):
    """The fused gate/up layout: one tensor in gate, up all NULL; accepted
    layouts get as far as the workspace check (no launch here)."""
    fused = _layer()
    fused.up = (None, None, None)
    fused.gate_up_fused = True
    assert _call(L, layer=fused, ws=None) == moe.MOE_FFN_EWORKSPACE
    both = _layer()
    both.gate_up_fused = True  # up given as well
    assert _call(L, layer=both) == moe.MOE_FFN_EINVAL
    bad = _layer()
    bad.up = (None, None, None)
    bad.gate_up_fused = 2
    assert _call(L, layer=bad) == moe.MOE_FFN_EINVAL
    lay = _layer()
    lay.up = (None, None, None)
    lay.gate_up_fused = True
    lay.gate = (lay.gate[0], None, lay.gate[2])
    assert _call(L, layer=lay) == moe.MOE_FFN_EINVAL
    lay = _layer()
    lay.up = (None, None, None)
    lay.gate_up_fused = True
    lay.gate = (_Fake(0x60000008), lay.gate[1], lay.gate[2])
    assert _call(L, layer=lay) == moe.MOE_FFN_EALIGN
    sep = _layer()
    sep.up = (None, None, None)  # separate layout without up
    assert _call(L, layer=sep) == moe.MOE_FFN_EINVAL


def test_weights_scale_arguments(L):
    """expert_weights_scale: finite and >= 0 (0 = unscaled); anything else is
    rejected before any launch."""
    for bad in (-1.0, float("nan"), float("inf"), -float("inf")):
        lay = _layer()
        lay.weights_scale = bad
        assert _call(L, layer=lay) == moe.MOE_FFN_EINVAL, bad
    for ok in (0.0, 1.0, 2.5):
        lay = _layer()
        lay.weights_scale = ok
        assert _call(L, layer=lay, ws=None) == moe.MOE_FFN_EWORKSPACE, ok


def test_gating_arguments(L):
    for g, want in ((0, moe.MOE_FFN_EWORKSPACE), (1, moe.MOE_FFN_EWORKSPACE), (2, moe.MOE_FFN_EINVAL),
                    (-1, moe.MOE_FFN_EINVAL)):
        lay = _layer()
        lay.gating = g
        assert _call(L, layer=lay, ws=None) == want, g


def _block(L, T=4, h=0x20000000, nw=0x21000000, eps=1e-6, y=0x30000000, ws=0x40000000, wsb=None, path=0,
           layer=None):
    layer = layer or _layer()
    r, ex, sh = layer.structs()
    wsb = moe.moe_ffn_block_workspace_size(max(T, 1)) if wsb is None else wsb
    return L.moe_ffn_block_forward_traced(ctypes.byref(moe.DIMS), T, h, nw, eps, ctypes.byref(r), ctypes.byref(ex),
                                          ctypes.byref(sh), y, None, None, ws, wsb, None, path, None)


def test_block_entry_point_rejects_bad_arguments(L):
    """The block entry point: the FFN's checks, then the norm weight and eps,
    then its larger workspace (the FFN's size alone is not enough)."""
    assert _block(L, T=0) == moe.MOE_FFN_OK
    assert _block(L, T=-1) == moe.MOE_FFN_EINVAL
    assert _block(L, h=None) == moe.MOE_FFN_EINVAL
    assert _block(L, nw=None) == moe.MOE_FFN_EINVAL
    assert _block(L, eps=-1e-6) == moe.MOE_FFN_EINVAL
    assert _block(L, eps=float("nan")) == moe.MOE_FFN_EINVAL
    assert _block(L, eps=float("inf")) == moe.MOE_FFN_EINVAL
    assert _block(L, nw=0x21000004) == moe.MOE_FFN_EALIGN
    assert _block(L, h=0x20000002) == moe.MOE_FFN_EALIGN
    assert _block(L, ws=None) == moe.MOE_FFN_EWORKSPACE
    assert _block(L, wsb=moe.moe_ffn_workspace_size(4)) == moe.MOE_FFN_EWORKSPACE
    assert _block(L, path=9) == moe.MOE_FFN_EINVAL
    for T in (1, 64, 65, 4096, 32768, 100000):
        b, f = moe.moe_ffn_block_workspace_size(T), moe.moe_ffn_workspace_size(T)
        assert b >= f + min(T, 32768) * 2048 * 2 and b % 256 == 0
    assert moe.moe_ffn_block_workspace_size(40000) == moe.moe_ffn_block_workspace_size(32768)
    assert moe.moe_ffn_block_workspace_size(0) == 0


def test_workspace_is_bounded_by_the_prefill_slice(L):
    """Prefill runs in passes of at most MOE_FFN_PREFILL_CHUNK_T tokens, so
    the workspace stops growing there (and is never smaller than a pass
    needs)."""
    chunk = 32768
    w = moe.moe_ffn_workspace_size(chunk)
    assert moe.moe_ffn_workspace_size(chunk + 1) == w
    assert moe.moe_ffn_workspace_size(1 << 20) == w
    assert moe.moe_ffn_workspace_size(chunk - 1) < w
    assert "#define MOE_FFN_PREFILL_CHUNK_T 32768" in open(HEADER).read()


def test_binding_refuses_misshapen_tensors(L):
    """The binding checks torch tensors before any call: a host tensor, a
    strided view, another dtype or too few rows never reach the library."""
    torch = pytest.importorskip("torch")
    lay = _layer()
    y = _Fake(0x30000000)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.moe_ffn_forward(torch.zeros((4, 2048), dtype=torch.int16), lay, y, None)
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.moe_ffn_forward_noalloc(torch.zeros((4, 2048), dtype=torch.int16), lay, y)
    bad = _layer()
    bad.router_w = torch.zeros((256, 2048), dtype=torch.float32)
    with pytest.raises(ValueError, match="router_w"):
        moe.moe_ffn_forward(_Fake(0x20000000), bad, y, None, T=4)


def test_noalloc_rejects_before_launch(L):
    """moe_ffn_forward_noalloc: T above its maximum is MOE_FFN_ETOOBIG, bad
    arguments get moe_ffn_forward's statuses, T == 0 launches nothing."""
    layer = _layer()
    r, ex, sh = layer.structs()

    def call(T, x=0x20000000, y=0x30000000, dims=moe.DIMS):
        return L.moe_ffn_forward_noalloc(ctypes.byref(dims), T, x, ctypes.byref(r), ctypes.byref(ex),
                                         ctypes.byref(sh), y, None, None, None)

    assert call(0) == moe.MOE_FFN_OK
    assert call(moe.NOALLOC_MAX_T + 1) == moe.MOE_FFN_ETOOBIG
    assert call(4096) == moe.MOE_FFN_ETOOBIG
    assert call(-1) == moe.MOE_FFN_EINVAL
    assert call(4, x=None) == moe.MOE_FFN_EINVAL
    assert call(4, x=0x20000008) == moe.MOE_FFN_EALIGN
    assert call(4, dims=moe.Dims(2048, 256, 8, 512, 512, 32)) == moe.MOE_FFN_EUNSUPPORTED
    assert moe.moe_ffn_status_string(moe.MOE_FFN_ETOOBIG) != "unknown status"
    assert "#define MOE_FFN_NOALLOC_MAX_T 64" in open(HEADER).read()


def test_hash_router_arguments(L):
    """A hash table needs token ids and n_vocab >= 1, both 16-byte aligned;
    accepted arguments get as far as the workspace check."""
    layer = _layer()
    r, ex, sh = layer.structs()

    def call(tab, ids, nv, ws=0x40000000):
        r.tid2eid, r.token_ids, r.n_vocab = tab, ids, nv
        return L.moe_ffn_forward_path(ctypes.byref(moe.DIMS), 4, 0x20000000, ctypes.byref(r), ctypes.byref(ex),
                                      ctypes.byref(sh), 0x30000000, None, None, ws, 16, None, 0)

    assert call(0x50000000, None, 100) == moe.MOE_FFN_EINVAL
    assert call(0x50000000, 0x51000000, 0) == moe.MOE_FFN_EINVAL
    assert call(0x50000004, 0x51000000, 100) == moe.MOE_FFN_EALIGN
    assert call(0x50000000, 0x51000008, 100) == moe.MOE_FFN_EALIGN
    assert call(0x50000000, 0x51000000, 100) == moe.MOE_FFN_EWORKSPACE
    assert call(None, None, 0) == moe.MOE_FFN_EWORKSPACE
