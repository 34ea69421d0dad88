"""The C-ABI library: it loads, exports every entry point include/moe.h declares, and its
host-side validation rejects bad arguments before anything is enqueued (no GPU needed:
these paths return before the first HIP call)."""
import ctypes
import os
import re

import pytest

import sparse_moe_ffn_gemm_amd as moe
from sparse_moe_ffn_gemm_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe.h")
FAKE = 1 << 20          # an aligned non-null address; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = moe.lib()
    for code, name in _lib.STATUS.items():
        assert L.moe_status_str(code).decode() == name
    assert L.moe_status_str(-99).decode() == "MOE_ERR_UNKNOWN"


@pytest.mark.parametrize("shape,ok", [
    ((16, 256, 8, 2, 256), True), ((1, 64, 1, 1, 64), True), ((8192, 2880, 128, 4, 2880), True),
    ((16384, 7168, 256, 8, 2048), True), ((0, 256, 8, 2, 256), False), ((16, 250, 8, 2, 256), False),
    ((16, 256, 8, 2, 100), False), ((16, 256, 300, 2, 256), False), ((16, 256, 8, 9, 256), False),
    ((16, 256, 4, 5, 256), False), ((16, 256, 8, 0, 256), False)])
def test_workspace_bytes_envelope(shape, ok):
    n = moe.lib().moe_workspace_bytes(*shape)
    assert (n > 0) == ok
    if ok:
        r = moe.workspace_layout(*shape)
        assert r.total == n
        T, H, E, k, I = shape
        assert r.y + 2 * T * k * H <= n and r.xq % 256 == 0 and r.y % 256 == 0


def _fwd(L, **kw):
    a = dict(x=FAKE, rw=FAKE, rb=None, w13=FAKE, s13=FAKE, b13=None, w2=FAKE, s2=FAKE, b2=None,
             T=16, H=256, E=8, k=2, I=256, out=FAKE, routing=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return L.moe_forward(a["x"], a["rw"], a["rb"], a["w13"], a["s13"], a["b13"], a["w2"], a["s2"],
                         a["b2"], a["T"], a["H"], a["E"], a["k"], a["I"], a["out"], a["routing"],
                         a["ws"], a["wsb"], None)


def test_forward_error_paths():
    L = moe.lib()
    assert _fwd(L, x=None) == -1
    assert _fwd(L, w13=None) == -1
    assert _fwd(L, ws=None) == -1
    assert _fwd(L, out=FAKE + 8) == -1                      # misaligned
    assert _fwd(L, T=0) == -2
    assert _fwd(L, H=96) == -2
    assert _fwd(L, I=32) == -2
    assert _fwd(L, k=3, E=2) == -2
    assert _fwd(L, E=257) == -2
    need = L.moe_workspace_bytes(16, 256, 8, 2, 256)
    assert _fwd(L, wsb=need - 1) == -3
    bad = _lib.Routing(FAKE, None, FAKE, FAKE, FAKE, FAKE)
    assert _fwd(L, routing=ctypes.byref(bad)) == -1


def test_route_and_quantize_error_paths():
    L = moe.lib()
    r = _lib.Routing(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.moe_route(None, FAKE, None, 16, 256, 8, 2, ctypes.byref(r), FAKE, 1 << 40, None) == -1
    assert L.moe_route(FAKE, FAKE, None, 16, 256, 8, 2, None, FAKE, 1 << 40, None) == -1
    assert L.moe_route(FAKE, FAKE, None, 16, 200, 8, 2, ctypes.byref(r), FAKE, 1 << 40, None) == -2
    assert L.moe_route(FAKE, FAKE, None, 16, 256, 8, 2, ctypes.byref(r), FAKE, 16, None) == -3
    assert L.moe_quantize_weights(None, 1, 128, 128, FAKE, FAKE, None) == -1
    assert L.moe_quantize_weights(FAKE, 0, 128, 128, FAKE, FAKE, None) == -1
    assert L.moe_quantize_weights(FAKE, 1, 128, 120, FAKE, FAKE, None) == -2
    assert L.moe_quantize_activations(FAKE, 4, 100, FAKE, FAKE, None) == -2
    assert L.moe_quantize_activations(FAKE + 2, 4, 128, FAKE, FAKE, None) == -1


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        moe.quantize_activations(x)


def _fwd_mx(fn, **kw):
    a = dict(x=FAKE, rw=FAKE, rb=None, w13=FAKE, s13=FAKE, b13=None, w2=FAKE, s2=FAKE, b2=None,
             T=16, H=256, E=8, k=2, I=256, out=FAKE, routing=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return fn(a["x"], a["rw"], a["rb"], a["w13"], a["s13"], a["b13"], a["w2"], a["s2"], a["b2"],
              a["T"], a["H"], a["E"], a["k"], a["I"], a["out"], a["routing"], a["ws"], a["wsb"], None)


def test_mx_error_paths():
    """MXFP8 / MXFP4 entry points: null and misaligned arguments, shapes the quantisers'
    tiled storage cannot hold (N not a multiple of 16, K not of 32), and decode-sized
    MXFP4 layers wider than the row-run kernel's LDS tile."""
    L = moe.lib()
    for q in (L.moe_quantize_weights_mx, L.moe_quantize_weights_mxfp4):
        assert q(None, 1, 128, 128, FAKE, FAKE, None) == -1
        assert q(FAKE, 0, 128, 128, FAKE, FAKE, None) == -1
        assert q(FAKE, 1, 120, 128, FAKE, FAKE, None) == -2      # N % 16
        assert q(FAKE, 1, 128, 48, FAKE, FAKE, None) == -2       # K % 32
        assert q(FAKE + 4, 1, 128, 128, FAKE, FAKE, None) == -1  # misaligned source
    assert L.moe_quantize_activations_mx(FAKE, 4, 96, FAKE, FAKE, None) == -2
    for fn in (L.moe_forward_mx, L.moe_forward_mxfp4):
        assert _fwd_mx(fn, x=None) == -1
        assert _fwd_mx(fn, s13=FAKE + 2) == -1                  # scale words need 4-byte alignment
        assert _fwd_mx(fn, T=0) == -2
        need = L.moe_workspace_bytes(16, 256, 8, 2, 256)
        assert _fwd_mx(fn, wsb=need - 1) == -3
    # 4 tokens over 2 experts (16-row tiles) with H = 8448: MXFP4 refuses, MXFP8 does not
    # reach a launch either way here (its workspace is too small on purpose)
    assert _fwd_mx(L.moe_forward_mxfp4, T=4, H=8448, E=2, k=1, I=128) == -2
    assert _fwd_mx(L.moe_forward_mx, T=4, H=8448, E=2, k=1, I=128, wsb=16) == -3
