"""The C-ABI library: it loads, exports every entry point include/moe.h declares, and its
host-side validation rejects bad arguments before anything is enqueued (no GPU needed:
these paths return before the first HIP call)."""
import ctypes
import os
import re

import pytest

import sparse_moe_ffn_gemm_amd as moe
from sparse_moe_ffn_gemm_amd import _lib

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
FAKE = 1 << 20          # an aligned non-null address; never dereferenced by these calls


def declared_functions():
    """Every function declared in include/*.h (the layer's API and the test-only export)."""
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


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
    # 32-bit GEMM offsets: T k I (the h rows GEMM2 reads) and 2 I H (one expert's w13) < 2^31
    ((262144, 7168, 256, 8, 2048), False), ((131072, 7168, 256, 8, 2048), False),
    ((131071, 7168, 256, 8, 2048), True), ((64, 65536, 8, 2, 16384), False),
    ((64, 32768, 8, 2, 32704), True),
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


def test_forward_rejects_shapes_past_32bit_gemm_offsets():
    """Shapes whose GEMM operand offsets would pass 2^31 bytes are refused before anything
    is enqueued (MOE_ERR_UNSUPPORTED_SHAPE), by every forward entry point."""
    L = moe.lib()
    for fn in (L.moe_forward_mx, L.moe_forward_mxfp4):
        assert _fwd_mx(fn, T=262144, H=7168, E=256, k=8, I=2048) == -2
        assert _fwd_mx(fn, T=64, H=65536, E=8, k=2, I=16384) == -2
    assert _fwd(L, T=262144, H=7168, E=256, k=8, I=2048) == -2
    assert _fwd(L, T=64, H=65536, E=8, k=2, I=16384) == -2
    r = _lib.Routing(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    # routing alone reads only x [T, H] and W: its envelope is T H < 2^31
    assert L.moe_route(FAKE, FAKE, None, 262144, 8192, 256, 8, ctypes.byref(r), FAKE, 16, None) == -2


def test_raw_gemm_export_error_paths():
    """The test-only GEMM export validates its arguments on the host."""
    L = moe.lib()
    cnt = (ctypes.c_int32 * 2)(10, 20)
    raw = lambda **kw: L.moe_test_gemm_raw(
        kw.get("gemm", 2), kw.get("fmt", 0), kw.get("bm", 64), kw.get("A", FAKE), FAKE,
        kw.get("A_rows", 30), kw.get("perm", None), 1, kw.get("cnt", cnt), 2, FAKE, FAKE,
        kw.get("N", 128), kw.get("K", 128), FAKE, FAKE, kw.get("wsb", 1 << 30), None)
    assert raw(gemm=3) == -1
    assert raw(fmt=3) == -1
    assert raw(A=None) == -1
    assert raw(gemm=1) == -1                     # GEMM1 needs perm
    assert raw(A=FAKE + 4) == -1
    assert raw(bm=32) == -2
    assert raw(N=96) == -2 and raw(K=100) == -2
    assert raw(fmt=1, bm=64) == -2               # MX formats: 16- or 256-row tiles only
    assert raw(A_rows=20) == -2                  # GEMM2 reads one A row per routed row
    assert raw(wsb=16) == -3
    assert L.moe_test_gemm_raw_workspace_bytes(30, 2, 128) > 0
    assert L.moe_test_gemm_raw_workspace_bytes(30, 0, 128) == 0


def test_noalloc_entry_point_rejects_before_touching_the_device():
    """moe_forward_noalloc refuses layers whose workspace exceeds its fixed 64 MiB
    (MOE_ERR_WORKSPACE_TOO_SMALL), bad shapes and null pointers, all before any HIP call."""
    L = moe.lib()
    na = lambda **kw: L.moe_forward_noalloc(
        kw.get("x", FAKE), FAKE, None, FAKE, FAKE, None, FAKE, FAKE, None, kw.get("T", 64),
        kw.get("H", 2880), kw.get("E", 32), kw.get("k", 4), kw.get("I", 2880), FAKE, None, None)
    assert L.moe_workspace_bytes(8192, 2880, 128, 4, 2880) > _lib.NOALLOC_BYTES
    assert na(T=8192, E=128) == -3                  # the prefill layer does not fit
    assert na(T=64, H=100) == -2
    assert na(x=None) == -1
    assert L.moe_workspace_bytes(64, 2880, 32, 4, 2880) <= _lib.NOALLOC_BYTES


def test_fused_entry_point_rejects_before_touching_the_device():
    """moe_forward_fused validates the format, pointers, the general envelope and its own
    decode envelope (T <= 128, T E <= 16384, at most 24 rows per expert, H, I <= 8192) and
    the workspace size before any HIP call."""
    L = moe.lib()

    def fz(**kw):
        a = dict(x=FAKE, s13=FAKE, T=64, H=2880, E=32, k=4, I=2880, fmt=0, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return L.moe_forward_fused(a["x"], FAKE, None, FAKE, a["s13"], None, FAKE, FAKE, None,
                                   a["T"], a["H"], a["E"], a["k"], a["I"], a["fmt"], FAKE, None,
                                   a["ws"], a["wsb"], None)
    assert fz(fmt=3) == -1 and fz(fmt=-1) == -1
    assert fz(x=None) == -1
    assert fz(s13=FAKE + 2) == -1                   # scale pointers 4-byte aligned
    assert fz(H=100) == -2
    assert fz(T=129, E=128, k=1) == -2              # more tokens than the routing tail holds
    assert fz(T=128, E=256, k=1) == -2              # T E > 16384
    assert fz(T=64, E=8, k=4) == -2                 # 32 rows per expert: not decode-sized
    assert fz(T=8192, E=128) == -2                  # the prefill layer
    assert fz(H=8256) == -2                         # H > 8192
    need = L.moe_workspace_bytes(64, 2880, 32, 4, 2880)
    assert fz(wsb=need - 1) == -3
    assert L.moe_fused_status(None, 64, 2880, 32, 4, 2880, None) == -1
    assert L.moe_fused_status(FAKE, 64, 100, 32, 4, 2880, None) == -2
