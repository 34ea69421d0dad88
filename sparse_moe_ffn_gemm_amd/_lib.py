"""ctypes binding of ``libmoe_mi355x.so`` (argument marshalling only).

Every step of the layer runs in the library's HIP kernels; this module only checks
torch tensors (device, dtype, contiguity), passes their device pointers and the
current HIP stream, and turns status codes into exceptions.  There is no fallback:
if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED_SHAPE",
          -3: "MOE_ERR_WORKSPACE_TOO_SMALL", -4: "MOE_ERR_HIP", -5: "MOE_ERR_DEVICE_WAIT"}

EXPORTS = ["moe_status_str", "moe_workspace_bytes", "moe_workspace_layout",
           "moe_quantize_weights", "moe_quantize_activations", "moe_route", "moe_forward",
           "moe_forward_profiled", "moe_quantize_weights_mx", "moe_quantize_activations_mx",
           "moe_forward_mx", "moe_forward_mx_profiled", "moe_quantize_weights_mxfp4",
           "moe_forward_mxfp4", "moe_forward_mxfp4_profiled",
           "moe_forward_noalloc", "moe_forward_fused", "moe_fused_status",
           # test-only (include/moe_test.h)
           "moe_test_gemm_raw_workspace_bytes", "moe_test_gemm_raw", "moe_test_set_fused_spin_limit"]

# stage i runs between profiling events i and i + 1 (include/moe.h, moe_forward_profiled)
PROFILE_STAGES = ["router_gemm", "topk_softmax", "dispatch_scan", "dispatch_scatter",
                  "x_scale_gather", "gemm1", "gemm2", "combine"]


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


class Routing(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_gates", ctypes.c_void_p),
                ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("inv_perm", ctypes.c_void_p)]


class WorkspaceRegions(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("xq", "sx", "h", "sh", "y", "topk_ids", "topk_gates", "expert_counts",
                 "expert_offsets", "perm", "inv_perm", "total")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_moe_ffn_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.moe_status_str.argtypes = [i]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_workspace_bytes.argtypes = [i, i, i, i, i]
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_layout.argtypes = [i, i, i, i, i, ctypes.POINTER(WorkspaceRegions)]
        L.moe_workspace_layout.restype = i
        L.moe_quantize_weights.argtypes = [vp, i, i, i, vp, vp, vp]
        L.moe_quantize_weights.restype = i
        L.moe_quantize_activations.argtypes = [vp, i, i, vp, vp, vp]
        L.moe_quantize_activations.restype = i
        L.moe_route.argtypes = [vp, vp, vp, i, i, i, i, ctypes.POINTER(Routing), vp, sz, vp]
        L.moe_route.restype = i
        L.moe_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp,
                                  ctypes.POINTER(Routing), vp, sz, vp]
        L.moe_forward.restype = i
        L.moe_forward_profiled.argtypes = L.moe_forward.argtypes + [ctypes.POINTER(ctypes.c_void_p)]
        L.moe_forward_profiled.restype = i
        L.moe_quantize_weights_mx.argtypes = [vp, i, i, i, vp, vp, vp]
        L.moe_quantize_weights_mx.restype = i
        L.moe_quantize_activations_mx.argtypes = [vp, i, i, vp, vp, vp]
        L.moe_quantize_activations_mx.restype = i
        L.moe_forward_mx.argtypes = L.moe_forward.argtypes
        L.moe_forward_mx.restype = i
        L.moe_forward_mx_profiled.argtypes = L.moe_forward_profiled.argtypes
        L.moe_forward_mx_profiled.restype = i
        L.moe_quantize_weights_mxfp4.argtypes = [vp, i, i, i, vp, vp, vp]
        L.moe_quantize_weights_mxfp4.restype = i
        L.moe_forward_mxfp4.argtypes = L.moe_forward.argtypes
        L.moe_forward_mxfp4.restype = i
        L.moe_forward_mxfp4_profiled.argtypes = L.moe_forward_profiled.argtypes
        L.moe_forward_mxfp4_profiled.restype = i
        L.moe_forward_noalloc.argtypes = L.moe_forward.argtypes[:16] + [vp]
        L.moe_forward_noalloc.restype = i
        L.moe_forward_fused.argtypes = L.moe_forward.argtypes[:14] + [i] + L.moe_forward.argtypes[14:]
        L.moe_forward_fused.restype = i
        L.moe_fused_status.argtypes = [vp, i, i, i, i, i, vp]
        L.moe_fused_status.restype = i
        L.moe_test_set_fused_spin_limit.argtypes = [i]
        L.moe_test_set_fused_spin_limit.restype = i
        L.moe_test_gemm_raw_workspace_bytes.argtypes = [i, i, i]
        L.moe_test_gemm_raw_workspace_bytes.restype = sz
        L.moe_test_gemm_raw.argtypes = [i, i, i, vp, vp, i, vp, i, ctypes.POINTER(ctypes.c_int32), i,
                                        vp, vp, i, i, vp, vp, sz, vp]
        L.moe_test_gemm_raw.restype = i
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        raise MoEError(status, what)


def _dev(t: Optional[torch.Tensor], dtype, name: str, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _fp8(t: torch.Tensor, name: str, shape=None):
    if t is not None and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return _dev(t, torch.uint8, name, shape)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def kb(n: int) -> int:
    return (n + 127) // 128


def workspace_bytes(T: int, H: int, E: int, top_k: int, I: int) -> int:
    return int(lib().moe_workspace_bytes(T, H, E, top_k, I))


def workspace_layout(T: int, H: int, E: int, top_k: int, I: int) -> WorkspaceRegions:
    r = WorkspaceRegions()
    _check(lib().moe_workspace_layout(T, H, E, top_k, I, ctypes.byref(r)), "moe_workspace_layout")
    return r


def new_workspace(T, H, E, top_k, I, device="cuda") -> torch.Tensor:
    n = workspace_bytes(T, H, E, top_k, I)
    if n == 0:
        raise MoEError(-2, "moe_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def quantize_weights(w: torch.Tensor, codes: torch.Tensor = None, scales: torch.Tensor = None):
    """128x128 block quantisation of w [E, N, K] (or [N, K]) fp32 -> (codes uint8, scales fp32)."""
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    E, N, K = w3.shape
    if codes is None:
        codes = torch.empty((E, N, K), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((E, kb(N), kb(K)), dtype=torch.float32, device=w.device)
    st = lib().moe_quantize_weights(_dev(w3, torch.float32, "w"), E, N, K,
                                    _fp8(codes.view(E, N, K), "codes"),
                                    _dev(scales.view(E, kb(N), kb(K)), torch.float32, "scales"),
                                    _stream(w.device))
    _check(st, "moe_quantize_weights")
    if squeeze:
        return codes.view(N, K), scales.view(kb(N), kb(K))
    return codes, scales


def quantize_activations(x: torch.Tensor):
    """Per-token 1x128 quantisation of x [T, H] bf16 -> (codes uint8 [T,H], scales [T, ceil(H/128)])."""
    T, H = x.shape
    codes = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    scales = torch.empty((T, kb(H)), dtype=torch.float32, device=x.device)
    _check(lib().moe_quantize_activations(_dev(x, torch.bfloat16, "x"), T, H, _fp8(codes, "codes"),
                                          _dev(scales, torch.float32, "scales"), _stream(x.device)),
           "moe_quantize_activations")
    return codes, scales


def mx_row(K: int) -> int:
    """Bytes of one row of MXFP8 scale codes for K elements (4 per 128-wide K-step)."""
    return 4 * kb(K)


def quantize_weights_mx(w: torch.Tensor, codes: torch.Tensor = None, scales: torch.Tensor = None):
    """MXFP8 quantisation of w [E, N, K] (or [N, K]) fp32, N a multiple of 16 -> (e4m3 codes
    uint8 [E, N, K], E8M0 codes uint8 [E, *mx_scale_shape(N, K)] in scale tiles, pads 127)."""
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    E, N, K = w3.shape
    ss = mx_scale_shape(N, K)
    if codes is None:
        codes = torch.empty((E, N, K), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((E,) + ss, dtype=torch.uint8, device=w.device)
    st = lib().moe_quantize_weights_mx(_dev(w3, torch.float32, "w"), E, N, K,
                                       _fp8(codes.view(E, N, K), "codes"),
                                       _dev(scales.view((E,) + ss), torch.uint8, "scales"),
                                       _stream(w.device))
    _check(st, "moe_quantize_weights_mx")
    if squeeze:
        return codes.view(N, K), scales.view(ss)
    return codes, scales


def mx_scale_shape(N: int, K: int):
    """Shape of one weight matrix's E8M0 scale tiles (MXFP8 and MXFP4): 16-row x 128-K
    tiles (tile (n, j) holds rows 16n..16n+15 over K [128j, 128j+128)), each row's four
    codes of the K-block: [N/16, ceil(K/128), 16, 4]."""
    return (N // 16, kb(K), 16, 4)


def mxfp4_shapes(N: int, K: int):
    """Shapes of one matrix's MXFP4 storage, in the same tiles: codes [N/16, ceil(K/128),
    16, 64] (64 bytes per tile row, two codes a byte, zeros past K) and the scale tiles."""
    return (N // 16, kb(K), 16, 64), mx_scale_shape(N, K)


def quantize_weights_mxfp4(w: torch.Tensor, codes: torch.Tensor = None, scales: torch.Tensor = None):
    """MXFP4 quantisation of w [E, N, K] (or [N, K]) fp32 (N a multiple of 16, K of 32) ->
    (e2m1 codes uint8 [E, *mxfp4_shapes(N, K)[0]], E8M0 codes uint8 [E, *mxfp4_shapes[1]])
    in the tiled layout of ``mxfp4_shapes`` (scale pads 127)."""
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    E, N, K = w3.shape
    cs, ss = mxfp4_shapes(N, K)
    if codes is None:
        codes = torch.empty((E,) + cs, dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((E,) + ss, dtype=torch.uint8, device=w.device)
    st = lib().moe_quantize_weights_mxfp4(_dev(w3, torch.float32, "w"), E, N, K,
                                          _dev(codes.view((E,) + cs), torch.uint8, "codes"),
                                          _dev(scales.view((E,) + ss), torch.uint8, "scales"),
                                          _stream(w.device))
    _check(st, "moe_quantize_weights_mxfp4")
    if squeeze:
        return codes.view(cs), scales.view(ss)
    return codes, scales


def quantize_activations_mx(x: torch.Tensor):
    """Per-token 1x32 MXFP8 quantisation of x [T, H] bf16 -> (codes uint8 [T, H], E8M0 scale
    codes uint8 [T, 4 ceil(H/128)])."""
    T, H = x.shape
    codes = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    scales = torch.empty((T, mx_row(H)), dtype=torch.uint8, device=x.device)
    _check(lib().moe_quantize_activations_mx(_dev(x, torch.bfloat16, "x"), T, H, _fp8(codes, "codes"),
                                             _dev(scales, torch.uint8, "scales"), _stream(x.device)),
           "moe_quantize_activations_mx")
    return codes, scales


def new_routing(T: int, E: int, top_k: int, device="cuda") -> dict:
    i32 = dict(dtype=torch.int32, device=device)
    return dict(topk_ids=torch.empty((T, top_k), **i32),
                topk_gates=torch.empty((T, top_k), dtype=torch.float32, device=device),
                expert_counts=torch.empty(E, **i32), expert_offsets=torch.empty(E + 1, **i32),
                perm=torch.empty(T * top_k, **i32), inv_perm=torch.empty(T * top_k, **i32))


def _routing_struct(r: dict, T: int, E: int, top_k: int) -> Routing:
    return Routing(_dev(r["topk_ids"], torch.int32, "topk_ids", (T, top_k)),
                   _dev(r["topk_gates"], torch.float32, "topk_gates", (T, top_k)),
                   _dev(r["expert_counts"], torch.int32, "expert_counts", (E,)),
                   _dev(r["expert_offsets"], torch.int32, "expert_offsets", (E + 1,)),
                   _dev(r["perm"], torch.int32, "perm", (T * top_k,)),
                   _dev(r["inv_perm"], torch.int32, "inv_perm", (T * top_k,)))


def route(x, router_w, router_b, top_k: int, routing: dict = None, workspace=None) -> dict:
    """Router GEMM + top-k + softmax + dispatch tables."""
    T, H = x.shape
    E = router_w.shape[0]
    if routing is None:
        routing = new_routing(T, E, top_k, x.device)
    if workspace is None:
        workspace = new_workspace(T, H, E, top_k, 64, x.device)
    rs = _routing_struct(routing, T, E, top_k)
    st = lib().moe_route(_dev(x, torch.bfloat16, "x"), _dev(router_w, torch.float32, "router_w", (E, H)),
                         _dev(router_b, torch.float32, "router_b", (E,)), T, H, E, top_k,
                         ctypes.byref(rs), _dev(workspace, torch.uint8, "workspace"),
                         workspace.numel(), _stream(x.device))
    _check(st, "moe_route")
    return routing


def _forward_args(x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2, top_k, out,
                  routing, workspace):
    T, H = x.shape
    E = router_w.shape[0]
    # MXFP4 weights are 16-row tiles: w13 [E, 2I/16, ceil(H/128), 16, 64]
    fp4 = w13.dim() == 5
    I = w13.shape[1] * 8 if fp4 else w2.shape[2]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = new_workspace(T, H, E, top_k, I, x.device)
    rs = _routing_struct(routing, T, E, top_k) if routing is not None else None
    mx = w13_scales.dtype == torch.uint8          # MX E8M0 codes, else fp32 block scales
    if mx:                                         # MXFP8 / MXFP4: scale tiles
        s13 = _dev(w13_scales, torch.uint8, "w13_scales", (E,) + mx_scale_shape(2 * I, H))
        s2 = _dev(w2_scales, torch.uint8, "w2_scales", (E,) + mx_scale_shape(H, I))
    else:
        s13 = _dev(w13_scales, torch.float32, "w13_scales", (E, kb(2 * I), kb(H)))
        s2 = _dev(w2_scales, torch.float32, "w2_scales", (E, kb(H), kb(I)))
    args = [
        _dev(x, torch.bfloat16, "x"), _dev(router_w, torch.float32, "router_w", (E, H)),
        _dev(router_b, torch.float32, "router_b", (E,)),
        _fp8(w13, "w13", (E,) + mxfp4_shapes(2 * I, H)[0] if fp4 else (E, 2 * I, H)), s13,
        _dev(b13, torch.bfloat16, "b13", (E, 2 * I)),
        _fp8(w2, "w2", (E,) + mxfp4_shapes(H, I)[0] if fp4 else (E, H, I)), s2,
        _dev(b2, torch.bfloat16, "b2", (E, H)),
        T, H, E, top_k, I, _dev(out, torch.bfloat16, "out", (T, H)),
        ctypes.byref(rs) if rs is not None else None,
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(x.device)]
    return out, args, (rs, workspace), ("mxfp4" if fp4 else "mxfp8") if mx else "block"


def forward(x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2, top_k: int,
            out=None, routing: dict = None, workspace=None) -> torch.Tensor:
    """The layer forward: out [T, H] bf16.  uint8 weight scales (E8M0 codes) select the
    MXFP8 layer (``quantize_weights_mx``) or, with tiled MXFP4 weights (5-d, from
    ``quantize_weights_mxfp4``), the MXFP4-weight layer; fp32 scales the block-scaled layer."""
    out, args, _keep, fmt = _forward_args(x, router_w, router_b, w13, w13_scales, b13, w2,
                                          w2_scales, b2, top_k, out, routing, workspace)
    fn = {"block": "moe_forward", "mxfp8": "moe_forward_mx", "mxfp4": "moe_forward_mxfp4"}[fmt]
    _check(getattr(lib(), fn)(*args), fn)
    return out


FORMATS = {"block": 0, "mxfp8": 1, "mxfp4": 2}   # weight_format of moe_forward_fused


def forward_fused(x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2, top_k: int,
                  out=None, routing: dict = None, workspace=None) -> torch.Tensor:
    """``forward`` through moe_forward_fused: a decode-sized layer in one persistent kernel
    (the weight format is read off the scales as in ``forward``)."""
    out, args, _keep, fmt = _forward_args(x, router_w, router_b, w13, w13_scales, b13, w2,
                                          w2_scales, b2, top_k, out, routing, workspace)
    args = args[:14] + [FORMATS[fmt]] + args[14:]
    _check(lib().moe_forward_fused(*args), "moe_forward_fused")
    return out


def fused_status(workspace: torch.Tensor, T: int, H: int, E: int, top_k: int, I: int) -> int:
    """moe_fused_status of the last moe_forward_fused on ``workspace`` (synchronises the
    current stream): 0 (MOE_OK) or -5 (MOE_ERR_DEVICE_WAIT)."""
    st = lib().moe_fused_status(_dev(workspace, torch.uint8, "workspace"), T, H, E, top_k, I,
                                _stream(workspace.device))
    if st not in (0, -5):
        _check(st, "moe_fused_status")
    return st


def set_fused_spin_limit(polls: int) -> int:
    """Test hook (include/moe_test.h): bound on the polls of every wait in later fused
    launches; negative = give up at once.  Returns the previous bound."""
    return lib().moe_test_set_fused_spin_limit(polls)


NOALLOC_BYTES = 64 << 20   # the library's fixed workspace of moe_forward_noalloc


def forward_noalloc(x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2, top_k: int,
                    out=None, routing: dict = None) -> torch.Tensor:
    """``forward`` (block-scaled weights) through moe_forward_noalloc: no workspace argument,
    the library's fixed per-device array instead (layers whose workspace is at most
    64 MiB)."""
    T, H = x.shape
    E = router_w.shape[0]
    I = w2.shape[2]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    rs = _routing_struct(routing, T, E, top_k) if routing is not None else None
    args = [
        _dev(x, torch.bfloat16, "x"), _dev(router_w, torch.float32, "router_w", (E, H)),
        _dev(router_b, torch.float32, "router_b", (E,)),
        _fp8(w13, "w13", (E, 2 * I, H)), _dev(w13_scales, torch.float32, "w13_scales", (E, kb(2 * I), kb(H))),
        _dev(b13, torch.bfloat16, "b13", (E, 2 * I)),
        _fp8(w2, "w2", (E, H, I)), _dev(w2_scales, torch.float32, "w2_scales", (E, kb(H), kb(I))),
        _dev(b2, torch.bfloat16, "b2", (E, H)),
        T, H, E, top_k, I, _dev(out, torch.bfloat16, "out", (T, H)),
        ctypes.byref(rs) if rs is not None else None, _stream(x.device)]
    _check(lib().moe_forward_noalloc(*args), "moe_forward_noalloc")
    return out


def forward_profiled(events, x, router_w, router_b, w13, w13_scales, b13, w2, w2_scales, b2,
                     top_k: int, out=None, routing: dict = None, workspace=None) -> torch.Tensor:
    """``forward`` that also records ``events`` (9 torch.cuda.Event(enable_timing=True),
    recorded on the current stream) before each stage and after the last; a ``None``
    entry leaves that boundary unrecorded."""
    if len(events) != len(PROFILE_STAGES) + 1:
        raise ValueError("need one event per stage plus one")
    out, args, _keep, fmt = _forward_args(x, router_w, router_b, w13, w13_scales, b13, w2,
                                          w2_scales, b2, top_k, out, routing, workspace)
    for ev in events:          # materialise the underlying hipEvent_t
        if ev is not None and ev.cuda_event == 0:
            ev.record()
    arr = (ctypes.c_void_p * len(events))(*[0 if ev is None else ev.cuda_event for ev in events])
    fn = {"block": "moe_forward_profiled", "mxfp8": "moe_forward_mx_profiled",
          "mxfp4": "moe_forward_mxfp4_profiled"}[fmt]
    _check(getattr(lib(), fn)(*args, arr), fn)
    return out


def gemm_raw_accumulators(gemm: int, fmt: str, bm: int, A: torch.Tensor, A_scales: torch.Tensor,
                  counts, B: torch.Tensor, B_scales: torch.Tensor, N: int, K: int,
                  perm: torch.Tensor = None, top_k: int = 1) -> torch.Tensor:
    """TEST-ONLY (include/moe_test.h): one grouped GEMM (``gemm`` 1 or 2) of the layer's
    kernels with its raw fp32 accumulators as the output, C [sum(counts), N].  ``counts`` are
    the routed rows per expert (host ints); ``fmt`` "block", "mxfp8" or "mxfp4"; ``bm`` the
    M-tile rows that select the kernel family as in the forward."""
    import numpy as np
    cnt = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
    rows, E = int(cnt.sum()), int(cnt.size)
    dev = A.device
    C = torch.empty((rows, N), dtype=torch.float32, device=dev)
    n = int(lib().moe_test_gemm_raw_workspace_bytes(rows, E, K))
    if n == 0:
        raise MoEError(-2, "moe_test_gemm_raw_workspace_bytes")
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    f = {"block": 0, "mxfp8": 1, "mxfp4": 2}[fmt]
    sdt = torch.float32 if fmt == "block" else torch.uint8
    st = lib().moe_test_gemm_raw(
        gemm, f, bm, _fp8(A, "A"), _dev(A_scales, sdt, "A_scales"), A.shape[0],
        _dev(perm, torch.int32, "perm"), top_k,
        cnt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), E, _fp8(B, "B"),
        _dev(B_scales, sdt, "B_scales"), N, K, _dev(C, torch.float32, "C"),
        _dev(ws, torch.uint8, "workspace"), ws.numel(), _stream(dev))
    _check(st, "moe_test_gemm_raw")
    return C
