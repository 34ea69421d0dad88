"""GPU tests of the decode-sized layer in one persistent kernel (moe_forward_fused).

"Hosting Qwen on Blackwell", section "Expert Parallel": for decode the dispatch, the expert
GEMMs and the combine run as one kernel.  The fused kernel runs each stage with the
arithmetic of the multi-kernel path, so:

1. where that path also takes the one-workgroup routing tail (top_k <= 4) and the row-run
   GEMM tiles (H and I = 64 mod 128), the fused call is compared with moe_forward bit for
   bit: out, the six routing tables, and the x codes, h and y in the workspace;
2. every fused layer is checked against the oracle by the same LayerCheck as the
   multi-kernel path (routing bit-exact, h in its analytic window, oracle GEMM2 + combine
   on the GPU's h at the literal tolerance, plain oracle rel. Frobenius), on every routed
   row and token;
3. the bounded waits' error path: with the wait bound forced to give up at once (a host
   setting, so no wait ever spins out), every workgroup still exits, the status word
   reports the error, and the next call with the normal bound is correct again.
"""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_gemm_amd as moe
from sparse_moe_ffn_gemm_amd import _lib
from synth import SHAPES, custom_shape
from gpu_helpers import GpuLayer, check_all_rows, say

pytestmark = pytest.mark.gpu

# layers the multi-kernel path runs with the routing tail and the row-run tiles
SAME_PATH = [
    SHAPES["gpt-oss-20b-decode"],
    custom_shape(T=1, H=192, E=8, top_k=2, I=320, seed=71),                # one token
    custom_shape(T=37, H=448, E=16, top_k=4, I=192, seed=72),              # ragged everything
    custom_shape(T=64, H=320, E=64, top_k=1, I=448, seed=73, expert_bias=False),
    custom_shape(T=128, H=192, E=128, top_k=1, I=192, seed=74, router="one_per_expert"),
    custom_shape(T=24, H=704, E=4, top_k=4, I=320, seed=75),               # k = E
    custom_shape(T=64, H=192, E=256, top_k=2, I=64, seed=76),              # 256 experts, I = 64
]
# other decode-sized layers (top_k 8, K multiples of 128): oracle parity only
OTHER = [
    SHAPES["qwen3-235b-decode"],
    custom_shape(T=16, H=256, E=16, top_k=1, I=128, seed=43, router="one_per_expert"),
    custom_shape(T=50, H=512, E=64, top_k=8, I=256, seed=77),
    custom_shape(T=3, H=128, E=2, top_k=1, I=128, seed=78),                # most rows in one expert
]


def _regions(g):
    s = g.shape
    kb = lambda n: (n + 127) // 128
    fp = g.fmt != "block"
    return [("xq", torch.uint8, (s.T, s.H)),
            ("sx", torch.uint8 if fp else torch.float32, (s.T, 4 * kb(s.H) if fp else kb(s.H))),
            ("h", torch.uint8, (s.rows, s.I)),
            ("sh", torch.uint8 if fp else torch.float32, (s.rows, 4 * kb(s.I) if fp else kb(s.I))),
            ("y", torch.float16, (s.rows, s.H))]


def _snapshot(g):
    return {name: g.ws_view(name, dt, shp).clone() for name, dt, shp in _regions(g)}


def _same(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("fmt", ["block", "mxfp8", "mxfp4"])
@pytest.mark.parametrize("shape", SAME_PATH, ids=[s.name for s in SAME_PATH])
def test_fused_bit_identical_to_multi_kernel(shape, fmt):
    g = GpuLayer(shape, fmt=fmt)
    out_ref, r_ref = g.run()
    ref = _snapshot(g)
    g.layer.workspace(shape.T).fill_(0x5A)          # nothing may survive from the first call
    out, r = g.run(fused=True)
    got = _snapshot(g)
    for k in r_ref:
        assert torch.equal(r[k], r_ref[k]), f"routing table {k}"
    for name in ref:
        assert _same(got[name], ref[name]), f"workspace region {name}"
    assert _same(out, out_ref), "out"
    say(f"  bit-identical: out, routing, {', '.join(ref)}")


@pytest.mark.parametrize("shape", SAME_PATH[:3] + OTHER, ids=[s.name for s in SAME_PATH[:3] + OTHER])
def test_fused_oracle_parity(shape):
    check_all_rows(shape, fused=True)


@pytest.mark.parametrize("name,fmt", [("gpt-oss-20b-decode", "mxfp8"), ("gpt-oss-20b-decode", "mxfp4"),
                                      ("qwen3-235b-decode", "mxfp8")])
@pytest.mark.timeout(900)
def test_fused_oracle_parity_mx(name, fmt):
    check_all_rows(SHAPES[name], fmt=fmt, fused=True)


def test_fused_mxfp4_top8_same_gemms_as_multi_kernel():
    """qwen3-235b-decode with MXFP4 weights: the multi-kernel path routes top-8 with its
    separate top-k kernel (another summation order of the router partials) but streams the
    experts with the same row-run tiles, so the routing decisions, the x codes, h and y must
    be identical and the gates and out equal up to fp32 rounding of the logit sums (the
    multi-kernel path itself is checked against the oracle on this layer)."""
    shape = SHAPES["qwen3-235b-decode"]
    g = GpuLayer(shape, fmt="mxfp4")
    out_ref, r_ref = g.run()
    ref = _snapshot(g)
    out, r = g.run(fused=True)
    got = _snapshot(g)
    for k in ("topk_ids", "expert_counts", "expert_offsets", "perm", "inv_perm"):
        assert torch.equal(r[k], r_ref[k]), f"routing table {k}"
    # each path's gates lie within the oracle's gate tolerance (1e-6 + 4 fp32 ulps of logits
    # of magnitude below 8): their difference within twice that
    gd = (r["topk_gates"] - r_ref["topk_gates"]).abs().max().item()
    assert gd <= 2 * (1e-6 + 4 * 2.0 ** -21), gd
    for name in ref:
        assert _same(got[name], ref[name]), f"workspace region {name}"
    # out = sum_j g_j y_j rounded once to bf16: the gate difference moves the fp32 sum by at
    # most gd * sum_j |y_j|, the two roundings add at most one bf16 ulp each
    y = got["y"].float()
    ysum = y[r["inv_perm"].long()].abs().view(shape.T, shape.top_k, shape.H).sum(dim=1)
    d = (out.float() - out_ref.float()).abs()
    ulp = torch.clamp(torch.maximum(out.float().abs(), out_ref.float().abs()), min=2.0 ** -126) * 2.0 ** -7
    tol = 2 * ulp + gd * ysum
    assert bool((d <= tol).all()), float((d / tol).max())
    say(f"  identical routing, x codes, h, y; gates within {gd:.1e}")


def test_fused_deterministic_across_calls_and_streams():
    shape = SHAPES["gpt-oss-20b-decode"]
    g = GpuLayer(shape)
    a = g.layer(g.x, fused=True).clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = g.layer(g.x, fused=True).clone()
    s.synchronize()
    c = g.layer(g.x, fused=True).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_fused_smaller_call_after_larger_reuses_workspace():
    shape = SHAPES["gpt-oss-20b-decode"]
    g = GpuLayer(shape)
    ws = g.layer.workspace(shape.T)
    full = g.layer(g.x, fused=True).clone()
    x5 = g.x[:5].contiguous()
    part = moe.forward_fused(x5, g.layer.router_w, g.layer.router_b, g.layer.w13, g.layer.w13_scales,
                             g.layer.b13, g.layer.w2, g.layer.w2_scales, g.layer.b2, shape.top_k,
                             workspace=ws)
    ref5 = moe.forward(x5, g.layer.router_w, g.layer.router_b, g.layer.w13, g.layer.w13_scales,
                       g.layer.b13, g.layer.w2, g.layer.w2_scales, g.layer.b2, shape.top_k)
    torch.cuda.synchronize()
    assert moe.fused_status(ws, 5, shape.H, shape.E, shape.top_k, shape.I) == 0
    assert torch.equal(part, ref5)
    again = g.layer(g.x, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(again, full)


def test_fused_wait_error_path_and_recovery():
    """Every wait told to give up at once: the launch still completes (each workgroup
    leaves), the status word reports MOE_ERR_DEVICE_WAIT; with the bound restored the next
    call is bit-identical to moe_forward."""
    shape = SHAPES["gpt-oss-20b-decode"]
    g = GpuLayer(shape)
    ref = g.layer(g.x).clone()
    ws = g.layer.workspace(shape.T)
    prev = _lib.set_fused_spin_limit(-1)
    try:
        g.layer(g.x, fused=True)
        torch.cuda.synchronize()
        st = moe.fused_status(ws, shape.T, shape.H, shape.E, shape.top_k, shape.I)
    finally:
        _lib.set_fused_spin_limit(prev)
    assert st == -5
    out = g.layer(g.x, fused=True)
    torch.cuda.synchronize()
    assert moe.fused_status(ws, shape.T, shape.H, shape.E, shape.top_k, shape.I) == 0
    assert torch.equal(out, ref)


def test_fused_rejects_prefill_sized_layers():
    shape = SHAPES["tiny"]
    g = GpuLayer(shape)
    big = custom_shape(T=129, H=256, E=8, top_k=2, I=256, seed=5)
    x = torch.zeros((big.T, big.H), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError) as e:
        moe.forward_fused(x, g.layer.router_w, g.layer.router_b, g.layer.w13, g.layer.w13_scales,
                          g.layer.b13, g.layer.w2, g.layer.w2_scales, g.layer.b2, shape.top_k)
    assert "UNSUPPORTED_SHAPE" in str(e.value)
