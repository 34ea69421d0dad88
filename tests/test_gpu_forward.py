"""GPU parity of the whole layer (moe_forward) against the oracle.

Small layers are compared element by element on every output, plus the intermediates
(x codes/scales bit-exact, h codes up to rare one-code flips, y).  Full-size layers run in
the launch configuration the benchmark times; their routing tables are compared in
full and their outputs on sampled tokens the oracle evaluates one by one.
"""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_gemm_amd as moe
from oracle import moe_ref as R
from synth import SHAPES, custom_shape, make_inputs
from gpu_helpers import (GpuLayer, OracleExperts, bits_host, compare_out, dispatched_allowance,
                         h_codes_close, routing_exact, say)

pytestmark = pytest.mark.gpu

SMALL = [
    SHAPES["tiny"],
    custom_shape(T=37, H=192, E=5, top_k=2, I=192, seed=31),        # ragged K/N blocks
    custom_shape(T=1, H=256, E=8, top_k=2, I=256, seed=32),         # single token
    custom_shape(T=9, H=128, E=1, top_k=1, I=128, seed=33),         # dense FFN
    custom_shape(T=4, H=256, E=64, top_k=2, I=128, seed=34),        # most experts idle
    custom_shape(T=150, H=320, E=4, top_k=4, I=384, seed=35),       # k = E, >128 rows/expert
    custom_shape(T=200, H=256, E=16, top_k=3, I=128, seed=36, router="hot"),  # one hot expert
    custom_shape(T=96, H=384, E=8, top_k=2, I=320, seed=37, expert_bias=False),
    # > 160 rows per expert: 256-row tiles, a short last tile per expert, ragged K and N
    custom_shape(T=600, H=320, E=4, top_k=2, I=320, seed=38),
    custom_shape(T=700, H=448, E=2, top_k=1, I=192, seed=39, expert_bias=False),
    # every expert exactly one token (the pages' decode GEMM benchmark)
    custom_shape(T=16, H=256, E=16, top_k=1, I=128, seed=43, router="one_per_expert"),
]


def _workspace_view(layer, T, region, dtype, shape):
    r = moe.workspace_layout(T, layer.H, layer.E, layer.top_k, layer.I)
    ws = layer.workspace(T)
    off = getattr(r, region)
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype).view(*shape)


def _run(g: GpuLayer):
    s = g.shape
    routing = moe.new_routing(s.T, s.E, s.top_k)
    say(f"forward {s.name}: T={s.T} H={s.H} E={s.E} k={s.top_k} I={s.I}")
    out = g.layer(g.x, routing=routing)
    torch.cuda.synchronize()
    return out, routing


@pytest.mark.parametrize("shape", SMALL, ids=[s.name for s in SMALL])
def test_forward_small_full_parity(shape):
    g = GpuLayer(shape)
    out, routing = _run(g)
    ox = OracleExperts(shape, g.li)
    ox.prepare(range(shape.E))
    ref = R.forward_dispatched(g.li.x, g.li.router_w, g.li.router_b, shape.top_k, shape.I,
                               ox.view(0), ox.view(1), g.li.b13, ox.view(2), ox.view(3), g.li.b2)
    routing_exact(routing, ref, shape.T, shape.top_k, shape.name)
    # intermediates
    T, H, I, rows = shape.T, shape.H, shape.I, shape.T * shape.top_k
    xq = _workspace_view(g.layer, T, "xq", torch.uint8, (T, H)).cpu().numpy()
    sx = _workspace_view(g.layer, T, "sx", torch.float32, (T, -(-H // 128))).cpu().numpy()
    assert np.array_equal(xq, ref["xq"]) and np.array_equal(sx, ref["sx"])
    hq = _workspace_view(g.layer, T, "h", torch.uint8, (rows, I)).cpu().numpy()
    hs = _workspace_view(g.layer, T, "sh", torch.float32, (rows, -(-I // 128))).cpu().numpy()
    h_codes_close(hq, ref)
    hs_rel = np.abs(hs / ref["hs"] - 1).max()
    say(f"  h scales: max rel diff {hs_rel:.2e}")
    assert hs_rel < 1e-4
    y = _workspace_view(g.layer, T, "y", torch.float16, (rows, H)).cpu().numpy().astype(np.float64)
    y_rel = np.linalg.norm(y - ref["y"]) / max(np.linalg.norm(ref["y"]), 1e-300)
    say(f"  y rel err {y_rel:.2e}")
    assert y_rel < 3e-3
    compare_out(bits_host(out), ref["out"], shape.name,
                allowance=dispatched_allowance(ref, ox, shape.T, shape.top_k))


@pytest.mark.parametrize("name", ["gpt-oss-20b-decode", "qwen3-235b-decode"])
@pytest.mark.timeout(900)
def test_forward_decode_layers_all_tokens(name):
    shape = SHAPES[name]
    g = GpuLayer(shape)
    out, routing = _run(g)
    ref = OracleExperts(shape, g.li).forward()
    routing_exact(routing, ref, shape.T, shape.top_k, name)
    compare_out(bits_host(out), ref["out"], name, allowance=ref["allowance"])


@pytest.mark.parametrize("name,n_sample", [("gpt-oss-120b-prefill", 12), ("qwen3-235b-prefill", 8),
                                           ("deepseek-v3-skewed", 6)])
@pytest.mark.timeout(1200)
def test_forward_prefill_layers_sampled(name, n_sample):
    shape = SHAPES[name]
    g = GpuLayer(shape)
    out, routing = _run(g)
    ox = OracleExperts(shape, g.li)
    rng = np.random.default_rng(99)
    toks = np.sort(rng.choice(shape.T, size=n_sample, replace=False))
    toks[-1] = shape.T - 1                                   # include the last (ragged) tile
    ref = ox.forward(token_subset=toks)
    routing_exact(routing, ref, shape.T, shape.top_k, name)
    compare_out(bits_host(out)[toks], ref["out"], f"{name} tokens {toks.tolist()}",
                allowance=ref["allowance"])


def test_forward_deterministic_and_reentrant():
    shape = SHAPES["gpt-oss-20b-decode"]
    g = GpuLayer(shape)
    a = g.layer(g.x).clone()
    b = g.layer(g.x).clone()
    ws2 = moe.new_workspace(shape.T, shape.H, shape.E, shape.top_k, shape.I)
    c = moe.forward(g.x, g.layer.router_w, g.layer.router_b, g.layer.w13, g.layer.w13_scales,
                    g.layer.b13, g.layer.w2, g.layer.w2_scales, g.layer.b2, shape.top_k,
                    workspace=ws2)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("shape", [SHAPES["gpt-oss-20b-decode"],
                                   custom_shape(T=150, H=448, E=70, top_k=2, I=128, seed=40),
                                   custom_shape(T=300, H=2880, E=8, top_k=2, I=128, seed=41)],
                         ids=["gpt-oss-20b-decode", "T150-H448-E70", "T300-H2880-E8"])
def test_forward_activation_codes_match_quantiser(shape):
    """The router kernel quantises x for GEMM1 (1x128 groups): its codes and scales in the
    workspace are bit-identical to moe_quantize_activations' (ragged last group, several
    token tiles, H slices and expert tiles)."""
    g = GpuLayer(shape)
    g.layer(g.x)
    codes, scales = moe.quantize_activations(g.x)
    torch.cuda.synchronize()
    kb = (shape.H + 127) // 128
    xq = _workspace_view(g.layer, shape.T, "xq", torch.uint8, (shape.T, shape.H))
    sx = _workspace_view(g.layer, shape.T, "sx", torch.float32, (shape.T, kb))
    assert torch.equal(xq, codes)
    assert torch.equal(sx.view(torch.int32), scales.view(torch.int32))


def test_forward_profiled_matches_forward_with_partial_events():
    """The per-stage timing entry point does the same work: bit-identical output with all
    stage events, and with only the GEMM1 boundaries recorded (NULL entries elsewhere)."""
    shape = SHAPES["gpt-oss-20b-decode"]
    g = GpuLayer(shape)
    args = (g.x, g.layer.router_w, g.layer.router_b, g.layer.w13, g.layer.w13_scales,
            g.layer.b13, g.layer.w2, g.layer.w2_scales, g.layer.b2, shape.top_k)
    ref = moe.forward(*args).clone()
    full = [torch.cuda.Event(enable_timing=True) for _ in range(len(moe.PROFILE_STAGES) + 1)]
    a = moe.forward_profiled(full, *args).clone()
    part = [None] * (len(moe.PROFILE_STAGES) + 1)
    i1 = moe.PROFILE_STAGES.index("gemm1")
    part[i1], part[i1 + 1] = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b = moe.forward_profiled(part, *args).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, ref) and torch.equal(b, ref)
    assert all(full[i].elapsed_time(full[i + 1]) >= 0 for i in range(len(full) - 1))
    assert part[i1].elapsed_time(part[i1 + 1]) > 0


def test_forward_smaller_call_after_larger_reuses_workspace():
    shape = SHAPES["tiny"]
    g = GpuLayer(shape)
    ws = moe.new_workspace(shape.T, shape.H, shape.E, shape.top_k, shape.I)
    full = moe.forward(g.x, g.layer.router_w, g.layer.router_b, g.layer.w13, g.layer.w13_scales,
                       g.layer.b13, g.layer.w2, g.layer.w2_scales, g.layer.b2, shape.top_k,
                       workspace=ws).clone()
    part = moe.forward(g.x[:5].contiguous(), g.layer.router_w, g.layer.router_b, g.layer.w13,
                       g.layer.w13_scales, g.layer.b13, g.layer.w2, g.layer.w2_scales, g.layer.b2,
                       shape.top_k, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(part, full[:5])
