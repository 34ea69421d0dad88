"""GPU parity of the whole layer (moe_forward, 128x128 block-scaled weights) against the oracle.

Every layer is checked by ``gpu_helpers.LayerCheck``: routing bit-exact, x codes and the
weights' codes bit-exact, the GPU's h inside the analytic window, the oracle's GEMM2 +
combine on the GPU's own h at the literal tolerance, and the plain oracle at relative
Frobenius 5e-3.  Small and decode-sized layers are checked on every routed row and every
token; the full-size prefill layers, in the launch configuration the benchmark times, on
whole experts (a full + overflow tile pair, the hottest expert) and on sampled tokens.
"""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_gemm_amd as moe
from synth import SHAPES, custom_shape
from gpu_helpers import GpuLayer, check_all_rows, check_prefill

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
    # 64-row LDS-ring tiles (25..96 rows per expert) and 128-row ones (97..160)
    custom_shape(T=160, H=256, E=8, top_k=2, I=256, seed=44),
    custom_shape(T=260, H=384, E=4, top_k=2, I=192, seed=45),
]


@pytest.mark.parametrize("shape", SMALL, ids=[s.name for s in SMALL])
def test_forward_small_full_parity(shape):
    check_all_rows(shape)


@pytest.mark.parametrize("name", ["gpt-oss-20b-decode", "qwen3-235b-decode"])
@pytest.mark.timeout(900)
def test_forward_decode_layers_all_tokens(name):
    check_all_rows(SHAPES[name])


@pytest.mark.parametrize("name,n_sample", [("gpt-oss-120b-prefill", 32), ("qwen3-235b-prefill", 24),
                                           ("deepseek-v3-skewed", 12)])
@pytest.mark.timeout(1500)
def test_forward_prefill_layers(name, n_sample):
    check_prefill(SHAPES[name], "block", n_sample, 99)


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
    xq = g.ws_view("xq", torch.uint8, (shape.T, shape.H))
    sx = g.ws_view("sx", torch.float32, (shape.T, kb))
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
