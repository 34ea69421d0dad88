"""GPU parity of the MXFP8 variant ("Hosting Qwen on Blackwell", section "Quantization":
weights converted statically to MXFP8) against the oracle's MXFP8 layer.

Weight and activation codes and E8M0 scales are bit-exact (the pad bytes of the scale rows
are 127); the layers are checked by ``gpu_helpers.LayerCheck`` (routing exact, h inside the
analytic window with its E8M0 codes, the oracle's GEMM2 + combine on the GPU's h at the
literal tolerance, the plain oracle at relative Frobenius 5e-3).
"""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_gemm_amd as moe
from oracle import moe_ref as R
from synth import SHAPES, custom_shape
from gpu_helpers import GpuLayer, bf16_dev, check_all_rows, check_prefill, say
from layouts import untile_scales

pytestmark = pytest.mark.gpu

FMT = "mxfp8"


def _split(scales: np.ndarray, K: int):
    """(E8M0 codes of the K/32 blocks, pad bytes) of padded scale rows."""
    return scales[..., :K // 32], scales[..., K // 32:]


def _wide(rng, shape, blocks_axis_len):
    a = rng.standard_normal(shape) * 0.02
    a *= np.exp2(rng.integers(-20, 20, size=shape[:-1] + (blocks_axis_len // 32,))).repeat(32, axis=-1)
    return a.astype(np.float32)


@pytest.mark.parametrize("E,N,K", [(2, 192, 2880), (3, 64, 256), (1, 96, 96)])
def test_weight_quantiser_bit_exact(E, N, K):
    rng = np.random.default_rng(E * 1000 + K)
    w = _wide(rng, (E, N, K), K)
    w[0, :5, :32] = 0.0                                          # all-zero blocks
    say(f"mx weights E={E} N={N} K={K}")
    codes, scales = moe.quantize_weights_mx(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    rc, rs = R.quantize_mx(w)
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    assert scales.shape == (E,) + moe.mx_scale_shape(N, K)
    real, pad = _split(untile_scales(scales, N, K), K)
    assert np.array_equal(codes, rc)
    assert np.array_equal(real, rs)
    assert np.all(pad == 127)


@pytest.mark.parametrize("T,H", [(37, 2880), (5, 256), (64, 192)])
def test_activation_quantiser_bit_exact(T, H):
    rng = np.random.default_rng(T + H)
    x32 = _wide(rng, (T, H), H) * 50
    x32[0] = 0.0
    xb = bf16_dev(R.f64_to_bf16_bits(x32.astype(np.float64)))
    say(f"mx activations T={T} H={H}")
    codes, scales = moe.quantize_activations_mx(xb)
    torch.cuda.synchronize()
    xr = R.bf16_to_f64(R.f64_to_bf16_bits(x32.astype(np.float64))).astype(np.float32)
    rc, rs = R.quantize_mx(xr)
    real, pad = _split(scales.cpu().numpy(), H)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(real, rs)
    assert np.all(pad == 127)


SMALL = [
    SHAPES["tiny"],
    custom_shape(T=37, H=192, E=5, top_k=2, I=192, seed=51),        # K tails (K = 64 mod 128)
    custom_shape(T=9, H=128, E=1, top_k=1, I=128, seed=52),         # dense FFN
    custom_shape(T=4, H=256, E=64, top_k=2, I=128, seed=53),        # most experts idle
    custom_shape(T=150, H=320, E=4, top_k=4, I=384, seed=54),       # > 64 rows: full tile body
    custom_shape(T=600, H=320, E=4, top_k=2, I=320, seed=55),       # several 256-row tiles
    custom_shape(T=96, H=384, E=8, top_k=2, I=320, seed=56, expert_bias=False),
    # every expert exactly one token (the pages' decode GEMM benchmark)
    custom_shape(T=16, H=256, E=16, top_k=1, I=128, seed=58, router="one_per_expert"),
    custom_shape(T=1, H=256, E=8, top_k=2, I=256, seed=71),         # single token
    custom_shape(T=200, H=256, E=16, top_k=3, I=128, seed=72, router="hot"),  # one hot expert
    custom_shape(T=33, H=64, E=256, top_k=8, I=64, seed=73),        # smallest H, I; most experts, top-8
    custom_shape(T=700, H=448, E=2, top_k=1, I=192, seed=74, expert_bias=False),  # large groups, K tails
]


@pytest.mark.parametrize("shape", SMALL, ids=[s.name for s in SMALL])
def test_forward_mx_small_full_parity(shape):
    check_all_rows(shape, FMT)


@pytest.mark.parametrize("name", ["gpt-oss-20b-decode", "qwen3-235b-decode"])
@pytest.mark.timeout(900)
def test_forward_mx_decode_layers_all_tokens(name):
    check_all_rows(SHAPES[name], FMT)


@pytest.mark.parametrize("name,n_sample", [("gpt-oss-120b-prefill", 16), ("qwen3-235b-prefill", 16)])
@pytest.mark.timeout(1500)
def test_forward_mx_prefill_layers(name, n_sample):
    check_prefill(SHAPES[name], FMT, n_sample, 98)


@pytest.mark.parametrize("shape", [SHAPES["gpt-oss-20b-decode"],
                                   custom_shape(T=300, H=2880, E=8, top_k=2, I=128, seed=57)],
                         ids=["gpt-oss-20b-decode", "T300-H2880-E8"])
def test_forward_mx_activation_codes_match_quantiser(shape):
    """The router kernel's MXFP8 x codes and scale rows (pads included) are bit-identical to
    moe_quantize_activations_mx's."""
    g = GpuLayer(shape, fmt=FMT)
    g.layer(g.x)
    codes, scales = moe.quantize_activations_mx(g.x)
    torch.cuda.synchronize()
    xq = g.ws_view("xq", torch.uint8, (shape.T, shape.H))
    sx = g.ws_view("sx", torch.uint8, (shape.T, moe.mx_row(shape.H)))
    assert torch.equal(xq, codes) and torch.equal(sx, scales)


def test_forward_mx_profiled_and_deterministic():
    shape = SHAPES["gpt-oss-20b-decode"]
    g = GpuLayer(shape, fmt=FMT)
    args = (g.x, g.layer.router_w, g.layer.router_b, g.layer.w13, g.layer.w13_scales,
            g.layer.b13, g.layer.w2, g.layer.w2_scales, g.layer.b2, shape.top_k)
    a = moe.forward(*args).clone()
    b = moe.forward(*args).clone()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(moe.PROFILE_STAGES) + 1)]
    c = moe.forward_profiled(ev, *args).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c)
