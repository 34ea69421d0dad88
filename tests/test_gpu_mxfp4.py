"""GPU parity of the MXFP4-weight layer ("GPT-OSS on day 0": the expert weights ship as
MXFP4; "Hosting Qwen on Blackwell", section "Quantization": activations quantised per
token at run time, here MXFP8) against the oracle's "mxfp4" layer.

Packed e2m1 weight codes and their E8M0 scales are bit-exact in the tiled storage (code
bytes past K zero, scale pads 127); x codes
and scales are bit-exact; the layers are checked by ``gpu_helpers.LayerCheck`` like the other
formats.
"""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_gemm_amd as moe
from oracle import moe_ref as R
from synth import SHAPES, custom_shape
from gpu_helpers import GpuLayer, check_all_rows, check_prefill, say
from layouts import untile_fp4, untile_scales
from test_gpu_mx import _split, _wide

pytestmark = pytest.mark.gpu

FMT = "mxfp4"


def untile(codes: np.ndarray, scales: np.ndarray, N: int, K: int):
    """Row-major packed codes [E, N, K/2] and E8M0 rows [E, N, 4 ceil(K/128)] of the tiled
    storage (16-row x 128-K tiles), and the code bytes past K."""
    c, tail = untile_fp4(codes, N, K)
    return c, untile_scales(scales, N, K), tail


@pytest.mark.parametrize("E,N,K", [(2, 192, 2880), (3, 64, 256), (1, 96, 96), (2, 16, 32)])
def test_weight_quantiser_bit_exact(E, N, K):
    rng = np.random.default_rng(E * 1000 + K + 4)
    w = _wide(rng, (E, N, K), K)
    w[0, :5, :32] = 0.0                                          # all-zero blocks
    # exact ties between neighbouring e2m1 values, at a block scale of 1 (block max 6)
    w[-1, -1, :32] = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4, np.float32)
    w[-1, -1, 1:32:8] *= -1
    say(f"mxfp4 weights E={E} N={N} K={K}")
    codes, scales = moe.quantize_weights_mxfp4(torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    rc, rs = R.quantize_mxfp4(w)
    cs, ss = moe.mxfp4_shapes(N, K)
    assert codes.shape == (E,) + cs and scales.shape == (E,) + ss
    c, s, tail = untile(codes.cpu().numpy(), scales.cpu().numpy(), N, K)
    real, pad = _split(s, K)
    assert np.array_equal(c, rc)
    assert np.all(tail == 0)
    assert np.array_equal(real, rs)
    assert np.all(pad == 127)


SMALL = [
    SHAPES["tiny"],
    custom_shape(T=37, H=192, E=5, top_k=2, I=192, seed=61),        # K tails (K = 64 mod 128)
    custom_shape(T=9, H=128, E=1, top_k=1, I=128, seed=62),         # dense FFN
    custom_shape(T=4, H=256, E=64, top_k=2, I=128, seed=63),        # most experts idle
    custom_shape(T=150, H=320, E=4, top_k=4, I=384, seed=64),       # 256-row tile kernel
    custom_shape(T=600, H=320, E=4, top_k=2, I=320, seed=65),       # full + narrow 256-row tiles
    custom_shape(T=300, H=192, E=4, top_k=2, I=192, seed=67),       # 256-row tiles, K tails
    custom_shape(T=40, H=256, E=2, top_k=1, I=128, seed=60),        # 20 rows per expert: 16-row tiles
    custom_shape(T=96, H=384, E=8, top_k=2, I=320, seed=66, expert_bias=False),
    custom_shape(T=16, H=256, E=16, top_k=1, I=128, seed=68, router="one_per_expert"),
    # the decode GEMM benchmark's shape at a high expert-parallel degree (32-column tiles)
    custom_shape(T=4, H=4096, E=4, top_k=1, I=1536, seed=3, expert_bias=False,
                 router="one_per_expert"),
    custom_shape(T=1, H=256, E=8, top_k=2, I=256, seed=81),         # single token
    custom_shape(T=200, H=256, E=16, top_k=3, I=128, seed=82, router="hot"),  # one hot expert
    custom_shape(T=33, H=64, E=256, top_k=8, I=64, seed=83),        # smallest H, I; most experts, top-8
    custom_shape(T=700, H=448, E=2, top_k=1, I=192, seed=84, expert_bias=False),  # large groups, K tails
]


@pytest.mark.parametrize("shape", SMALL, ids=[s.name for s in SMALL])
def test_forward_mxfp4_small_full_parity(shape):
    check_all_rows(shape, FMT)


@pytest.mark.parametrize("name", ["gpt-oss-20b-decode", "qwen3-235b-decode"])
@pytest.mark.timeout(900)
def test_forward_mxfp4_decode_layers_all_tokens(name):
    check_all_rows(SHAPES[name], FMT)


@pytest.mark.parametrize("name,n_sample", [("gpt-oss-120b-prefill", 16), ("qwen3-235b-prefill", 16)])
@pytest.mark.timeout(1500)
def test_forward_mxfp4_prefill_layers(name, n_sample):
    """The prefill-sized layers (the 256-row tile kernel and its narrow overflow tiles) on
    whole experts and sampled tokens (the last one included)."""
    check_prefill(SHAPES[name], FMT, n_sample, 97)


def test_forward_mxfp4_rejects_wide_layers():
    """The decode-sized MXFP4 GEMMs stage a 16-row activation tile of all of K in LDS:
    H, I <= 8192 there."""
    shape = custom_shape(T=4, H=8192 + 256, E=2, top_k=1, I=128, seed=69)
    g = GpuLayer(shape, fmt=FMT)
    with pytest.raises(RuntimeError):
        g.layer(g.x)
    torch.cuda.synchronize()


def test_forward_mxfp4_profiled_and_deterministic():
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
