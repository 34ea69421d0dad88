"""GPU parity of the MXFP4-weight layer ("GPT-OSS on day 0": the expert weights ship as
MXFP4; "Hosting Qwen on Blackwell", section "Quantization": activations quantised per
token at run time, here MXFP8) against the oracle's "mxfp4" layer.

Packed e2m1 weight codes and their E8M0 scales are bit-exact in the tiled storage (code
bytes past K zero, scale pads 127); x codes
and scales are bit-exact; the routing tables are exact; h codes may differ only inside the
accumulation window; outputs meet the tolerance of the other formats.
"""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_gemm_amd as moe
from oracle import moe_ref as R
from synth import SHAPES, custom_shape
from gpu_helpers import GpuLayer, OracleExperts, bits_host, compare_out, routing_exact, say
from test_gpu_mx import _split, _wide, _ws_view, _check_h_dispatched, untile_scales

pytestmark = pytest.mark.gpu

FMT = "mxfp4"


def untile(codes: np.ndarray, scales: np.ndarray, N: int, K: int):
    """Row-major packed codes [E, N, K/2] and E8M0 rows [E, N, 4 ceil(K/128)] of the tiled
    storage (16-row x 128-K tiles), and the code bytes past K."""
    E, KB = codes.shape[0], -(-K // 128)
    c = codes.reshape(E, N // 16, KB, 16, 64).transpose(0, 1, 3, 2, 4).reshape(E, N, KB * 64)
    return c[..., :K // 2], untile_scales(scales, N, K), c[..., K // 2:]


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
    g = GpuLayer(shape, fmt=FMT)
    routing = moe.new_routing(shape.T, shape.E, shape.top_k)
    say(f"mxfp4 forward {shape.name}: T={shape.T} H={shape.H} E={shape.E} k={shape.top_k} I={shape.I}")
    out = g.layer(g.x, routing=routing)
    torch.cuda.synchronize()
    ox = OracleExperts(shape, g.li, fmt=FMT)
    ref = ox.forward()
    routing_exact(routing, ref, shape.T, shape.top_k, shape.name)
    T, H, I, rows = shape.T, shape.H, shape.I, shape.T * shape.top_k
    xq = _ws_view(g.layer, T, "xq", torch.uint8, (T, H)).cpu().numpy()
    sx = _ws_view(g.layer, T, "sx", torch.uint8, (T, moe.mx_row(H))).cpu().numpy()
    real, pad = _split(sx, H)
    assert np.array_equal(xq, ref["xq"]) and np.array_equal(real, ref["sx"]) and np.all(pad == 127)
    hq = _ws_view(g.layer, T, "h", torch.uint8, (rows, I)).cpu().numpy()
    hs = _ws_view(g.layer, T, "sh", torch.uint8, (rows, moe.mx_row(I))).cpu().numpy()
    _check_h_dispatched(g, ox, ref, hq, hs, fmt=FMT)
    compare_out(bits_host(out), ref["out"], shape.name, allowance=ref["allowance"])


@pytest.mark.timeout(900)
def test_forward_mxfp4_decode_layer_all_tokens():
    shape = SHAPES["gpt-oss-20b-decode"]
    g = GpuLayer(shape, fmt=FMT)
    routing = moe.new_routing(shape.T, shape.E, shape.top_k)
    say(f"mxfp4 forward {shape.name}")
    out = g.layer(g.x, routing=routing)
    torch.cuda.synchronize()
    ref = OracleExperts(shape, g.li, fmt=FMT).forward()
    routing_exact(routing, ref, shape.T, shape.top_k, shape.name)
    compare_out(bits_host(out), ref["out"], shape.name, allowance=ref["allowance"])


@pytest.mark.timeout(1200)
def test_forward_mxfp4_prefill_layer_sampled():
    """The prefill-sized layer (every expert ~256 rows: the 256-row tile kernel and its
    narrow overflow tiles), checked on sampled tokens (the last one included)."""
    shape = SHAPES["gpt-oss-120b-prefill"]
    g = GpuLayer(shape, fmt=FMT)
    routing = moe.new_routing(shape.T, shape.E, shape.top_k)
    say(f"mxfp4 forward {shape.name}")
    out = g.layer(g.x, routing=routing)
    torch.cuda.synchronize()
    rng = np.random.default_rng(97)
    toks = np.sort(rng.choice(shape.T, size=6, replace=False))
    toks[-1] = shape.T - 1
    ref = OracleExperts(shape, g.li, fmt=FMT).forward(token_subset=toks)
    routing_exact(routing, ref, shape.T, shape.top_k, shape.name)
    compare_out(bits_host(out)[toks], ref["out"], f"{shape.name} tokens {toks.tolist()}",
                allowance=ref["allowance"])


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
