"""GPU parity of the MXFP8 variant ("Hosting Qwen on Blackwell", section "Quantization":
weights converted statically to MXFP8) against the oracle's MXFP8 layer.

Weight and activation codes and E8M0 scales are bit-exact (the pad bytes of the scale rows
are 127); the routing tables are exact; h codes may differ only inside the accumulation
window; outputs meet the same tolerance as the block-scaled layer.
"""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_gemm_amd as moe
from oracle import moe_ref as R
from synth import SHAPES, custom_shape
from gpu_helpers import (GpuLayer, OracleExperts, bf16_dev, bits_host, compare_out, routing_exact,
                         say, H_EPS, _group128_max)

pytestmark = pytest.mark.gpu

FMT = "mxfp8"


def _split(scales: np.ndarray, K: int):
    """(E8M0 codes of the K/32 blocks, pad bytes) of padded scale rows."""
    return scales[..., :K // 32], scales[..., K // 32:]


def untile_scales(scales: np.ndarray, N: int, K: int) -> np.ndarray:
    """Padded E8M0 rows [E, N, 4 ceil(K/128)] of weight scale tiles [E, N/16, KB, 16, 4]."""
    E, KB = scales.shape[0], -(-K // 128)
    return scales.reshape(E, N // 16, KB, 16, 4).transpose(0, 1, 3, 2, 4).reshape(E, N, KB * 4)


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


def _ws_view(layer, T, region, dtype, shape):
    r = moe.workspace_layout(T, layer.H, layer.E, layer.top_k, layer.I)
    off = getattr(r, region)
    nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    return layer.workspace(T)[off:off + nbytes].view(dtype).view(*shape)


def _check_h(gpu_hq, gpu_hs, ref_h, ref_hq, ref_hs, what):
    """h codes: equal to the oracle's, or inside the accumulation window (the device h may
    differ by H_EPS of its 1x128 group maximum); E8M0 codes equal except for blocks whose
    maximum is that close to a power of two."""
    I = ref_h.shape[1]
    hs_real, hs_pad = _split(gpu_hs, I)
    assert np.all(hs_pad == 127), what
    amax = np.abs(ref_h).reshape(ref_h.shape[0], -1, 32).max(axis=2)
    eps = (H_EPS * _group128_max(ref_h)).reshape(ref_h.shape[0], -1, 32).max(axis=2)
    edge_lo = np.ldexp(1.0, ref_hs.astype(int) - 127 + 8)
    near = (np.abs(amax - edge_lo) <= eps) | (np.abs(amax - 2 * edge_lo) <= eps)
    bad_scale = (hs_real != ref_hs) & ~near
    say(f"  {what}: h scale codes differing {int((hs_real != ref_hs).sum())} "
        f"(outside the window: {int(bad_scale.sum())}) of {ref_hs.size}")
    assert not bad_scale.any()
    same_scale = np.repeat(hs_real == ref_hs, 32, axis=1)[:, :I]
    s = np.ldexp(1.0, np.repeat(ref_hs.astype(int) - 127, 32, axis=1)[:, :I])
    e = H_EPS * _group128_max(ref_h)
    lo = R.e4m3_decode(R.e4m3_encode(((ref_h - e) / s).astype(np.float32)))
    hi = R.e4m3_decode(R.e4m3_encode(((ref_h + e) / s).astype(np.float32)))
    g = R.e4m3_decode(gpu_hq)
    ok = ~same_scale | ((g >= lo) & (g <= hi))
    diff = (gpu_hq != ref_hq) & same_scale
    say(f"  {what}: h codes differing {int(diff.sum())} of {diff.size}; all within the window: "
        f"{bool(ok.all())}")
    assert ok.all()
    return int(diff.sum()), diff.size


@pytest.mark.parametrize("shape", SMALL, ids=[s.name for s in SMALL])
def test_forward_mx_small_full_parity(shape):
    g = GpuLayer(shape, fmt=FMT)
    routing = moe.new_routing(shape.T, shape.E, shape.top_k)
    say(f"mx forward {shape.name}: T={shape.T} H={shape.H} E={shape.E} k={shape.top_k} I={shape.I}")
    out = g.layer(g.x, routing=routing)
    torch.cuda.synchronize()
    ox = OracleExperts(shape, g.li, fmt=FMT)
    ref = ox.forward()
    routing_exact(routing, ref, shape.T, shape.top_k, shape.name)
    T, H, I, rows = shape.T, shape.H, shape.I, shape.T * shape.top_k
    # x codes and scales (quantised inside the router kernel): bit-exact, pads 127
    xq = _ws_view(g.layer, T, "xq", torch.uint8, (T, H)).cpu().numpy()
    sx = _ws_view(g.layer, T, "sx", torch.uint8, (T, moe.mx_row(H))).cpu().numpy()
    real, pad = _split(sx, H)
    assert np.array_equal(xq, ref["xq"]) and np.array_equal(real, ref["sx"]) and np.all(pad == 127)
    # h (routed rows in dispatch order) against the oracle's experts on the same rows
    hq = _ws_view(g.layer, T, "h", torch.uint8, (rows, I)).cpu().numpy()
    hs = _ws_view(g.layer, T, "sh", torch.uint8, (rows, moe.mx_row(I))).cpu().numpy()
    _check_h_dispatched(g, ox, ref, hq, hs)
    compare_out(bits_host(out), ref["out"], shape.name, allowance=ref["allowance"])


def _check_h_dispatched(g, ox, ref, hq, hs, fmt=FMT):
    """The oracle's h per routed row in dispatch order (expert segments of perm)."""
    shape, li = g.shape, g.li
    x32 = R.bf16_to_f64(li.x).astype(np.float32)
    xd = R.dequantize_mx(*R.quantize_mx(x32))
    tok = ref["perm"] // shape.top_k
    ndiff = n = 0
    for e in range(shape.E):
        p0, p1 = ref["offsets"][e], ref["offsets"][e + 1]
        if p1 == p0:
            continue
        c13, s13, c2, s2 = ox.cache[e]
        _, rq, rs, h64 = R.expert_ffn(xd[tok[p0:p1]], c13, s13, li.b13[e], c2, s2, li.b2[e],
                                      shape.I, fmt)
        d, m = _check_h(hq[p0:p1], hs[p0:p1], h64, rq, rs, f"expert {e}")
        ndiff, n = ndiff + d, n + m
    say(f"  h codes differing over the layer: {ndiff} of {n}")
    assert ndiff <= 0.01 * n


@pytest.mark.timeout(900)
def test_forward_mx_decode_layer_all_tokens():
    shape = SHAPES["gpt-oss-20b-decode"]
    g = GpuLayer(shape, fmt=FMT)
    routing = moe.new_routing(shape.T, shape.E, shape.top_k)
    say(f"mx forward {shape.name}")
    out = g.layer(g.x, routing=routing)
    torch.cuda.synchronize()
    ref = OracleExperts(shape, g.li, fmt=FMT).forward()
    routing_exact(routing, ref, shape.T, shape.top_k, shape.name)
    compare_out(bits_host(out), ref["out"], shape.name, allowance=ref["allowance"])


@pytest.mark.timeout(1200)
def test_forward_mx_prefill_layer_sampled():
    shape = SHAPES["gpt-oss-120b-prefill"]
    g = GpuLayer(shape, fmt=FMT)
    routing = moe.new_routing(shape.T, shape.E, shape.top_k)
    say(f"mx forward {shape.name}")
    out = g.layer(g.x, routing=routing)
    torch.cuda.synchronize()
    rng = np.random.default_rng(98)
    toks = np.sort(rng.choice(shape.T, size=8, replace=False))
    toks[-1] = shape.T - 1
    ref = OracleExperts(shape, g.li, fmt=FMT).forward(token_subset=toks)
    routing_exact(routing, ref, shape.T, shape.top_k, shape.name)
    compare_out(bits_host(out)[toks], ref["out"], f"{shape.name} tokens {toks.tolist()}",
                allowance=ref["allowance"])


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
    xq = _ws_view(g.layer, shape.T, "xq", torch.uint8, (shape.T, shape.H))
    sx = _ws_view(g.layer, shape.T, "sx", torch.uint8, (shape.T, moe.mx_row(shape.H)))
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
