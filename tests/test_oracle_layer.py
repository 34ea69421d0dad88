"""Pins of the oracle's whole layer (router -> top-k softmax -> biased SwiGLU experts on
FP8 block-scaled weights -> gate-weighted combine).

"GPT-OSS on day 0", section "On Hopper": SwiGLU experts, softmax after top-k,
experts with biases, FP8 128x128 block scaling; section "Kernels -> MoE": bias in
the GEMM accumulator, weighted combine.  The pages print no worked example of
the layer, so the float results are pinned by an independent scalar per-token
evaluation, closed-form special cases and invariances.
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from synth import f32_to_bf16_bits, bf16_bits_to_f32

TABLE = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn) \
    .to(torch.float64).numpy()
POS = np.arange(0, 0x7F)


def nearest_code(v):
    """Scalar brute-force nearest e4m3 code (ties -> even), independent of the oracle."""
    a = min(abs(float(v)), 448.0)
    d = np.abs(TABLE[POS] - a)
    best = np.flatnonzero(d == d.min())
    c = int(best[0]) if best.size == 1 else int([b for b in best if b % 2 == 0][0])
    return c | (0x80 if math.copysign(1.0, float(v)) < 0 else 0)


def scalar_quant_dequant_row(vals32, group=128):
    """Quantise a float32 row in 1 x group blocks and return the dequantised float64 values."""
    out = []
    for g0 in range(0, len(vals32), group):
        grp = vals32[g0:g0 + group]
        amax = np.float32(max(abs(float(v)) for v in grp))
        s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
        for v in grp:
            out.append(TABLE[nearest_code(np.float32(v) / s)] * float(s))
    return out


def scalar_quant_dequant_matrix(w32):
    """128x128 block quantisation of a float32 matrix, dequantised (vectorised brute force)."""
    N, K = w32.shape
    out = np.zeros((N, K))
    pos_vals = TABLE[POS]
    for r0 in range(0, N, 128):
        for c0 in range(0, K, 128):
            blk = w32[r0:r0 + 128, c0:c0 + 128]
            amax = np.float32(np.abs(blk).max())
            s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
            v = np.minimum(np.abs((blk / s).astype(np.float64)), 448.0)
            d = np.abs(v[..., None] - pos_vals)
            m = d.min(-1, keepdims=True)
            cand = (d == m)
            # ties -> even code: prefer even indices among equal distances
            even_pref = np.where(cand & (POS % 2 == 0), 1, 0) + np.where(cand, 1, 0)
            code = np.argmax(even_pref, axis=-1)
            mag = pos_vals[code]
            out[r0:r0 + 128, c0:c0 + 128] = np.where(blk < 0, -mag, mag) * float(s)
    return out


def silu(z):
    return z / (1.0 + math.exp(-z))


def brute_force_layer(x_bits, W, b, k, I, w13, w2, b13_bits, b2_bits):
    """Per token, scalar loops: route, then run the selected experts, then sum."""
    T, H = x_bits.shape
    E = W.shape[0]
    x = bf16_bits_to_f32(x_bits)
    b13 = bf16_bits_to_f32(b13_bits).astype(np.float64)
    b2 = bf16_bits_to_f32(b2_bits).astype(np.float64)
    W13d = [scalar_quant_dequant_matrix(w13[e]) for e in range(E)]
    W2d = [scalar_quant_dequant_matrix(w2[e]) for e in range(E)]
    out = np.zeros((T, H))
    for t in range(T):
        logit = [sum(float(x[t, h]) * float(W[e, h]) for h in range(H)) + float(b[e])
                 for e in range(E)]
        sel = sorted(range(E), key=lambda e: (-logit[e], e))[:k]
        z = [math.exp(logit[e] - logit[sel[0]]) for e in sel]
        gates = [v / sum(z) for v in z]
        xd = scalar_quant_dequant_row(x[t].astype(np.float32))
        for g, e in zip(gates, sel):
            C = [sum(xd[h] * W13d[e][n, h] for h in range(H)) + b13[e, n] for n in range(2 * I)]
            hrow = np.array([silu(C[i]) * C[I + i] for i in range(I)]).astype(np.float32)
            hd = scalar_quant_dequant_row(hrow)
            for c in range(H):
                y = sum(hd[i] * W2d[e][c, i] for i in range(I)) + b2[e, c]
                out[t, c] += g * y
    return out


def make_small(T, H, E, k, I, seed, expert_bias=True):
    rng = np.random.default_rng(seed)
    x_bits = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    W = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(E) * 0.01).astype(np.float32)
    w13 = (rng.standard_normal((E, 2 * I, H)) * 0.02).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float32)
    sc = 0.01 if expert_bias else 0.0
    b13 = f32_to_bf16_bits((rng.standard_normal((E, 2 * I)) * sc).astype(np.float32))
    b2 = f32_to_bf16_bits((rng.standard_normal((E, H)) * sc).astype(np.float32))
    return x_bits, W, b, w13, w2, b13, b2


def oracle_forward(x_bits, W, b, k, I, w13, w2, b13, b2, dispatched=False, **kw):
    c13, s13 = R.quantize_blocks(w13)
    c2, s2 = R.quantize_blocks(w2)
    f = R.forward_dispatched if dispatched else R.forward
    return f(x_bits, W, b, k, I, c13, s13, b13, c2, s2, b2, **kw)


@pytest.mark.parametrize("dispatched", [False, True])
def test_layer_matches_scalar_brute_force(dispatched):
    # H = I = 192: ragged 64-wide blocks along K and N; w13 row-block 1 straddles gate/up
    T, H, E, k, I = 6, 192, 5, 2, 192
    args = make_small(T, H, E, k, I, seed=11)
    got = oracle_forward(*args[:3], k, I, *args[3:], dispatched=dispatched)["out"]
    ref = brute_force_layer(args[0], args[1], args[2], k, I, args[3], args[4], args[5], args[6])
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_dense_e1_k1_equals_biased_swiglu_ffn():
    T, H, E, k, I = 9, 256, 1, 1, 128
    x_bits, W, b, w13, w2, b13, b2 = make_small(T, H, E, k, I, seed=12)
    got = oracle_forward(x_bits, W, b, k, I, w13, w2, b13, b2)
    assert np.all(got["gates"] == 1.0)
    x = bf16_bits_to_f32(x_bits)
    xd = np.array([scalar_quant_dequant_row(x[t]) for t in range(T)])
    W13 = scalar_quant_dequant_matrix(w13[0])
    W2 = scalar_quant_dequant_matrix(w2[0])
    C = xd @ W13.T + bf16_bits_to_f32(b13[0])
    hh = (C[:, :I] / (1 + np.exp(-C[:, :I])) * C[:, I:]).astype(np.float32)
    hd = np.array([scalar_quant_dequant_row(r) for r in hh])
    ref = hd @ W2.T + bf16_bits_to_f32(b2[0])
    assert np.allclose(got["out"], ref, rtol=1e-10, atol=1e-12)


def test_zero_expert_weights_give_bias_only_output():
    T, H, E, k, I = 12, 128, 6, 3, 64
    x_bits, W, b, w13, w2, b13, b2 = make_small(T, H, E, k, I, seed=13)
    w13[:] = 0
    w2[:] = 0
    got = oracle_forward(x_bits, W, b, k, I, w13, w2, b13, b2)
    b2f = bf16_bits_to_f32(b2).astype(np.float64)
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            ref[t] += got["gates"][t, j] * b2f[got["ids"][t, j]]
    assert np.allclose(got["out"], ref, rtol=1e-14, atol=0)


def test_b2_linearity():
    T, H, E, k, I = 10, 128, 4, 2, 128
    x_bits, W, b, w13, w2, b13, b2 = make_small(T, H, E, k, I, seed=14)
    with_b2 = oracle_forward(x_bits, W, b, k, I, w13, w2, b13, b2)
    no_b2 = oracle_forward(x_bits, W, b, k, I, w13, w2, b13, np.zeros_like(b2))
    b2f = bf16_bits_to_f32(b2).astype(np.float64)
    delta = np.einsum("tk,tkh->th", with_b2["gates"], b2f[with_b2["ids"]])
    assert np.allclose(with_b2["out"] - no_b2["out"], delta, rtol=1e-9, atol=1e-12)


def test_token_permutation_invariance():
    T, H, E, k, I = 16, 256, 8, 2, 256
    x_bits, W, b, w13, w2, b13, b2 = make_small(T, H, E, k, I, seed=15)
    a = oracle_forward(x_bits, W, b, k, I, w13, w2, b13, b2)
    p = np.random.default_rng(0).permutation(T)
    c = oracle_forward(x_bits[p], W, b, k, I, w13, w2, b13, b2)
    assert np.allclose(c["out"], a["out"][p], rtol=1e-12, atol=1e-15)
    assert np.array_equal(c["ids"], a["ids"][p])


def test_expert_relabelling_invariance():
    T, H, E, k, I = 16, 128, 6, 3, 128
    x_bits, W, b, w13, w2, b13, b2 = make_small(T, H, E, k, I, seed=16)
    a = oracle_forward(x_bits, W, b, k, I, w13, w2, b13, b2)
    q = np.random.default_rng(1).permutation(E)        # new label i holds old expert q[i]
    c = oracle_forward(x_bits, W[q], b[q], k, I, w13[q], w2[q], b13[q], b2[q])
    assert np.allclose(c["out"], a["out"], rtol=1e-12, atol=1e-15)
    assert np.array_equal(q[c["ids"]], a["ids"])


def test_token_subset_equals_full():
    T, H, E, k, I = 20, 256, 8, 2, 128
    args = make_small(T, H, E, k, I, seed=17)
    full = oracle_forward(*args[:3], k, I, *args[3:])
    sub = [3, 0, 19, 7]
    part = oracle_forward(*args[:3], k, I, *args[3:], token_subset=sub)
    assert np.allclose(part["out"], full["out"][sub], rtol=1e-12, atol=1e-15)
    disp = oracle_forward(*args[:3], k, I, *args[3:], dispatched=True)
    assert np.allclose(disp["out"], full["out"], rtol=1e-12, atol=1e-15)
