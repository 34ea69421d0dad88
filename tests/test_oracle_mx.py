"""Pins of the oracle's MXFP8 variant ("Hosting Qwen on Blackwell", section
"Quantization": the weights converted statically to MXFP8).  The pages name the format
only; its definition is the OCP Microscaling one (32-element blocks along K, a shared
E8M0 power-of-two scale, e4m3 elements).  The pages print no MXFP8 values, so the rule
is pinned by an integer search for the exponent, the error bound of the e4m3 rounding,
exact round trips, invariances and an independent scalar evaluation of the layer.
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


def floor_log2(a: float) -> int:
    """Largest n with 2^n <= a (a > 0), by search over integers."""
    n = 0
    while math.ldexp(1.0, n) > a:
        n -= 1
    while math.ldexp(1.0, n + 1) <= a:
        n += 1
    return n


def scalar_mx_block(vals32):
    """MXFP8 of one 32-block with scalar loops: (codes, scale code, dequantised values)."""
    amax = max(abs(float(v)) for v in vals32)
    X = 0 if amax == 0 else min(127, max(-127, floor_log2(amax) - 8))
    codes, deq = [], []
    for v in vals32:
        u = min(abs(float(v)) * math.ldexp(1.0, -X), 448.0)
        d = np.abs(TABLE[POS] - u)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if best.size == 1 else int([b for b in best if b % 2 == 0][0])
        neg = math.copysign(1.0, float(v)) < 0
        codes.append(c | (0x80 if neg else 0))
        deq.append((-1.0 if neg else 1.0) * TABLE[c] * math.ldexp(1.0, X))
    return codes, X + 127, deq


def _spacing(val):
    a = np.abs(val)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.ldexp(1.0, (e - 3).astype(int))


def _wide_rows(rng, R_, K):
    """Rows whose 32-blocks span many binades (tiny, normal and huge blocks)."""
    a = rng.standard_normal((R_, K))
    a *= np.exp2(rng.integers(-40, 40, size=(R_, K // 32))).repeat(32, axis=1)
    return a.astype(np.float32)


def test_scale_is_floor_log2_amax_minus_8():
    rng = np.random.default_rng(1)
    a = _wide_rows(rng, 40, 256)
    _, s = R.quantize_mx(a)
    blocks = a.reshape(40, 8, 32)
    for i in range(40):
        for j in range(8):
            amax = float(np.abs(blocks[i, j]).max())
            assert s[i, j] == min(127, max(-127, floor_log2(amax) - 8)) + 127


def test_scale_clamps_at_the_e8m0_range():
    a = np.zeros((3, 32), np.float32)
    a[0, 0] = 2.0 ** -140            # floor(log2) - 8 = -148 -> -127
    a[1, 0] = np.float32(3.0e38)     # 2^127 range: exponent 127 - 8 = 119 (no clamp)
    a[2, 5] = -1.0                   # exponent -8
    q, s = R.quantize_mx(a)
    assert list(s[:, 0]) == [0, 119 + 127, 119]
    assert R.e4m3_decode(q[2:3, 5])[0] == -256.0


def test_elements_within_half_spacing_or_clamped():
    rng = np.random.default_rng(2)
    a = _wide_rows(rng, 64, 512)
    q, s = R.quantize_mx(a)
    X = (s.astype(np.int64) - 127).repeat(32, axis=1)
    u = a.astype(np.float64) * np.ldexp(1.0, -X)          # the scaled value, exact
    d = R.e4m3_decode(q)
    clamped = np.abs(u) > 448
    assert np.all(np.abs(d[clamped]) == 448.0)
    assert np.all(np.sign(d[clamped]) == np.sign(u[clamped]))
    ok = ~clamped
    assert np.all(np.abs(u[ok] - d[ok]) <= 0.5 * _spacing(d[ok]) + 1e-300)


def test_block_maximum_lands_in_256_448():
    rng = np.random.default_rng(3)
    a = _wide_rows(rng, 32, 256)
    q, _ = R.quantize_mx(a)
    mx = np.abs(R.e4m3_decode(q)).reshape(32, 8, 32).max(axis=-1)
    assert np.all((mx >= 256) & (mx <= 448))


def test_zero_block_codes_and_unit_scale():
    a = np.zeros((2, 64), np.float32)
    a[1, 40] = 0.5
    q, s = R.quantize_mx(a)
    assert not q[0].any() and list(s[0]) == [127, 127]
    assert s[1, 0] == 127 and not q[1, :32].any()


def test_power_of_two_scaling_shifts_only_the_scale():
    rng = np.random.default_rng(4)
    a = (rng.standard_normal((8, 128)) * 0.03).astype(np.float32)
    q0, s0 = R.quantize_mx(a)
    for m in (-5, 3, 17):
        q1, s1 = R.quantize_mx((a * np.float32(2.0 ** m)).astype(np.float32))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1.astype(int), s0.astype(int) + m)


def test_exact_round_trip():
    # values decode(c) 2^X with the block maximum in [256, 448] come back unchanged
    rng = np.random.default_rng(5)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    codes = rng.choice(finite, size=(16, 96)).astype(np.uint8)
    big = rng.choice(np.array([c for c in range(0x78, 0x7F)]), size=(16, 3))   # 256 .. 448
    for j in range(3):
        codes[np.arange(16), 32 * j + 7] = big[:, j] | (0x80 * (j % 2))
    X = rng.integers(-100, 100, size=(16, 3))
    vals = R.e4m3_decode(codes) * np.ldexp(1.0, X).repeat(32, axis=1)
    q, s = R.quantize_mx(vals.astype(np.float32))
    assert np.array_equal(s.astype(int), X + 127)
    assert np.array_equal(R.e4m3_decode(q), R.e4m3_decode(codes))


@pytest.mark.parametrize("shape", [(3, 32), (5, 96), (2, 192)])
def test_matches_scalar_quantiser(shape):
    rng = np.random.default_rng(6)
    a = _wide_rows(rng, shape[0], shape[1])
    a[0, :32] = 0.0
    # block 0 of the last row: amax 1 (X = -8); after scaling by 2^8 two elements sit
    # exactly halfway between codes: 1.0625 -> 1.0 (0x38) and 17 -> 16 (0x58), the even ones
    a[-1, :32] = np.float32(2.0 ** -12)
    a[-1, 0] = 1.0
    a[-1, 3] = np.float32(1.0625 * 2.0 ** -8)
    a[-1, 4] = np.float32(17.0 * 2.0 ** -8)
    q, s = R.quantize_mx(a)
    assert s[-1, 0] == 127 - 8 and q[-1, 3] == 0x38 and q[-1, 4] == 0x58
    for i in range(shape[0]):
        for j in range(shape[1] // 32):
            codes, sc, deq = scalar_mx_block(a[i, 32 * j:32 * j + 32])
            assert s[i, j] == sc
            assert list(q[i, 32 * j:32 * j + 32]) == codes
            assert np.array_equal(R.dequantize_mx(q[i:i + 1, 32 * j:32 * j + 32], s[i:i + 1, j:j + 1])[0],
                                  np.array(deq))


def test_dense_e1_k1_layer_equals_scalar_mx_ffn():
    """E = 1, k = 1: the oracle's MXFP8 layer equals a dense biased SwiGLU FFN whose x, w13,
    h and w2 are quantised block by block with the scalar MX quantiser."""
    T, H, I = 5, 96, 64
    rng = np.random.default_rng(7)
    x_bits = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    W = (rng.standard_normal((1, H)) * 0.05).astype(np.float32)
    b = np.zeros(1, np.float32)
    w13 = (rng.standard_normal((1, 2 * I, H)) * 0.02).astype(np.float32)
    w2 = (rng.standard_normal((1, H, I)) * 0.02).astype(np.float32)
    b13 = f32_to_bf16_bits((rng.standard_normal((1, 2 * I)) * 0.01).astype(np.float32))
    b2 = f32_to_bf16_bits((rng.standard_normal((1, H)) * 0.01).astype(np.float32))
    c13, s13 = R.quantize_mx(w13)
    c2, s2 = R.quantize_mx(w2)
    got = R.forward(x_bits, W, b, 1, I, c13, s13, b13, c2, s2, b2, fmt="mxfp8")
    assert np.all(got["gates"] == 1.0)

    def deq_rows(m):
        return np.array([sum((scalar_mx_block(r[c:c + 32])[2] for c in range(0, len(r), 32)), [])
                         for r in m])

    x = bf16_bits_to_f32(x_bits)
    xd = deq_rows(x)
    W13 = deq_rows(w13[0])
    W2 = deq_rows(w2[0])
    C = xd @ W13.T + bf16_bits_to_f32(b13[0])
    hh = (C[:, :I] / (1 + np.exp(-C[:, :I])) * C[:, I:]).astype(np.float32)
    ref = deq_rows(hh) @ W2.T + bf16_bits_to_f32(b2[0])
    assert np.allclose(got["out"], ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------------------
# MXFP4 expert weights ("GPT-OSS on day 0": the checkpoints ship with MXFP4 expert weights):
# e2m1 elements (sign, 2 exponent bits with bias 1, 1 mantissa bit) in OCP MX blocks of 32
# along K with E8M0 scales, two codes per byte (element 2j in the low nibble).
# ---------------------------------------------------------------------------------------

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table():
    want = E2M1 + [-v for v in E2M1]
    got = R.e2m1_decode(np.arange(16))
    assert np.array_equal(got, np.array(want))
    assert np.signbit(got[8])                      # code 8 is negative zero


def _brute_e2m1(v: float) -> int:
    a = min(abs(v), 6.0)
    d = [abs(a - t) for t in E2M1]
    best = [i for i, x in enumerate(d) if x == min(d)]
    c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
    return c | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_encoder_matches_brute_force():
    v = np.concatenate([np.linspace(-7.5, 7.5, 6001), np.array(E2M1) + 0.0,
                        [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.0, 1e9, -1e9]])
    assert [int(c) for c in R.e2m1_encode(v)] == [_brute_e2m1(float(x)) for x in v]


def test_e2m1_ties_to_even_and_clamp():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 100.0, -0.25, -5.0])
    assert list(R.e2m1_encode(v)) == [0, 2, 2, 4, 4, 6, 6, 7, 7, 8, 14]


def scalar_mxfp4_block(vals32):
    amax = max(abs(float(v)) for v in vals32)
    X = 0 if amax == 0 else min(127, max(-127, floor_log2(amax) - 2))
    codes = [_brute_e2m1(float(v) * math.ldexp(1.0, -X)) for v in vals32]
    deq = [R.e2m1_decode(np.array([c]))[0] * math.ldexp(1.0, X) for c in codes]
    return codes, X + 127, deq


@pytest.mark.parametrize("shape", [(3, 32), (4, 128), (2, 192)])
def test_mxfp4_matches_scalar_quantiser_and_packing(shape):
    rng = np.random.default_rng(8)
    a = _wide_rows(rng, shape[0], shape[1])
    a[0, :32] = 0.0
    packed, s = R.quantize_mxfp4(a)
    assert packed.shape == (shape[0], shape[1] // 2)
    codes = R.unpack_e2m1(packed)
    for i in range(shape[0]):
        for j in range(shape[1] // 32):
            c, sc, deq = scalar_mxfp4_block(a[i, 32 * j:32 * j + 32])
            assert s[i, j] == sc
            assert list(codes[i, 32 * j:32 * j + 32]) == c
            assert np.array_equal(R.dequantize_mxfp4(packed[i:i + 1, 16 * j:16 * j + 16], s[i:i + 1, j:j + 1])[0],
                                  np.array(deq))
    # packing: element 2j in the low nibble of byte j
    assert np.array_equal(packed & 15, codes[:, 0::2]) and np.array_equal(packed >> 4, codes[:, 1::2])


def test_mxfp4_scale_rule_and_bounds():
    rng = np.random.default_rng(9)
    a = _wide_rows(rng, 48, 256)
    packed, s = R.quantize_mxfp4(a)
    blocks = a.reshape(48, 8, 32)
    X = s.astype(np.int64) - 127
    for i in range(48):
        for j in range(8):
            amax = float(np.abs(blocks[i, j]).max())
            assert X[i, j] == min(127, max(-127, floor_log2(amax) - 2))
    u = a.astype(np.float64) * np.ldexp(1.0, -np.repeat(X, 32, axis=1))   # in [-8, 8)
    d = R.e2m1_decode(R.unpack_e2m1(packed))
    clamped = np.abs(u) > 6
    assert np.all(np.abs(d[clamped]) == 6.0)
    # spacing of e2m1 at the decoded value: 0.5 below 2, 1 in [2, 4), 2 in [4, 6]
    sp = np.where(np.abs(d) < 2, 0.5, np.where(np.abs(d) < 4, 1.0, 2.0))
    ok = ~clamped
    assert np.all(np.abs(u[ok] - d[ok]) <= 0.5 * sp[ok])
    mx = np.abs(d).reshape(48, 8, 32).max(axis=-1)
    assert np.all((mx == 4.0) | (mx == 6.0))       # the block maximum lands in [4, 8)


def test_mxfp4_round_trip_and_power_of_two():
    rng = np.random.default_rng(10)
    codes = rng.integers(0, 16, size=(8, 64)).astype(np.uint8)
    codes[:, 5] = 7                                   # each block holds a 6
    codes[:, 37] = 15
    X = rng.integers(-60, 60, size=(8, 2))
    vals = R.e2m1_decode(codes) * np.ldexp(1.0, X).repeat(32, axis=1)
    packed, s = R.quantize_mxfp4(vals.astype(np.float32))
    assert np.array_equal(s.astype(int), X + 127)
    assert np.array_equal(R.e2m1_decode(R.unpack_e2m1(packed)), R.e2m1_decode(codes))
    a = (rng.standard_normal((4, 96)) * 0.02).astype(np.float32)
    p0, s0 = R.quantize_mxfp4(a)
    p1, s1 = R.quantize_mxfp4((a * np.float32(2.0 ** 9)).astype(np.float32))
    assert np.array_equal(p0, p1) and np.array_equal(s1.astype(int), s0.astype(int) + 9)


def test_dense_e1_k1_layer_mxfp4_weights_equals_scalar_ffn():
    T, H, I = 4, 64, 64
    rng = np.random.default_rng(11)
    x_bits = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    W = (rng.standard_normal((1, H)) * 0.05).astype(np.float32)
    b = np.zeros(1, np.float32)
    w13 = (rng.standard_normal((1, 2 * I, H)) * 0.02).astype(np.float32)
    w2 = (rng.standard_normal((1, H, I)) * 0.02).astype(np.float32)
    b13 = f32_to_bf16_bits((rng.standard_normal((1, 2 * I)) * 0.01).astype(np.float32))
    b2 = f32_to_bf16_bits((rng.standard_normal((1, H)) * 0.01).astype(np.float32))
    c13, s13 = R.quantize_mxfp4(w13)
    c2, s2 = R.quantize_mxfp4(w2)
    got = R.forward(x_bits, W, b, 1, I, c13, s13, b13, c2, s2, b2, fmt="mxfp4")

    def deq8(m):
        return np.array([sum((scalar_mx_block(r[c:c + 32])[2] for c in range(0, len(r), 32)), [])
                         for r in m])

    def deq4(m):
        return np.array([sum((scalar_mxfp4_block(r[c:c + 32])[2] for c in range(0, len(r), 32)), [])
                         for r in m])

    xd = deq8(bf16_bits_to_f32(x_bits))
    C = xd @ deq4(w13[0]).T + bf16_bits_to_f32(b13[0])
    hh = (C[:, :I] / (1 + np.exp(-C[:, :I])) * C[:, I:]).astype(np.float32)
    ref = deq8(hh) @ deq4(w2[0]).T + bf16_bits_to_f32(b2[0])
    assert np.allclose(got["out"], ref, rtol=1e-10, atol=1e-12)
