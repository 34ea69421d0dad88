"""Pins of the oracle's FP8 e4m3 codec and block quantiser.

The pages fix FP8 with 128x128 block scaling ("GPT-OSS on day 0", section "On
Hopper").  The e4m3 variant is read as OCP e4m3fn.  The codec is pinned to
torch's independent float8_e4m3fn implementation and to a brute-force
nearest-value search; the quantiser to its invariants and to an independent
scalar implementation.
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe_ref as R


def torch_decode_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_spot_values():
    d = R.e4m3_decode(np.array([0x38, 0x08, 0x01, 0x7E, 0x00, 0x80, 0xB8, 0xFE, 0x07, 0x40]))
    assert d[0] == 1.0
    assert d[1] == 2.0 ** -6
    assert d[2] == 2.0 ** -9
    assert d[3] == 448.0
    assert d[4] == 0.0 and not np.signbit(d[4])
    assert d[5] == 0.0 and np.signbit(d[5])
    assert d[6] == -1.0
    assert d[7] == -448.0
    assert d[8] == 7 * 2.0 ** -9          # largest subnormal
    assert d[9] == 2.0
    assert np.isnan(R.e4m3_decode(np.array([0x7F, 0xFF]))).all()


def test_decode_matches_torch_all_codes():
    ours = R.e4m3_decode(np.arange(256))
    ref = torch_decode_table()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def _brute_encode(v32):
    """Nearest finite code by exhaustive search; ties -> even code; sign kept."""
    table = torch_decode_table()
    pos_codes = np.arange(0, 0x7F)             # 0x00..0x7E finite non-negative
    pos_vals = table[pos_codes]
    out = np.empty(v32.shape, np.uint8)
    for i, v in enumerate(v32.astype(np.float64).ravel()):
        a = min(abs(v), 448.0)
        d = np.abs(pos_vals - a)
        best = np.flatnonzero(d == d.min())
        c = best[0] if best.size == 1 else [b for b in best if b % 2 == 0][0]
        out.ravel()[i] = c | (0x80 if math.copysign(1.0, v) < 0 else 0)
    return out


def _sweep_values():
    table = torch_decode_table()
    pos = np.sort(table[0:0x7F])
    mids = (pos[:-1] + pos[1:]) / 2
    base = np.concatenate([pos, mids, [448.0, 449.0, 460.0, 463.9, 464.0, 470.0, 1e6, 1e-12]])
    v = base.astype(np.float32)
    up = np.nextafter(v, np.float32(np.inf))
    dn = np.nextafter(v, np.float32(0))
    rng = np.random.default_rng(7)
    rnd = np.concatenate([rng.uniform(0, 448, 3000), np.exp(rng.uniform(-12, 6.1, 3000))]).astype(np.float32)
    allv = np.concatenate([v, up, dn, rnd])
    return np.concatenate([allv, -allv]).astype(np.float32)


def test_encode_matches_brute_force_nearest():
    v = _sweep_values()
    assert np.array_equal(R.e4m3_encode(v), _brute_encode(v))


def test_encode_ties_to_even():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): even code wins
    assert R.e4m3_encode(np.float32(1.0625)) == 0x38
    # 17 halfway between 16 (0x58) and 18 (0x59)
    assert R.e4m3_encode(np.float32(17.0)) == 0x58
    # 19 halfway between 18 (0x59) and 20 (0x5A) -> 0x5A
    assert R.e4m3_encode(np.float32(19.0)) == 0x5A
    # halfway between the two smallest subnormals 2^-9 and 2^-8 -> 2^-8 (0x02)
    assert R.e4m3_encode(np.float32(1.5 * 2 ** -9)) == 0x02
    # half of the smallest subnormal -> 0 ; negative -> negative zero
    assert R.e4m3_encode(np.float32(2 ** -10)) == 0x00
    assert R.e4m3_encode(np.float32(-(2 ** -10))) == 0x80


def test_encode_clamps_to_448():
    v = np.array([448.0, 460.0, 464.0, 1e30, -1e30], np.float32)
    assert list(R.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_encode_matches_torch_cast_in_range():
    v = _sweep_values()
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(R.e4m3_encode(v), ref)


# ---------------------------------------------------------------------------------------
# quantiser
# ---------------------------------------------------------------------------------------

def _spacing(val):
    a = np.abs(val)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.ldexp(1.0, (e - 3).astype(int))


@pytest.mark.parametrize("shape", [(256, 256), (192, 320), (2 * 96, 64)])
def test_block_quantiser_invariants(shape):
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    w[:128, :128] = 0.0                                   # an all-zero block
    codes, scales = R.quantize_blocks(w)
    N, K = shape
    assert scales.shape == (-(-N // 128), -(-K // 128))
    assert scales[0, 0] == 1.0 and not codes[:128, :128].any()
    d = R.e4m3_decode(codes)
    for i in range(scales.shape[0]):
        for j in range(scales.shape[1]):
            blk = np.s_[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            if np.abs(w[blk]).max() == 0:
                continue
            # the largest element of every non-zero block maps to +-448
            assert np.abs(d[blk]).max() == 448.0
            assert scales[i, j] == np.float32(np.abs(w[blk]).max() / np.float32(448))
            # reconstruction error within half a code spacing (plus fp32 division rounding)
            err = np.abs(w[blk].astype(np.float64) - d[blk] * scales[i, j])
            bound = scales[i, j] * (0.5 * _spacing(d[blk]) + 448 * 2.0 ** -23)
            assert (err <= bound).all()


def test_block_quantiser_power_of_two_equivariance():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((256, 192)) * 0.05).astype(np.float32)
    c1, s1 = R.quantize_blocks(w)
    c2, s2 = R.quantize_blocks(w * np.float32(8.0))
    assert np.array_equal(c1, c2)
    assert np.array_equal(s2, s1 * np.float32(8.0))


def _scalar_quantise_group(vals):
    """Independent scalar 1xG quantiser: amax -> fp32 scale -> brute-force nearest code."""
    amax = np.float32(max(abs(float(v)) for v in vals))
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    q = _brute_encode(np.array([np.float32(v) / s for v in vals], np.float32))
    return q, s


def test_activation_quantiser_matches_scalar_reference():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((5, 320)).astype(np.float32)    # groups 128, 128, 64 (ragged)
    a[2, 128:256] = 0.0
    codes, scales = R.quantize_activations(a)
    assert scales.shape == (5, 3)
    for r in range(5):
        for g in range(3):
            sl = slice(g * 128, min((g + 1) * 128, 320))
            q, s = _scalar_quantise_group(a[r, sl])
            assert scales[r, g] == s
            assert np.array_equal(codes[r, sl], q)


def test_batched_weight_quantiser_equals_per_matrix():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((3, 384, 192)) * 0.02).astype(np.float32)
    cb, sb = R.quantize_blocks(w)
    for e in range(3):
        c, s = R.quantize_blocks(w[e])
        assert np.array_equal(cb[e], c) and np.array_equal(sb[e], s)


def test_bf16_output_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.14159, 1e-3, 0.0])
    bits = R.f64_to_bf16_bits(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    # halfway cases go to even
    assert R.f64_to_bf16_bits(np.array([1.0 + 2 ** -8]))[0] == 0x3F80
    assert R.f64_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82
