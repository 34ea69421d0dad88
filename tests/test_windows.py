"""CPU pins of the analytic parity windows (tests/windows.py) that the GPU tests apply.

A window must hold every result an fp32 evaluation of the layer's definition can give
(checked here against fp32 emulations in NumPy, in several orders) and must still
reject the plausible mistakes of a kernel (a wrong code, a wrong scale, gate and up
swapped, a dropped bias, a wrong accumulation) -- planted in oracle-side data on the CPU.
"""
import numpy as np
import pytest

from oracle import moe_ref as R
import windows as W
from layouts import pad_scale_rows, tile_fp4, tile_scales, untile_fp4, untile_scales


def _quantised_operands(rng, R_, N, K):
    x32 = rng.standard_normal((R_, K)).astype(np.float32)
    w32 = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    xq, sx = R.quantize_activations(x32)
    wq, sw = R.quantize_blocks(w32)
    return xq, sx, wq, sw


def _fp32_blocked(xq, sx, wq, sw, order="forward"):
    """fp32 emulation of the block-scaled GEMM: per 128-K block an fp32 sum of the code
    products (in the given order), promoted by one fp32 multiply-add with fp32(sa sb)."""
    R_, K = xq.shape
    N = wq.shape[0]
    a = R.e4m3_decode(xq).astype(np.float32)
    b = R.e4m3_decode(wq).astype(np.float32)
    acc = np.zeros((R_, N), np.float32)
    for j in range(-(-K // 128)):
        ks = range(j * 128, min(K, j * 128 + 128))
        ks = list(ks)[::-1] if order == "reverse" else list(ks)
        p = np.zeros((R_, N), np.float32)
        for k in ks:
            p = (p + np.outer(a[:, k], b[:, k]).astype(np.float32)).astype(np.float32)
        s = (sx[:, j][:, None] * sw[np.arange(N) // 128, j][None, :]).astype(np.float32)
        acc = (acc + p * s).astype(np.float32)   # two roundings: inside the fma bound
    return acc


@pytest.mark.parametrize("order", ["forward", "reverse"])
def test_accumulation_bound_holds_for_fp32_evaluations(order):
    rng = np.random.default_rng(5)
    xq, sx, wq, sw = _quantised_operands(rng, 6, 40, 320)
    xd = R.dequantize_blocks(xq, sx, rows=1)
    wd = R.dequantize_blocks(wq, sw)
    exact = xd @ wd.T
    _, S, G = W.product_sums(xd, wd)
    bound = W.accumulation_bound(S, 320, G)
    err = np.abs(_fp32_blocked(xq, sx, wq, sw, order) - exact)
    assert np.all(err <= bound)
    assert err.max() > 0                       # the emulation does round
    # and the bound is not vacuous: a result missing one promoted block is far outside it
    wrong = _fp32_blocked(xq, sx, wq, sw, order) - (xd[:, :128] @ wd[:, :128].T)
    assert np.mean(np.abs(wrong - exact) > bound) > 0.9


def _layer_rows(rng, R_=12, H=256, I=192, bias=True):
    x32 = rng.standard_normal((R_, H)).astype(np.float32)
    xq, sx = R.quantize_activations(x32)
    xd = R.dequantize_blocks(xq, sx, rows=1)
    w13 = (rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32)
    c13, s13 = R.quantize_blocks(w13)
    W13 = R.dequantize_blocks(c13, s13)
    b13 = R.f64_to_bf16_bits(rng.standard_normal(2 * I) * 0.01 * bias)
    C, C_abs, C_gmax = W.product_sums(xd, W13)
    C += R.bf16_to_f64(b13)
    return C, (C_abs, C_gmax), H, I, xd, W13, b13


def _device_like_h(rng, C, C_abs, K, I, frac=0.999):
    """An fp32 evaluation: C perturbed inside its accumulation bound, SwiGLU in fp32."""
    dC = W.accumulation_bound(C_abs[0], K, C_abs[1])
    Cp = (C + frac * dC * rng.uniform(-1, 1, C.shape)).astype(np.float32)
    g, u = Cp[:, :I], Cp[:, I:]
    e = np.exp(-g).astype(np.float32)
    return (g * (np.float32(1) / (np.float32(1) + e)).astype(np.float32) * u).astype(np.float32)


def test_swiglu_window_contains_fp32_evaluations():
    rng = np.random.default_rng(7)
    C, C_abs, H, I, *_ = _layer_rows(rng)
    h, dh = W.swiglu_window(C, C_abs[0], H, I, C_abs[1])
    for _ in range(20):
        hd = _device_like_h(rng, C, C_abs, H, I)
        assert np.all(np.abs(hd - h) <= dh)
    # the window is narrow: a few per cent of the values' size, below one e4m3 step (1/8)
    assert np.median(dh / np.maximum(np.abs(h), 1e-30)) < 0.05


def _device_quantise(h32):
    """fp32 device-style 1x128 quantisation: scale fp32(amax / 448), codes of fp32(h / s)."""
    R_, I = h32.shape
    G = -(-I // 128)
    s = np.ones((R_, G), np.float32)
    q = np.zeros((R_, I), np.uint8)
    for gi in range(G):
        blk = h32[:, gi * 128:(gi + 1) * 128]
        amax = np.abs(blk).max(axis=1)
        s[:, gi] = np.where(amax > 0, amax / np.float32(448), np.float32(1))
        q[:, gi * 128:(gi + 1) * 128] = R.e4m3_encode((blk / s[:, gi:gi + 1]).astype(np.float32))
    return q, s


def test_block_h_check_accepts_fp32_quantisations():
    rng = np.random.default_rng(11)
    C, C_abs, H, I, *_ = _layer_rows(rng, R_=16, I=320)
    h, dh = W.swiglu_window(C, C_abs[0], H, I, C_abs[1])
    for trial in range(10):
        hd = _device_like_h(rng, C, C_abs, H, I)
        q, s = _device_quantise(hd)
        sok, cok, _ = W.block_h_check(h, dh, q, s)
        assert sok.all() and cok.all(), trial
    # the oracle's own quantisation of the exact h is inside too
    q0, s0 = R.quantize_activations(h.astype(np.float32))
    sok, cok, _ = W.block_h_check(h, dh, q0, s0)
    assert sok.all() and cok.all()


def test_block_h_check_rejects_plausible_mistakes():
    rng = np.random.default_rng(13)
    C, C_abs, H, I, xd, W13, b13 = _layer_rows(rng, R_=16, I=320)
    h, dh = W.swiglu_window(C, C_abs[0], H, I, C_abs[1])
    q0, s0 = R.quantize_activations(h.astype(np.float32))
    # one code step off (away from zero) on every element: the window admits one or two
    # codes around the exact quotient, so a uniform one-step error fails on a large share
    q1 = q0.copy()
    nz = (q0 & 0x7F) > 8
    q1[nz] = q0[nz] + 1
    assert np.mean(~W.block_h_check(h, dh, q1, s0)[1][nz]) > 0.3
    # a scale twice too large (codes of the right quotients for that scale)
    sok, _, _ = W.block_h_check(h, dh, q0, s0 * 2)
    assert not sok.any()
    # gate and up swapped
    hs = R.silu(C[:, I:]) * C[:, :I]
    qs, ss = R.quantize_activations(hs.astype(np.float32))
    sok, cok, _ = W.block_h_check(h, dh, qs, ss)
    assert (~sok).mean() > 0.9 and (~cok).mean() > 0.5
    # b13 dropped
    Cn = C - R.bf16_to_f64(b13)
    hn = R.silu(Cn[:, :I]) * Cn[:, I:]
    qn, sn = R.quantize_activations(hn.astype(np.float32))
    sok, cok, _ = W.block_h_check(h, dh, qn, sn)
    assert (~sok).mean() > 0.5 and (~cok).mean() > 0.3


def _device_quantise_mx(h32):
    q, c = R.quantize_mx(h32)          # the oracle's rule is the device's rule on fp32 h
    return q, c


def test_mx_h_check_accepts_fp32_and_rejects_mistakes():
    rng = np.random.default_rng(17)
    C, C_abs, H, I, *_ = _layer_rows(rng, R_=16, I=320)
    h, dh = W.swiglu_window(C, C_abs[0], H, I, C_abs[1])
    for _ in range(10):
        q, c = _device_quantise_mx(_device_like_h(rng, C, C_abs, H, I))
        sok, cok, _ = W.mx_h_check(h, dh, q, c)
        assert sok.all() and cok.all()
    q0, c0 = R.quantize_mx(h.astype(np.float32))
    sok, _, _ = W.mx_h_check(h, dh, q0, c0.astype(np.int64) + 1)
    assert (~sok).mean() > 0.9      # only blocks whose maximum lies near a power of two pass
    q1 = q0.copy()
    nz = (q0 & 0x7F) > 8
    q1[nz] += 1
    assert np.mean(~W.mx_h_check(h, dh, q1, c0)[1][nz]) > 0.3


def test_y_bound_holds_for_fp16_storage_and_rejects_errors():
    rng = np.random.default_rng(19)
    xq, sx, wq, sw = _quantised_operands(rng, 8, 64, 384)
    xd = R.dequantize_blocks(xq, sx, rows=1)
    wd = R.dequantize_blocks(wq, sw)
    b2 = R.bf16_to_f64(R.f64_to_bf16_bits(rng.standard_normal(64) * 0.01))
    y_ref, S, G = W.product_sums(xd, wd)
    y_ref += b2
    bound = W.y_bound(y_ref, S, 384, G)
    y16 = (_fp32_blocked(xq, sx, wq, sw) + b2.astype(np.float32)).astype(np.float16).astype(np.float64)
    assert np.all(np.abs(y16 - y_ref) <= bound)
    y_model = (_mma_group_model(xd, wd) + b2).astype(np.float16).astype(np.float64)
    assert np.all(np.abs(y_model - y_ref) <= bound)
    assert np.mean(np.abs(y16 * 1.03 - y_ref) > bound) > 0.5


def test_combine_bound_holds_and_rejects_swapped_gates():
    rng = np.random.default_rng(23)
    T, k, H = 20, 4, 96
    y = rng.standard_normal((T, k, H))
    dy = 2.0 ** -11 * np.abs(y)
    g = rng.dirichlet(np.ones(k), size=T)
    g32 = g.astype(np.float32)
    ydev = (y + dy * rng.uniform(-1, 1, y.shape)).astype(np.float16).astype(np.float32)
    acc = np.zeros((T, H), np.float32)
    for j in range(k):
        acc = (acc + g32[:, j:j + 1] * ydev[:, j]).astype(np.float32)
    out_ref = np.einsum("tk,tkh->th", g, y)
    out_dev = R.bf16_to_f64(R.f64_to_bf16_bits(acc.astype(np.float64)))
    dyb = dy + 2.0 ** -11 * (np.abs(y) + dy)
    bound = W.combine_bound(g, g32, y, dyb, out_ref)
    assert np.all(np.abs(out_dev - out_ref) <= bound)
    swapped = np.einsum("tk,tkh->th", g[:, ::-1], y)
    assert np.mean(np.abs(swapped - out_ref) > bound) > 0.9


def test_layouts_round_trip():
    rng = np.random.default_rng(29)
    E, N, K = 2, 48, 320
    codes = rng.integers(0, 255, (E, N, K // 32)).astype(np.uint8)
    rows = pad_scale_rows(codes, K)
    assert np.all(rows[..., K // 32:] == 127)
    assert np.array_equal(untile_scales(tile_scales(rows, N, K), N, K), rows)
    packed = rng.integers(0, 255, (E, N, K // 2)).astype(np.uint8)
    c, tail = untile_fp4(tile_fp4(packed, N, K), N, K)
    assert np.array_equal(c, packed) and np.all(tail == 0)


def _mma_group_model(a, b):
    """The matrix instruction's block sum on float64 operands [R, K] x [N, K] (K a multiple
    of 8): per group of 8 consecutive K, each product truncated toward zero to a multiple of
    2^(E - 13), E the exponent of the group's largest |product|; the group sums exact."""
    R_, K = a.shape
    out = np.zeros((R_, b.shape[0]))
    for g in range(K // 8):
        p = a[:, None, 8 * g:8 * g + 8] * b[None, :, 8 * g:8 * g + 8]
        M = np.abs(p).max(axis=2, keepdims=True)
        _, E = np.frexp(np.where(M > 0, M, 1.0))
        q = np.ldexp(1.0, E - 1 - 13)
        out += (np.sign(p) * np.floor(np.abs(p) / q) * q).sum(axis=2)
    return out


def test_accumulation_bound_covers_the_instruction_model():
    """The group-truncation model of the matrix instruction stays within the bound, on
    quantised Gaussian operands and on adversarial groups (one product 2^E, seven just
    below the 2^(E - 13) granule, so each loses almost a whole granule)."""
    rng = np.random.default_rng(31)
    xq, sx, wq, sw = _quantised_operands(rng, 8, 24, 384)
    a = R.dequantize_blocks(xq, sx, rows=1)
    b = R.dequantize_blocks(wq, sw)
    exact, S, G = W.product_sums(a, b)
    assert np.all(np.abs(_mma_group_model(a, b) - exact) <= W.accumulation_bound(S, 384, G))
    grp = np.array([1.0] + [2.0 ** -13 * (2 - 2.0 ** -3)] * 7)
    a = np.tile(grp, 16)[None, :]
    b = np.ones((1, 128))
    exact, S, G = W.product_sums(a, b)
    err = np.abs(_mma_group_model(a, b) - exact)
    bound = W.accumulation_bound(S, 128, G)
    assert err[0, 0] <= bound[0, 0] and err[0, 0] > 0.8 * bound[0, 0]   # the bound is tight here
