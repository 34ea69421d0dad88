"""Plain, slow CPU oracle of the sparse MoE FFN layer (float64, NumPy).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the
HIP path (``sparse_moe_ffn_gemm_amd``) and never imports it; both sides receive
their inputs from ``synth``.

What the layer computes, and where the pages state it:

* "GPT-OSS on day 0", section "On Hopper" (the layer's feature list): the MLP is
  a sparse mixture of experts with SwiGLU experts; the expert weights come from
  a softmax taken *after* top-k; the experts carry biases.  The same page fixes
  FP8 with 128x128 block scaling as the weight quantisation scheme.
* same page, section "Kernels -> MoE": routing picks the top-k experts and takes
  the softmax over the selected logits only (unlike DeepSeek-style routers that
  softmax over all experts); the bias enters the grouped GEMM as the initial
  accumulator value, once per output tile.
* same page, "Kernels -> MoE" on dispatch/combine, and "Hosting Qwen on
  Blackwell", section "MoE Dispatch - Combine / Expert Parallel": dispatch
  aggregates routing information and gathers each expert's tokens into the
  GEMM input buffers; combine is the gate-weighted accumulation of the expert
  outputs per token.

Readings where the pages are silent:
  e4m3 is the OCP "fn" variant (bias 7, max 448, no infinities, 0x7F/0xFF NaN);
  a scale is fp32(amax / 448) (IEEE fp32 divide), 1.0 for an all-zero block, and
  a code is the nearest e4m3 value (ties to even) of fp32(v / s) clamped to
  +-448; blocks tile each [N, K] matrix from (0, 0) with ragged edge blocks;
  activations are quantised per token in 1x128 groups along K with the same
  rule; w13 rows [0, I) are the gate projection and rows [I, 2I) the up
  projection; SwiGLU is silu(gate) * up with silu(z) = z / (1 + e^-z); b13 is
  added before SwiGLU and b2 to each expert's output (so it is gate-weighted);
  top-k order is descending logit with ties to the lower expert index; the
  dispatch order is expert-major and token-ascending inside an expert.

MXFP8 variant ("Hosting Qwen on Blackwell", section "Quantization": weights
converted statically to MXFP8): the OCP Microscaling format -- blocks of 32
consecutive elements along K share a power-of-two scale, stored as an E8M0 code
(exponent + 127), exponent floor(log2(amax)) - 8 so that the block maximum lands in
[256, 512) before the e4m3 rounding (clamped to +-448); an all-zero block gets
exponent 0; the activations (x, h) use the same 1x32 blocks along K.

MXFP4 expert weights ("GPT-OSS on day 0": the checkpoints ship with MXFP4 expert weights):
the same OCP MX blocks with e2m1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6),
exponent floor(log2(amax)) - 2 (the block maximum lands in [4, 8) before the rounding,
clamped to +-6), two codes per byte with element 2j in the low nibble; x and h stay MXFP8.

Pins (tests/test_oracle_*.py): the e4m3 codec against its closed-form definition
and torch's float8_e4m3fn, a brute-force nearest-code encoder and an independent
scalar quantiser; router logits, top-k and gates against pure-Python loops and
sorted(); the permutation against bincount / identity; the whole layer against
a per-token brute-force evaluation written with scalar loops, a dense E=1, k=1
SwiGLU FFN, the zero-weight (bias-only) case, b2-linearity and the token- and
expert-relabelling invariances.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 128


# ----------------------------------------------------------------------------------------
# FP8 e4m3 (OCP "fn") codec
# ----------------------------------------------------------------------------------------

def _e4m3_value(c: np.ndarray) -> np.ndarray:
    """The OCP e4m3fn definition, for an array of codes (int64)."""
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


_E4M3_TABLE = _e4m3_value(np.arange(256, dtype=np.int64))


def e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3 code, float64.

    e = bits 6..3, m = bits 2..0:  e >= 1: (-1)^s 2^(e-7) (1 + m/8);  e == 0:
    (-1)^s 2^-6 (m/8);  magnitude code 0x7F is NaN (no infinities).  The definition
    is evaluated once for all 256 codes and then looked up.
    """
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def _encode_flat(v32: np.ndarray) -> np.ndarray:
    a = np.minimum(np.abs(v32.astype(np.float64)), E4M3_MAX)
    _, ex = np.frexp(a)                 # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)          # binade exponent (subnormal range uses -6)
    step = np.ldexp(1.0, e - 3)
    q = np.rint(a / step) * step        # a / step is exact (power-of-two step)
    # code of q
    _, qe = np.frexp(q)
    qe = qe - 1                          # q = (1 + frac) 2^qe for q >= 2^-6
    normal = q >= 2.0 ** -6
    mant = np.where(normal, np.rint((np.ldexp(q, -np.where(normal, qe, 0)) - 1.0) * 8.0), 0.0)
    code_n = ((qe + 7) << 3) + mant.astype(np.int64)
    code_s = np.rint(q / 2.0 ** -9).astype(np.int64)
    mag = np.where(normal, code_n, code_s)
    sign = np.signbit(v32).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8)


def e4m3_encode(v) -> np.ndarray:
    """Nearest e4m3 code (ties to the even code) of float32 values, after clamping to +-448.

    The spacing of e4m3 values in the binade [2^e, 2^(e+1)) is 2^(e-3); below 2^-6
    (subnormals) it is 2^-9.  Rounding |v| to a multiple of that spacing with
    round-half-even gives the nearest representable value; its code is then read
    off the definition (exponent field e+7, mantissa = fraction * 8).  The sign bit
    is kept (a negative value that rounds to zero gives 0x80).  Evaluated in slices
    of the flattened input only to bound the temporaries.
    """
    v32 = np.asarray(v, dtype=np.float32)
    if np.isnan(v32).any():
        raise ValueError("NaN has no defined code here")
    flat = v32.reshape(-1)
    out = np.empty(flat.shape, np.uint8)
    step = 1 << 18
    for i in range(0, flat.size, step):
        out[i:i + step] = _encode_flat(flat[i:i + step])
    return out.reshape(v32.shape)


# ----------------------------------------------------------------------------------------
# Block quantisation (weights 128x128, activations 1x128)
# ----------------------------------------------------------------------------------------

def quantize_blocks(w, rows: int = BLOCK, cols: int = BLOCK):
    """Quantise a float32 matrix [N, K] (or a batch [..., N, K]) in rows x cols blocks.

    Per block: a = max |w| (fp32);  s = fp32(a / 448) if a > 0 else 1;
    code = e4m3_encode(fp32(w / s)).  Edge blocks are partial: the matrix is padded
    with zeros to whole blocks (zeros change no block maximum) and the padding is
    dropped afterwards.  Returns (codes uint8 [..., N, K], scales float32
    [..., ceil(N/rows), ceil(K/cols)])."""
    w = np.asarray(w, dtype=np.float32)
    *lead, N, K = w.shape
    nb, kb = -(-N // rows), -(-K // cols)
    pad = np.zeros(tuple(lead) + (nb * rows, kb * cols), np.float32)
    pad[..., :N, :K] = w
    blocks = pad.reshape(tuple(lead) + (nb, rows, kb, cols))
    amax = np.abs(blocks).max(axis=(-3, -1))                       # [..., nb, kb]
    scales = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = blocks / scales[..., :, None, :, None]                      # fp32 / fp32 -> fp32
    codes = e4m3_encode(q).reshape(pad.shape)[..., :N, :K]
    return np.ascontiguousarray(codes), scales


def dequantize_blocks(codes, scales, rows: int = BLOCK, cols: int = BLOCK) -> np.ndarray:
    """decode(code) * scale of its block, float64."""
    vals = e4m3_decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    N, K = vals.shape[-2:]
    for i in range(s.shape[-2]):
        for j in range(s.shape[-1]):
            vals[..., i * rows:(i + 1) * rows, j * cols:(j + 1) * cols] *= s[..., i, j, None, None]
    return vals


def quantize_activations(a32):
    """Per-row 1x128 quantisation of a float32 [R, K] matrix: (codes, scales [R, ceil(K/128)])."""
    return quantize_blocks(np.asarray(a32, dtype=np.float32), rows=1, cols=BLOCK)


# ----------------------------------------------------------------------------------------
# MXFP8 (microscaling): "Hosting Qwen on Blackwell", section "Quantization" -- the
# weights converted statically to MXFP8.  The format is the OCP Microscaling one: a
# block of 32 consecutive elements along K shares one E8M0 scale (a power of two, code
# = exponent + 127); the elements are e4m3.
# ----------------------------------------------------------------------------------------

MX_BLOCK = 32
E4M3_EMAX = 8          # exponent of the largest normal e4m3 value (448 = 1.75 * 2^8)


def quantize_mx(a):
    """MXFP8 quantisation of a float32 array [..., K] along its last axis (K a multiple
    of 32).  Per block of 32: amax = max |v|; shared exponent X = floor(log2(amax)) - 8,
    clamped to [-127, 127] (X = 0 for an all-zero block); element code =
    e4m3_encode(v * 2^-X) (an exact power-of-two scaling, then clamped to +-448).
    Returns (codes uint8 [..., K], scale codes uint8 [..., K/32] = X + 127)."""
    a = np.asarray(a, dtype=np.float32)
    K = a.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = a.reshape(a.shape[:-1] + (K // MX_BLOCK, MX_BLOCK)).astype(np.float64)
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)                       # amax = m 2^ex, m in [0.5, 1)
    X = np.where(amax > 0, np.clip(ex - 1 - E4M3_EMAX, -127, 127), 0).astype(np.int64)
    scaled = blocks * np.ldexp(1.0, -X)[..., None]          # exact in float64
    codes = e4m3_encode(scaled.astype(np.float32)).reshape(a.shape)
    return codes, (X + 127).astype(np.uint8)


def dequantize_mx(codes, scales) -> np.ndarray:
    """decode(code) * 2^(scale code - 127) of its 32-block, float64."""
    vals = e4m3_decode(codes)
    K = vals.shape[-1]
    X = np.asarray(scales, np.int64) - 127
    v = vals.reshape(vals.shape[:-1] + (K // MX_BLOCK, MX_BLOCK)) * np.ldexp(1.0, X)[..., None]
    return v.reshape(vals.shape)


# ----------------------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def router_logits(x_bits, router_w, router_b) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] W[e, h] + b[e], float64 (x taken exactly from bf16)."""
    x = bf16_to_f64(x_bits)
    return x @ np.asarray(router_w, np.float64).T + np.asarray(router_b, np.float64)


def topk_softmax(logits, k: int):
    """Top-k experts per token (descending logit, ties -> lower index) and the softmax
    over the k selected logits only: g_j = exp(l_j - l_1) / sum_i exp(l_i - l_1)."""
    logits = np.asarray(logits, np.float64)
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    gates = z / z.sum(axis=1, keepdims=True)
    return ids, gates


def permute(ids, E: int):
    """Dispatch tables: counts[e], offsets (exclusive prefix sum, E+1 entries), perm[p] =
    t*k + j for the p-th routed row in expert-major, token-ascending order, and inv =
    the inverse of perm (inv[t*k + j] = p)."""
    ids = np.asarray(ids, np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int32)   # ties keep t*k+j order
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return counts, offsets, perm, inv


# ----------------------------------------------------------------------------------------
# Experts and combine
# ----------------------------------------------------------------------------------------

def silu(z):
    return z / (1.0 + np.exp(-z))


# ----------------------------------------------------------------------------------------
# MXFP4 expert weights ("GPT-OSS on day 0": the checkpoints ship with MXFP4 expert
# weights): OCP MX blocks of 32 along K, E8M0 scales, e2m1 elements (sign, 2 exponent
# bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two codes per
# byte with element 2j in the low nibble.  The activations stay MXFP8.
# ----------------------------------------------------------------------------------------

E2M1_EMAX = 2          # exponent of the largest e2m1 value (6 = 1.5 * 2^2)
E2M1_MAX = 6.0


def e2m1_decode(codes) -> np.ndarray:
    """Value of each e2m1 code (0..15), float64."""
    c = np.asarray(codes, np.int64)
    e, m = (c >> 1) & 3, c & 1
    mag = np.where(e > 0, np.ldexp(1.0 + m / 2.0, e - 1), 0.5 * m)
    return np.where(c & 8, -mag, mag)


def e2m1_encode(v) -> np.ndarray:
    """Nearest e2m1 code (ties to the even code) of float values after clamping to +-6; the
    sign is kept (a negative value that rounds to zero gives 0x8)."""
    v = np.asarray(v, np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no defined code here")
    table = e2m1_decode(np.arange(8))                 # the 8 magnitudes, ascending
    mids = (table[:-1] + table[1:]) / 2               # halfway between neighbours
    a = np.minimum(np.abs(v), E2M1_MAX)
    # the nearest magnitude's index is the number of midpoints below |v|; exactly on a
    # midpoint both neighbours are nearest and the even code is taken
    below = np.searchsorted(mids, a, side="left")     # midpoints < |v|
    upto = np.searchsorted(mids, a, side="right")     # midpoints <= |v|
    code = np.where(below == upto, below, np.where(below % 2 == 0, below, upto))
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def quantize_mxfp4(a):
    """MXFP4 of a float32 array [..., K] along K (K a multiple of 32): per 32-block,
    X = floor(log2(amax)) - 2 clamped to [-127, 127] (0 for an all-zero block), codes
    e2m1_encode(v * 2^-X) (exact scaling, then clamped to +-6).  Returns (packed codes uint8
    [..., K/2], element 2j in the low nibble of byte j; scale codes uint8 [..., K/32])."""
    a = np.asarray(a, dtype=np.float32)
    K = a.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = a.reshape(a.shape[:-1] + (K // MX_BLOCK, MX_BLOCK)).astype(np.float64)
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)
    X = np.where(amax > 0, np.clip(ex - 1 - E2M1_EMAX, -127, 127), 0).astype(np.int64)
    codes = e2m1_encode(blocks * np.ldexp(1.0, -X)[..., None]).reshape(a.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (X + 127).astype(np.uint8)


def unpack_e2m1(packed) -> np.ndarray:
    """Codes [..., 2 n] of packed bytes [..., n] (low nibble first)."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def dequantize_mxfp4(packed, scales) -> np.ndarray:
    """decode(code) * 2^(scale code - 127) of its 32-block, float64."""
    vals = e2m1_decode(unpack_e2m1(packed))
    K = vals.shape[-1]
    X = np.asarray(scales, np.int64) - 127
    v = vals.reshape(vals.shape[:-1] + (K // MX_BLOCK, MX_BLOCK)) * np.ldexp(1.0, X)[..., None]
    return v.reshape(vals.shape)


def _quantizer(fmt: str):
    """(quantise a float32 activation matrix, dequantise it, dequantise an expert matrix)
    of the block-scaled ("block": 1x128 activations, 128x128 weights), the MXFP8 ("mxfp8":
    1x32 blocks along K for both) or the MXFP4-weight ("mxfp4": MXFP4 weights, MXFP8
    activations) format."""
    if fmt == "block":
        return (quantize_activations, lambda q, s: dequantize_blocks(q, s, rows=1, cols=BLOCK),
                dequantize_blocks)
    if fmt == "mxfp8":
        return quantize_mx, dequantize_mx, dequantize_mx
    if fmt == "mxfp4":              # MXFP4 weights, MXFP8 activations
        return quantize_mx, dequantize_mx, dequantize_mxfp4
    raise ValueError(f"unknown format {fmt}")


def expert_ffn(xd_rows, w13_codes, w13_scales, b13, w2_codes, w2_scales, b2, I: int,
               fmt: str = "block"):
    """One expert on its rows (float64).

    C = xd . deq(w13)^T + b13 ;  h = silu(C[:, :I]) * C[:, I:] ;  h is rounded to
    fp32 and quantised per row (1x128 groups, or 1x32 MX blocks) ;
    y = deq(h) . deq(w2)^T + b2.  Returns (y, h_codes, h_scales, h64)."""
    q_act, dq_act, dq_w = _quantizer(fmt)
    W13 = dq_w(w13_codes, w13_scales)
    C = xd_rows @ W13.T + bf16_to_f64(b13)
    h = silu(C[:, :I]) * C[:, I:]
    hq, hs = q_act(h.astype(np.float32))
    hd = dq_act(hq, hs)
    W2 = dq_w(w2_codes, w2_scales)
    y = hd @ W2.T + bf16_to_f64(b2)
    return y, hq, hs, h


def combine(y, gates, inv, T: int, k: int) -> np.ndarray:
    """out[t] = sum_j gates[t, j] * y[inv[t*k + j]]  (float64)."""
    yr = y[np.asarray(inv, np.int64).reshape(T, k)]          # [T, k, H]
    return np.einsum("tk,tkh->th", np.asarray(gates, np.float64), yr)


def f64_to_bf16_bits(a) -> np.ndarray:
    """Round float64 to bfloat16 once (nearest, ties to even) -- the output format."""
    a = np.asarray(a, np.float64)
    # exact: split via float32 is not single rounding, so round directly from float64
    m, e = np.frexp(a)                       # a = m 2^e, |m| in [0.5, 1)
    q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # 8 significant bits, half-even
    return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def forward(x_bits, router_w, router_b, top_k: int, I: int, w13_codes, w13_scales, b13,
            w2_codes, w2_scales, b2, token_subset=None, fmt: str = "block"):
    """The layer forward pass.

    ``w13_codes`` etc. are indexable by expert (arrays [E, ...] or dict-like of the
    experts needed).  With ``token_subset`` only those tokens are evaluated: routing,
    x quantisation and the combine are per token, so a token's output does not depend
    on which other tokens are present (the dispatch tables are still built over all
    tokens).  ``fmt`` = "mxfp8" takes MXFP8 weights (scales [E, N, K/32] E8M0 codes) and
    quantises x and h in 1x32 MX blocks.  Returns a dict of every stage's result."""
    q_act, dq_act, _ = _quantizer(fmt)
    T = x_bits.shape[0]
    E = router_w.shape[0]
    logits = router_logits(x_bits, router_w, router_b)
    ids, gates = topk_softmax(logits, top_k)
    counts, offsets, perm, inv = permute(ids, E)
    x32 = bf16_to_f64(x_bits).astype(np.float32)
    toks = np.arange(T) if token_subset is None else np.asarray(token_subset)
    xq, sx = q_act(x32[toks])
    xd = dq_act(xq, sx)
    H = x_bits.shape[1]
    y = np.zeros((toks.size, top_k, H))
    for e in np.unique(ids[toks]):
        rows_t, rows_j = np.nonzero(ids[toks] == e)
        ye, _, _, _ = expert_ffn(xd[rows_t], w13_codes[e], w13_scales[e], b13[e],
                                 w2_codes[e], w2_scales[e], b2[e], I, fmt)
        y[rows_t, rows_j] = ye
    out = np.einsum("tk,tkh->th", gates[toks], y)
    return dict(logits=logits, ids=ids, gates=gates, counts=counts, offsets=offsets, perm=perm,
                inv=inv, xq=xq, sx=sx, out=out, out_bf16=f64_to_bf16_bits(out), tokens=toks)


def forward_dispatched(x_bits, router_w, router_b, top_k: int, I: int, w13_codes, w13_scales,
                       b13, w2_codes, w2_scales, b2):
    """The same layer evaluated through the dispatch tables (permute -> per-expert
    contiguous segments -> combine via inv), as the pages' dispatch/combine split
    describes.  Used to pin ``forward`` and the tables against each other."""
    T = x_bits.shape[0]
    E = router_w.shape[0]
    logits = router_logits(x_bits, router_w, router_b)
    ids, gates = topk_softmax(logits, top_k)
    counts, offsets, perm, inv = permute(ids, E)
    x32 = bf16_to_f64(x_bits).astype(np.float32)
    xq, sx = quantize_activations(x32)
    xd = dequantize_blocks(xq, sx, rows=1, cols=BLOCK)
    tok_of_row = perm // top_k
    y = np.zeros((T * top_k, x_bits.shape[1]))
    hq = np.zeros((T * top_k, I), np.uint8)
    hs = np.ones((T * top_k, -(-I // BLOCK)), np.float32)
    h = np.zeros((T * top_k, I))
    for e in range(E):
        p0, p1 = offsets[e], offsets[e + 1]
        if p1 > p0:
            y[p0:p1], hq[p0:p1], hs[p0:p1], h[p0:p1] = expert_ffn(
                xd[tok_of_row[p0:p1]], w13_codes[e], w13_scales[e], b13[e], w2_codes[e],
                w2_scales[e], b2[e], I)
    out = combine(y, gates, inv, T, top_k)
    return dict(logits=logits, ids=ids, gates=gates, counts=counts, offsets=offsets, perm=perm,
                inv=inv, xq=xq, sx=sx, h=h, hq=hq, hs=hs, y=y, out=out,
                out_bf16=f64_to_bf16_bits(out))
