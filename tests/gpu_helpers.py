"""Shared helpers of the GPU parity tests: upload a synthetic layer, build the oracle's
own quantised weights for the experts a check needs, and compare outputs."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import sparse_moe_ffn_gemm_amd as moe
from oracle import moe_ref as R
from synth import LayerShape, expert_weights, make_inputs

REL_FRO_TOL = 5e-3
MAX_ELT_TOL = 2e-2
GATE_TOL = 1e-6
# Device error of h relative to its 1x128 group maximum.  Each K=128 FP8 matrix-core
# dot product on gfx950 carries up to ~6e-5 of the tile maximum (measured with random
# codes; every single product is exact); over up to 56 promoted K-blocks that stays below
# 2^-13.  Every code that a quotient within that distance (times 448 code units) of the
# oracle's h / s rounds to is a correct code; near zero that window spans several codes.
H_EPS = 2.0 ** -13


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


class GpuLayer:
    """Device tensors of one layer; expert weights quantised by the library (``fmt``
    "block": 128x128 block scales, "mxfp8": MXFP8, "mxfp4": MXFP4 weights)."""

    def __init__(self, shape: LayerShape, inputs=None, device="cuda", fmt="block"):
        self.shape = shape
        self.fmt = fmt
        self.li = inputs if inputs is not None else make_inputs(shape)
        li = self.li
        self.x = bf16_dev(li.x, device)
        b13 = bf16_dev(li.b13, device) if shape.expert_bias else None
        b2 = bf16_dev(li.b2, device) if shape.expert_bias else None
        self.layer = moe.MoELayer.from_expert_weights(
            torch.from_numpy(li.router_w), torch.from_numpy(li.router_b), shape.top_k, b13, b2,
            lambda e: expert_weights(shape, "w13", e, device),
            lambda e: expert_weights(shape, "w2", e, device), device=device, fmt=fmt)
        torch.cuda.synchronize()


def quantize_by_rows(quant, w: np.ndarray, rows: int = 128):
    """The oracle's weight quantiser applied to 128-row slices of w (every format's scale
    blocks lie within one slice, so the result is the whole-matrix one; the slices keep the
    oracle's per-element temporaries in cache)."""
    parts = [quant(w[i:i + rows]) for i in range(0, w.shape[0], rows)]
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


class OracleExperts:
    """Lazily quantised experts for the oracle (from the generator's fp32 weights), in the
    block-scaled, the MXFP8 or the MXFP4-weight format."""

    def __init__(self, shape: LayerShape, li, fmt="block"):
        self.shape, self.li = shape, li
        self.fmt = fmt
        self.cache = {}
        self.dev = "cuda" if _base(shape).weights_on_device else "cpu"

    def prepare(self, experts, threads=16):
        todo = [int(e) for e in experts if int(e) not in self.cache]
        # draw on the device serially, quantise on the host in parallel
        host = {e: (expert_weights(self.shape, "w13", e, self.dev).cpu().numpy(),
                    expert_weights(self.shape, "w2", e, self.dev).cpu().numpy()) for e in todo}

        quant = {"block": R.quantize_blocks, "mxfp8": R.quantize_mx,
                 "mxfp4": R.quantize_mxfp4}[self.fmt]

        def q(e):
            c13, s13 = quantize_by_rows(quant, host[e][0])
            c2, s2 = quantize_by_rows(quant, host[e][1])
            return e, (c13, s13, c2, s2)

        with ThreadPoolExecutor(max_workers=threads) as ex:
            for e, v in ex.map(q, todo):
                self.cache[e] = v

    def view(self, idx):
        cache = self.cache

        class _V:
            def __getitem__(self, e):
                return cache[int(e)][idx]
        return _V()

    def forward(self, token_subset=None):
        li = self.li
        ids = R.topk_softmax(R.router_logits(li.x, li.router_w, li.router_b), self.shape.top_k)[0]
        need = np.unique(ids if token_subset is None else ids[np.asarray(token_subset)])
        self.prepare(need)
        ref = R.forward(li.x, li.router_w, li.router_b, self.shape.top_k, self.shape.I,
                        self.view(0), self.view(1), li.b13, self.view(2), self.view(3), li.b2,
                        token_subset=token_subset, fmt=self.fmt)
        ref["allowance"] = self.flip_allowance(ref)
        return ref

    def dequant_w(self, codes, scales):
        deq = {"block": R.dequantize_blocks, "mxfp8": R.dequantize_mx,
               "mxfp4": R.dequantize_mxfp4}[self.fmt]
        return deq(codes, scales)

    def flip_allowance(self, ref):
        """Per output element of the evaluated tokens: sum_j g_j * |W2_j| . flip_delta(h_j)."""
        li, k, I = self.li, self.shape.top_k, self.shape.I
        toks = ref["tokens"]
        x32 = R.bf16_to_f64(li.x[toks]).astype(np.float32)
        if self.fmt != "block":                 # MXFP8 activations
            xd = R.dequantize_mx(*R.quantize_mx(x32))
        else:
            xq, sx = R.quantize_activations(x32)
            xd = R.dequantize_blocks(xq, sx, rows=1)
        allow = np.zeros((toks.size, li.x.shape[1]))
        for e in np.unique(ref["ids"][toks]):
            rt, rj = np.nonzero(ref["ids"][toks] == e)
            c13, s13, c2, s2 = self.cache[int(e)]
            _, hq, hs, h64 = R.expert_ffn(xd[rt], c13, s13, li.b13[e], c2, s2, li.b2[e], I,
                                          self.fmt)
            W2 = np.abs(self.dequant_w(c2, s2))
            delta = flip_delta(h64, hq, hs) if self.fmt == "block" else flip_delta_mx(h64, hq, hs)
            allow[rt] += ref["gates"][toks[rt], rj][:, None] * (delta @ W2.T)
        return allow


def dispatched_allowance(ref, experts: "OracleExperts", T: int, k: int):
    """flip allowance for a full dispatched oracle result (all tokens)."""
    rows = ref["h"].shape[0]
    contrib = np.zeros((rows, ref["y"].shape[1]))
    delta = flip_delta(ref["h"], ref["hq"], ref["hs"])
    for e in range(len(ref["counts"])):
        p0, p1 = ref["offsets"][e], ref["offsets"][e + 1]
        if p1 > p0:
            c2, s2 = experts.cache[e][2], experts.cache[e][3]
            contrib[p0:p1] = delta[p0:p1] @ np.abs(R.dequantize_blocks(c2, s2)).T
    return R.combine(contrib, ref["gates"], ref["inv"], T, k)


def _base(shape):
    from synth.cases import _base_shape
    return _base_shape(shape)


def bf16_ulp(ref: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(int) - 7)


def _h_window(h64: np.ndarray, hs: np.ndarray):
    """Decoded values of the lowest and highest codes that a quotient within H_EPS * 448 code
    units of the oracle's h / s can round to (the codes a correct kernel may produce given its
    fp32 accumulation error), and the per-element scale."""
    I = h64.shape[1]
    s = np.repeat(hs.astype(np.float64), 128, axis=1)[:, :I]
    v = h64 / s
    eps = H_EPS * 448
    return R.e4m3_decode(R.e4m3_encode(v - eps)), R.e4m3_decode(R.e4m3_encode(v + eps)), s


def flip_delta(h64: np.ndarray, hq: np.ndarray, hs: np.ndarray) -> np.ndarray:
    """For oracle h rows: the largest value change between the oracle's code and any code of
    the window ``_h_window`` (0 where the window holds only the oracle's code).  Near zero the
    window can span several codes, since the e4m3 spacing there is much finer than the
    accumulation error, which scales with the group's largest value.  Uses the oracle's own
    h, codes and scales only."""
    lo, hi, s = _h_window(h64, hs)
    dq = R.e4m3_decode(hq)
    return np.maximum(np.abs(lo - dq), np.abs(hi - dq)) * s


def _group128_max(h64: np.ndarray) -> np.ndarray:
    """max |h| over each element's 1x128 column group (the scale of the device's fp32
    accumulation error in h, whatever the quantisation format)."""
    I = h64.shape[1]
    g = -(-I // 128)
    pad = np.zeros((h64.shape[0], g * 128))
    pad[:, :I] = np.abs(h64)
    return np.repeat(pad.reshape(-1, g, 128).max(axis=2), 128, axis=1)[:, :I]


def flip_delta_mx(h64: np.ndarray, hq: np.ndarray, hs: np.ndarray) -> np.ndarray:
    """``flip_delta`` for MXFP8 h (1x32 blocks, E8M0 codes ``hs`` [rows, I/32]): the device's
    h may differ from the oracle's by H_EPS of its 1x128 group maximum; every code a value
    within that distance rounds to at the oracle's block scale is correct, and where the
    block maximum itself lies within that distance of a power of two the device may take
    the neighbouring exponent, so the codes of the block at that scale count too."""
    I = h64.shape[1]
    eps = H_EPS * _group128_max(h64)
    X = np.repeat(hs.astype(np.int64) - 127, 32, axis=1)[:, :I]
    dq = R.e4m3_decode(hq) * np.ldexp(1.0, X)
    out = np.zeros_like(h64)
    for dx in (0, -1, 1):
        s = np.ldexp(1.0, X + dx)
        lo = R.e4m3_decode(R.e4m3_encode(((h64 - eps) / s).astype(np.float32))) * s
        hi = R.e4m3_decode(R.e4m3_encode(((h64 + eps) / s).astype(np.float32))) * s
        d = np.maximum(np.abs(lo - dq), np.abs(hi - dq))
        if dx != 0:
            # only blocks whose maximum is within eps of the power of two between the scales
            amax = np.abs(h64).reshape(h64.shape[0], -1, 32).max(axis=2)
            edge = np.ldexp(1.0, (hs.astype(np.int64) - 127) + 8 + (1 if dx > 0 else 0))
            e_blk = eps.reshape(h64.shape[0], -1, 32).max(axis=2)
            near = np.abs(amax - edge) <= e_blk
            d = d * np.repeat(near, 32, axis=1)[:, :I]
        out = np.maximum(out, d)
    return out


def compare_out(gpu_bits: np.ndarray, ref: np.ndarray, what="", allowance=None):
    """Relative Frobenius <= 5e-3.  An element fails the max-elementwise bound only if its
    error exceeds max(2e-2 * RMS(ref), one bf16 ulp of the reference value) -- the output
    format cannot resolve less -- plus ``allowance``: the largest change that legitimate
    h code changes within the accumulation window can cause (``flip_delta`` through |W2|,
    gated).
    The literal max |err| / RMS is always reported."""
    g = R.bf16_to_f64(gpu_bits)
    d = g - ref
    rel = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    rms = np.sqrt(np.mean(ref * ref))
    lit = np.abs(d).max() / rms if rms > 0 else 0.0
    base = np.maximum(MAX_ELT_TOL * rms, bf16_ulp(ref))
    over = np.abs(d) > base
    bad = np.abs(d) > base + (0.0 if allowance is None else allowance)
    floor = np.abs(R.bf16_to_f64(R.f64_to_bf16_bits(ref)) - ref).max() / rms if rms > 0 else 0.0
    info = dict(rel_fro=rel, max_over_rms=lit, n_over_literal=int(over.sum()), n_bad=int(bad.sum()),
                n=d.size, floor=floor)
    say(f"  out parity {what}: rel_fro={rel:.3e} max/rms={lit:.3e} (bf16 floor {floor:.3e}) "
        f"over 2e-2*RMS (and 1 ulp): {int(over.sum())}, beyond h-flip allowance: {int(bad.sum())}"
        f" of {d.size}")
    assert rel <= REL_FRO_TOL, info
    assert not bad.any(), info
    return info


def gate_tolerance(ref_logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Per-token gate tolerance: 1e-6 plus the fp32 floor of the selected logits.

    The device evaluates logits in fp32 (two-level sum over H) and the softmax in fp32, so
    each selected logit carries a few fp32 ulps of its own magnitude; the softmax over the
    selected logits moves a gate by at most half the largest logit error.  Allowing 8 ulps
    per logit: tol_t = 1e-6 + 0.5 * 8 * ulp32(max_j |l_tj|)."""
    sel = np.take_along_axis(ref_logits, ids.astype(np.int64), axis=1)
    mx = np.abs(sel).max(axis=1)
    ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(mx, 2.0 ** -126))).astype(int) - 23)
    return GATE_TOL + 4.0 * ulp


def routing_exact(gpu: dict, ref: dict, T: int, k: int, what=""):
    ids = gpu["topk_ids"].cpu().numpy()
    assert np.array_equal(ids, ref["ids"]), f"{what}: ids differ at {np.argwhere(ids != ref['ids'])[:5]}"
    assert np.array_equal(gpu["expert_counts"].cpu().numpy(), ref["counts"]), what
    assert np.array_equal(gpu["expert_offsets"].cpu().numpy(), ref["offsets"]), what
    assert np.array_equal(gpu["perm"].cpu().numpy(), ref["perm"]), what
    assert np.array_equal(gpu["inv_perm"].cpu().numpy(), ref["inv"]), what
    g = gpu["topk_gates"].cpu().numpy().astype(np.float64)
    err = np.abs(g - ref["gates"]).max(axis=1)
    tol = gate_tolerance(ref["logits"], ref["ids"])
    say(f"  routing {what}: exact; max |gate err| = {err.max():.2e} (tolerance {tol.min():.1e}.."
        f"{tol.max():.1e})")
    assert np.all(err <= tol), np.argwhere(err > tol)[:5]


def h_codes_close(gpu_hq: np.ndarray, ref: dict, max_frac=0.01):
    """h codes may differ from the oracle's only within the window of ``_h_window`` (a
    quotient within H_EPS * 448 code units of the oracle's), and at most ``max_frac`` of
    them may differ."""
    ref_hq = ref["hq"]
    diff = gpu_hq != ref_hq
    frac = diff.mean()
    lo, hi, _ = _h_window(ref["h"], ref["hs"])
    g = R.e4m3_decode(gpu_hq)
    ok = (g >= lo) & (g <= hi)
    say(f"  h: {int(diff.sum())} of {diff.size} codes differ ({frac:.2e}); "
        f"all within the accumulation window: {bool(ok.all())}")
    if not ok.all():
        I = ref["h"].shape[1]
        for rr, cc in np.argwhere(~ok)[:5]:
            grp = slice((cc // 128) * 128, min((cc // 128 + 1) * 128, I))
            gmax = np.abs(ref["h"][rr, grp]).max()
            say(f"    row {rr} col {cc}: oracle code {ref_hq[rr, cc]:#04x} gpu {gpu_hq[rr, cc]:#04x} "
                f"h={ref['h'][rr, cc]:.6g} group max {gmax:.6g} scale {ref['hs'][rr, cc // 128]:.6g}")
    assert frac <= max_frac and ok.all()
