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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


class GpuLayer:
    """Device tensors of one layer; expert weights quantised by the library."""

    def __init__(self, shape: LayerShape, inputs=None, device="cuda"):
        self.shape = shape
        self.li = inputs if inputs is not None else make_inputs(shape)
        li = self.li
        self.x = bf16_dev(li.x, device)
        b13 = bf16_dev(li.b13, device) if shape.expert_bias else None
        b2 = bf16_dev(li.b2, device) if shape.expert_bias else None
        self.layer = moe.MoELayer.from_expert_weights(
            torch.from_numpy(li.router_w), torch.from_numpy(li.router_b), shape.top_k, b13, b2,
            lambda e: expert_weights(shape, "w13", e, device),
            lambda e: expert_weights(shape, "w2", e, device), device=device)
        torch.cuda.synchronize()


class OracleExperts:
    """Lazily quantised experts for the oracle (from the generator's fp32 weights)."""

    def __init__(self, shape: LayerShape, li):
        self.shape, self.li = shape, li
        self.cache = {}
        self.dev = "cuda" if _base(shape).weights_on_device else "cpu"

    def prepare(self, experts, threads=16):
        todo = [int(e) for e in experts if int(e) not in self.cache]
        # draw on the device serially, quantise on the host in parallel
        host = {e: (expert_weights(self.shape, "w13", e, self.dev).cpu().numpy(),
                    expert_weights(self.shape, "w2", e, self.dev).cpu().numpy()) for e in todo}

        def q(e):
            c13, s13 = R.quantize_blocks(host[e][0])
            c2, s2 = R.quantize_blocks(host[e][1])
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
        return R.forward(li.x, li.router_w, li.router_b, self.shape.top_k, self.shape.I,
                         self.view(0), self.view(1), li.b13, self.view(2), self.view(3), li.b2,
                         token_subset=token_subset)


def _base(shape):
    from synth.cases import _base_shape
    return _base_shape(shape)


def bf16_ulp(ref: np.ndarray) -> np.ndarray:
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(int) - 7)


def compare_out(gpu_bits: np.ndarray, ref: np.ndarray, what=""):
    """Relative Frobenius <= 5e-3; an element fails the max-elementwise bound only if its
    error exceeds both 2e-2 * RMS(ref) and one bf16 ulp of the reference value (the
    output format cannot resolve less).  Returns a dict of the measured errors."""
    g = R.bf16_to_f64(gpu_bits)
    d = g - ref
    rel = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    rms = np.sqrt(np.mean(ref * ref))
    lit = np.abs(d).max() / rms if rms > 0 else 0.0
    bad = np.abs(d) > np.maximum(MAX_ELT_TOL * rms, bf16_ulp(ref))
    floor = np.abs(R.bf16_to_f64(R.f64_to_bf16_bits(ref)) - ref).max() / rms if rms > 0 else 0.0
    info = dict(rel_fro=rel, max_over_rms=lit, n_bad=int(bad.sum()), n=d.size, floor=floor)
    say(f"  out parity {what}: rel_fro={rel:.3e} max/rms={lit:.3e} (bf16 floor {floor:.3e}) "
        f"bad={int(bad.sum())}/{d.size}")
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


def h_codes_close(gpu_hq: np.ndarray, ref_hq: np.ndarray, max_frac=0.01):
    """h codes may differ by one step where the fp32 device value and the oracle's value
    fall on different sides of a rounding boundary (the grouped GEMM's fp8 dot products
    accumulate with less than fp32 precision); nothing else may differ."""
    diff = gpu_hq != ref_hq
    frac = diff.mean()
    g = gpu_hq[diff].astype(np.int64)
    r = ref_hq[diff].astype(np.int64)
    same_sign = (g & 0x80) == (r & 0x80)
    step = np.abs((g & 0x7F) - (r & 0x7F))
    zero_pair = ((g & 0x7F) == 0) & ((r & 0x7F) <= 1) | ((r & 0x7F) == 0) & ((g & 0x7F) <= 1)
    adjacent = (same_sign & (step == 1)) | zero_pair
    say(f"  h: {int(diff.sum())} of {diff.size} codes differ ({frac:.2e}), all adjacent: "
        f"{bool(adjacent.all())}")
    assert frac <= max_frac and adjacent.all()
