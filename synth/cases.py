"""Seeded synthetic inputs for the sparse MoE FFN layer.

This module is shared by the CPU oracle (``oracle/``) and by the HIP path
(``sparse_moe_ffn_gemm_amd``): both sides receive exactly the same tensors from
here.  It holds none of the layer's arithmetic.  The single exception is a
*precondition* check: router logits are evaluated in float64 only to redraw
token rows whose top-k logits are closer than ``MARGIN`` (so that the routing
decision is tie-free and has one correct answer).  That value is never used as
an expected result.

Shapes follow the workloads the pages serve ("GPT-OSS on day 0": gpt-oss-20b /
gpt-oss-120b with hidden size 2880 and top-4 routing; "Hosting Qwen on
Blackwell", section "Prefillers": Qwen3 235B, 128 experts, top-8) plus a
DeepSeek-V3-shaped layer with Zipf-skewed expert popularity.  No real prompts or
routing traces exist here; the three synthetic routing regimes (random,
uniform-dense, Zipf-skewed) stand in for them.

Distributions (all float32 draws, PCG64 streams keyed by (seed, tag[, expert])):
  x            ~ N(0, 1)      -> bfloat16 (round to nearest even)
  router W     ~ N(0, 0.05^2) float32 [E, H]
  router b     ~ N(0, 0.01^2) float32 [E]      (Zipf rule for the skewed layer)
  w13, w2      ~ N(0, 0.02^2) float32 [E, 2I, H], [E, H, I]
  b13, b2      ~ N(0, 0.01^2) -> bfloat16      (zero when expert_bias=False)

Expert weights of the large layers are drawn per expert on the GPU with torch's
Philox generator (``weights_on_device``); a CPU consumer obtains the very same
values by copying them back (``expert_weights(..., device="cuda").cpu()``).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

MARGIN = 1e-3          # minimum gap between consecutive sorted top-(k+1) logits
BLOCK = 128            # quantisation block edge

# stream tags
_TAG_X, _TAG_RW, _TAG_RB, _TAG_B13, _TAG_B2, _TAG_ZIPF, _TAG_REDRAW = 1, 2, 3, 4, 5, 6, 7
_TAG_W13, _TAG_W2 = 100, 101


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    T: int
    H: int
    E: int
    top_k: int
    I: int
    seed: int
    expert_bias: bool = True
    router: str = "random"          # "random" | "zipf" | "hot" (expert 0 always chosen) |
                                    # "one_per_expert" (token t's first choice is expert t mod E)
    weights_on_device: bool = False  # draw expert weights with torch on the GPU
    token_slice_of: Optional[str] = None  # decode layer reusing a prefill layer's draw

    @property
    def rows(self) -> int:
        return self.T * self.top_k

    def fp8_flops(self) -> int:
        """Algorithmic FP8 flops of the two grouped GEMMs (routed rows only)."""
        return 2 * self.T * self.top_k * 3 * self.H * self.I

    def router_flops(self) -> int:
        return 2 * self.T * self.H * self.E


def _kb(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK


SHAPES = {
    s.name: s
    for s in [
        LayerShape("tiny", T=16, H=256, E=8, top_k=2, I=256, seed=0),
        LayerShape("gpt-oss-20b-decode", T=64, H=2880, E=32, top_k=4, I=2880, seed=1),
        LayerShape("gpt-oss-120b-prefill", T=8192, H=2880, E=128, top_k=4, I=2880, seed=2,
                   weights_on_device=True),
        LayerShape("qwen3-235b-decode", T=32, H=4096, E=128, top_k=8, I=1536, seed=3,
                   expert_bias=False, weights_on_device=True,
                   token_slice_of="qwen3-235b-prefill"),
        LayerShape("qwen3-235b-prefill", T=4096, H=4096, E=128, top_k=8, I=1536, seed=3,
                   expert_bias=False, weights_on_device=True),
        LayerShape("deepseek-v3-skewed", T=16384, H=7168, E=256, top_k=8, I=2048, seed=4,
                   router="zipf", weights_on_device=True),
    ]
}


def custom_shape(T, H, E, top_k, I, seed=1234, expert_bias=True, router="random",
                 name=None) -> LayerShape:
    """A host-generated layer of arbitrary size (edge cases, small tests)."""
    return LayerShape(name or f"custom-T{T}-H{H}-E{E}-k{top_k}-I{I}-s{seed}", T=T, H=H, E=E,
                      top_k=top_k, I=I, seed=seed, expert_bias=expert_bias, router=router)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _seed63(*key: int) -> int:
    return int(np.random.SeedSequence(list(key)).generate_state(1, np.uint64)[0] >> np.uint64(1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _zipf_bias(shape: LayerShape) -> np.ndarray:
    """Router bias giving Zipf(s=1.1) expert popularity: b_e = lam * ln p_rank(e)."""
    E, H = shape.E, shape.H
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** -1.1
    p /= p.sum()
    order = _rng(shape.seed, _TAG_ZIPF).permutation(E)   # expert e gets rank order[e]+1
    lam = 0.05 * math.sqrt(H)
    return (lam * np.log(p[order])).astype(np.float32)


def _margin_ok(x_bits: np.ndarray, W: np.ndarray, b: np.ndarray, k: int) -> np.ndarray:
    """Per row: every gap between consecutive sorted top-(k+1) logits is >= MARGIN."""
    x = bf16_bits_to_f32(x_bits).astype(np.float64)
    lg = x @ W.astype(np.float64).T + b.astype(np.float64)
    m = min(k + 1, lg.shape[1])
    top = -np.sort(-lg, axis=1)[:, :m]
    if m < 2:
        return np.ones(lg.shape[0], dtype=bool)
    return np.all(top[:, :-1] - top[:, 1:] >= MARGIN, axis=1)


@dataclasses.dataclass
class LayerInputs:
    """Host copies of one layer's non-expert inputs (numpy)."""
    shape: LayerShape
    x: np.ndarray            # [T, H] uint16 (bf16 bits)
    router_w: np.ndarray     # [E, H] float32
    router_b: np.ndarray     # [E] float32
    b13: np.ndarray          # [E, 2I] uint16 (bf16 bits)
    b2: np.ndarray           # [E, H] uint16 (bf16 bits)
    redraws: int             # number of x rows redrawn for the margin


def make_inputs(shape: LayerShape) -> LayerInputs:
    """Activations, router and expert biases for ``shape`` (deterministic in the seed)."""
    if shape.token_slice_of is not None:
        parent = make_inputs(SHAPES[shape.token_slice_of])
        return LayerInputs(shape, parent.x[: shape.T].copy(), parent.router_w, parent.router_b,
                           parent.b13, parent.b2, parent.redraws)
    T, H, E, I, k = shape.T, shape.H, shape.E, shape.I, shape.top_k
    s = shape.seed
    x = f32_to_bf16_bits(_normal(_rng(s, _TAG_X), (T, H), 1.0))
    W = _normal(_rng(s, _TAG_RW), (E, H), 0.05)
    if shape.router == "zipf":
        b = _zipf_bias(shape)
    else:
        b = _normal(_rng(s, _TAG_RB), (E,), 0.01)
    if shape.router == "hot":          # edge case: expert 0 is every token's first choice
        b[0] += np.float32(1000.0)
    if shape.router == "one_per_expert":
        # the pages' decode GEMM benchmark: every expert activated by a single token.  Row
        # e of W gains 40 x_e / |x_e|^2 (token e's own direction), so token e's logit for
        # expert e exceeds the random ones (std 0.05 sqrt(H)) by a wide margin, and with
        # T = E and top_k = 1 each expert gets exactly one token.
        xf = bf16_bits_to_f32(x).astype(np.float64)
        for e in range(min(E, T)):
            W[e] += (40.0 * xf[e] / np.dot(xf[e], xf[e])).astype(np.float32)
    if shape.expert_bias:
        b13 = f32_to_bf16_bits(_normal(_rng(s, _TAG_B13), (E, 2 * I), 0.01))
        b2 = f32_to_bf16_bits(_normal(_rng(s, _TAG_B2), (E, H), 0.01))
    else:
        b13 = np.zeros((E, 2 * I), np.uint16)
        b2 = np.zeros((E, H), np.uint16)
    redraws = 0
    rnd = 0
    ok = _margin_ok(x, W, b, k)
    while not ok.all():
        bad = np.nonzero(~ok)[0]
        redraws += bad.size
        x[bad] = f32_to_bf16_bits(_normal(_rng(s, _TAG_REDRAW, rnd), (bad.size, H), 1.0))
        ok[bad] = _margin_ok(x[bad], W, b, k)
        rnd += 1
        if rnd > 1000:
            raise RuntimeError("margin redraw did not converge")
    return LayerInputs(shape, x, W, b, b13, b2, redraws)


def _weights_shape(shape: LayerShape, which: str):
    if which == "w13":
        return (2 * shape.I, shape.H), _TAG_W13
    if which == "w2":
        return (shape.H, shape.I), _TAG_W2
    raise ValueError(which)


def _base_shape(shape: LayerShape) -> LayerShape:
    return SHAPES[shape.token_slice_of] if shape.token_slice_of else shape


def expert_weights(shape: LayerShape, which: str, e: int, device: str = "cpu"):
    """fp32 weights of one expert: w13 [2I, H] or w2 [H, I], as a torch tensor.

    Host-drawn layers return the same values on any device.  Device-drawn layers
    (``weights_on_device``) are drawn with torch's CUDA generator and must be
    requested with ``device="cuda"``; copy the result to the host for CPU use.
    """
    import torch

    base = _base_shape(shape)
    dims, tag = _weights_shape(base, which)
    if base.weights_on_device:
        if not device.startswith("cuda"):
            raise ValueError(f"{base.name}: expert weights are drawn on the GPU; use device='cuda'")
        g = torch.Generator(device=device)
        g.manual_seed(_seed63(base.seed, tag, e))
        w = torch.randn(dims, generator=g, device=device, dtype=torch.float32)
        return w.mul_(0.02)
    a = _normal(_rng(base.seed, tag, e), dims, 0.02)
    return torch.from_numpy(a).to(device)


def all_expert_weights_host(shape: LayerShape, which: str, threads: Optional[int] = None) -> np.ndarray:
    """[E, N, K] float32 for a host-drawn layer (threaded per expert)."""
    base = _base_shape(shape)
    if base.weights_on_device:
        raise ValueError(f"{base.name}: expert weights are drawn on the GPU")
    dims, tag = _weights_shape(base, which)
    out = np.empty((base.E,) + dims, np.float32)

    def fill(e):
        _rng(base.seed, tag, e).standard_normal(out=out[e], dtype=np.float32)
        out[e] *= np.float32(0.02)

    n = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(fill, range(base.E)))
    return out
