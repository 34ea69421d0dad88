"""GPU parity of routing: expert ids, counts, offsets, permutation and its inverse are
bit-exact against the oracle; gates within 1e-6.  Inputs satisfy the 1e-3 top-k logit
margin, so the routing decision has exactly one correct answer."""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_gemm_amd as moe
from oracle import moe_ref as R
from synth import SHAPES, custom_shape, make_inputs
from gpu_helpers import bf16_dev, routing_exact, say

pytestmark = pytest.mark.gpu

EDGE = [
    custom_shape(T=1, H=256, E=8, top_k=2, I=128, seed=21),
    custom_shape(T=5, H=64, E=1, top_k=1, I=64, seed=22),
    custom_shape(T=100, H=512, E=8, top_k=8, I=64, seed=23),       # k = E
    custom_shape(T=130, H=384, E=64, top_k=2, I=64, seed=24),       # ragged chunks
    custom_shape(T=300, H=256, E=256, top_k=8, I=64, seed=25),      # E = 256, idle experts
    custom_shape(T=200, H=256, E=16, top_k=3, I=64, seed=26, router="hot"),
    # the last single-chunk batch (scan and scatter in one workgroup) and the first two-chunk one
    custom_shape(T=256, H=192, E=32, top_k=4, I=64, seed=27),
    custom_shape(T=257, H=192, E=32, top_k=4, I=64, seed=28),
    # one-workgroup routing tail: fewer experts than list slots, uneven expert parts
    custom_shape(T=40, H=128, E=3, top_k=3, I=64, seed=29),
    custom_shape(T=64, H=128, E=70, top_k=4, I=64, seed=30),
    # the prefill routing kernel (T > 448): a ragged last 128-token tile, several H slices,
    # experts beyond one 128-expert tile, a single expert, top-8 of 256
    custom_shape(T=449, H=320, E=8, top_k=2, I=64, seed=31),
    custom_shape(T=700, H=1536, E=200, top_k=6, I=64, seed=32),
    custom_shape(T=520, H=192, E=1, top_k=1, I=64, seed=33),
    custom_shape(T=1000, H=576, E=256, top_k=8, I=64, seed=34, router="hot"),
]


def _run(shape, li):
    x = bf16_dev(li.x)
    W = torch.from_numpy(li.router_w).cuda()
    b = torch.from_numpy(li.router_b).cuda()
    say(f"route {shape.name}: T={shape.T} H={shape.H} E={shape.E} k={shape.top_k}")
    r = moe.route(x, W, b, shape.top_k)
    torch.cuda.synchronize()
    lg = R.router_logits(li.x, li.router_w, li.router_b)
    ids, gates = R.topk_softmax(lg, shape.top_k)
    counts, offsets, perm, inv = R.permute(ids, shape.E)
    ref = dict(logits=lg, ids=ids, gates=gates, counts=counts, offsets=offsets, perm=perm, inv=inv)
    routing_exact(r, ref, shape.name)
    return r


@pytest.mark.parametrize("name", list(SHAPES))
def test_route_configs(name):
    shape = SHAPES[name]
    _run(shape, make_inputs(shape))


@pytest.mark.parametrize("shape", EDGE, ids=[s.name for s in EDGE])
def test_route_edge_cases(shape):
    r = _run(shape, make_inputs(shape))
    if shape.router == "hot":
        assert np.all(r["topk_ids"].cpu().numpy()[:, 0] == 0)
        assert r["expert_counts"].cpu().numpy()[0] == shape.T


def test_route_deterministic():
    shape = SHAPES["deepseek-v3-skewed"]
    li = make_inputs(shape)
    x = bf16_dev(li.x)
    W = torch.from_numpy(li.router_w).cuda()
    b = torch.from_numpy(li.router_b).cuda()
    a = moe.route(x, W, b, shape.top_k)
    c = moe.route(x, W, b, shape.top_k)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], c[k]), k


@pytest.mark.parametrize("T,E,k", [(64, 32, 4), (64, 32, 8), (300, 32, 4), (7, 5, 3), (600, 32, 4),
                                   (530, 256, 8)])
def test_route_exact_ties(T, E, k):
    """A zero router gives every logit exactly 0: each token takes experts 0 .. k-1 (ties
    to the lower index) with gates 1/k, on the one-workgroup tail (k <= 4, one chunk), the
    single-chunk kernels (k = 8), the multi-chunk path (T = 300) and the prefill routing
    kernel (T > 448, one and two 128-expert tiles)."""
    g = torch.Generator().manual_seed(T * 1000 + E * 10 + k)
    x = torch.randn(T, 128, generator=g).to(torch.bfloat16).cuda()
    W = torch.zeros(E, 128, dtype=torch.float32, device="cuda")
    b = torch.zeros(E, dtype=torch.float32, device="cuda")
    say(f"route ties T={T} E={E} k={k}")
    r = moe.route(x, W, b, k)
    torch.cuda.synchronize()
    ids = r["topk_ids"].cpu().numpy()
    assert np.array_equal(ids, np.tile(np.arange(k, dtype=ids.dtype), (T, 1)))
    np.testing.assert_allclose(r["topk_gates"].cpu().numpy(), 1.0 / k, rtol=0, atol=1e-6)
    counts = r["expert_counts"].cpu().numpy()
    assert np.array_equal(counts, np.array([T] * k + [0] * (E - k)))
    # expert-major, token-ascending: slot e T + t holds (t, j = e)
    perm = r["perm"].cpu().numpy()
    want = np.array([t * k + e for e in range(k) for t in range(T)])
    assert np.array_equal(perm, want)
