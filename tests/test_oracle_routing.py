"""Pins of the oracle's router, top-k + softmax and dispatch tables.

"GPT-OSS on day 0", section "Kernels -> MoE": routing selects the top-k experts
and applies the softmax only over the selected logits.  "Hosting Qwen on
Blackwell", section "Expert Parallel": dispatch aggregates the routing
information and gathers each expert's tokens into its GEMM input buffer.
"""
import math

import numpy as np
import pytest

from oracle import moe_ref as R
from synth import f32_to_bf16_bits


def test_router_logits_brute_force_exact():
    rng = np.random.default_rng(1)
    T, H, E = 5, 24, 7
    x = rng.integers(-8, 9, (T, H)).astype(np.float32)          # exact in bf16
    W = rng.integers(-5, 6, (E, H)).astype(np.float32)
    b = rng.integers(-3, 4, E).astype(np.float32)
    got = R.router_logits(f32_to_bf16_bits(x), W, b)
    for t in range(T):
        for e in range(E):
            ref = sum(float(x[t, h]) * float(W[e, h]) for h in range(H)) + float(b[e])
            assert got[t, e] == ref


def test_router_logits_orientation_nonsymmetric():
    # x . W^T (not x . W): a single non-zero weight picks one hidden unit for one expert
    x = np.zeros((2, 4), np.float32)
    x[0, 1] = 1.0
    x[1, 3] = 2.0
    W = np.zeros((3, 4), np.float32)
    W[2, 1] = 5.0
    W[0, 3] = 7.0
    got = R.router_logits(f32_to_bf16_bits(x), W, np.array([0.5, 0.0, 0.0], np.float32))
    assert got.tolist() == [[0.5, 0.0, 5.0], [14.5, 0.0, 0.0]]


@pytest.mark.parametrize("k", [1, 2, 3, 8])
def test_topk_matches_sorted_brute_force(k):
    rng = np.random.default_rng(k)
    lg = np.round(rng.standard_normal((40, 8)), 1)               # many exact ties
    ids, gates = R.topk_softmax(lg, k)
    for t in range(lg.shape[0]):
        ref = sorted(range(8), key=lambda e: (-lg[t, e], e))[:k]
        assert ids[t].tolist() == ref
        z = [math.exp(lg[t, e] - lg[t, ref[0]]) for e in ref]
        assert np.allclose(gates[t], [v / sum(z) for v in z], rtol=0, atol=1e-15)


def test_gates_properties():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((64, 16)) * 4
    for k in (1, 2, 4, 8, 16):
        ids, g = R.topk_softmax(lg, k)
        assert np.all(np.abs(g.sum(1) - 1) <= 1e-15)
        assert np.all(np.diff(g, axis=1) <= 0)          # descending with the logits
        if k == 1:
            assert np.all(g == 1.0)
        if k == 2:                                       # closed form: sigmoid of the gap
            l1 = np.take_along_axis(lg, ids[:, :1].astype(int), 1)[:, 0]
            l2 = np.take_along_axis(lg, ids[:, 1:2].astype(int), 1)[:, 0]
            assert np.allclose(g[:, 0], 1 / (1 + np.exp(l2 - l1)), rtol=0, atol=1e-15)
    # k = E selects every expert in sorted order
    ids, _ = R.topk_softmax(lg, 16)
    assert np.array_equal(np.sort(ids, 1), np.tile(np.arange(16), (64, 1)))
    # equal logits -> 1/k each, lower indices first
    ids, g = R.topk_softmax(np.zeros((3, 8)), 4)
    assert np.all(g == 0.25) and np.all(ids == np.arange(4))


def test_softmax_after_topk_differs_from_softmax_over_all():
    # The page contrasts its router with DeepSeek-style routers that softmax over all experts.
    lg = np.array([[3.0, 2.0, 1.0, 0.0]])
    _, g = R.topk_softmax(lg, 2)
    full = np.exp(lg[0]) / np.exp(lg[0]).sum()
    assert abs(g.sum() - 1) < 1e-15 and abs(full[:2].sum() - 1) > 0.05
    assert np.allclose(g[0], full[:2] / full[:2].sum())


def test_permutation_tables():
    rng = np.random.default_rng(3)
    T, k, E = 50, 3, 9
    lg = rng.standard_normal((T, E))
    ids, _ = R.topk_softmax(lg, k)
    counts, offsets, perm, inv = R.permute(ids, E)
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    assert counts.sum() == T * k
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    # inverse: permute followed by unpermute is the identity
    assert np.array_equal(inv[perm], np.arange(T * k))
    assert np.array_equal(perm[inv], np.arange(T * k))
    # segment e holds exactly expert e's rows, tokens strictly increasing
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        t, j = seg // k, seg % k
        assert np.all(ids[t, j] == e)
        assert np.all(np.diff(t) > 0)
    # brute force: list of (expert, token, j) sorted
    ref = sorted(((ids[t, j], t, j) for t in range(T) for j in range(k)))
    assert perm.tolist() == [t * k + j for (_, t, j) in ref]


def test_permutation_with_idle_experts():
    ids = np.array([[0, 5], [5, 0], [0, 5]], np.int32)
    counts, offsets, perm, inv = R.permute(ids, 8)
    assert counts.tolist() == [3, 0, 0, 0, 0, 3, 0, 0]
    assert offsets.tolist() == [0, 3, 3, 3, 3, 3, 6, 6, 6]
    assert perm.tolist() == [0, 3, 4, 1, 2, 5]
