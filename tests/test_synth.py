"""The seeded input generator: determinism, the routing-margin precondition and the
skewed layer's expert-popularity observables."""
import numpy as np
import pytest

from oracle import moe_ref as R
from synth import SHAPES, MARGIN, make_inputs, expert_weights, all_expert_weights_host, custom_shape


def test_deterministic():
    a = make_inputs(SHAPES["tiny"])
    b = make_inputs(SHAPES["tiny"])
    assert np.array_equal(a.x, b.x) and np.array_equal(a.router_w, b.router_w)
    assert np.array_equal(a.b13, b.b13) and np.array_equal(a.b2, b.b2)
    w1 = expert_weights(SHAPES["tiny"], "w13", 3).numpy()
    w2 = all_expert_weights_host(SHAPES["tiny"], "w13")[3]
    assert np.array_equal(w1, w2)
    assert w1.shape == (512, 256)


@pytest.mark.parametrize("name", ["tiny", "gpt-oss-20b-decode", "qwen3-235b-decode"])
def test_margin_precondition(name):
    li = make_inputs(SHAPES[name])
    lg = R.router_logits(li.x, li.router_w, li.router_b)
    k = li.shape.top_k
    top = -np.sort(-lg, axis=1)[:, : k + 1]
    assert np.all(top[:, :-1] - top[:, 1:] >= MARGIN)


def test_qwen_decode_is_prefix_of_prefill():
    d = make_inputs(SHAPES["qwen3-235b-decode"])
    p = make_inputs(SHAPES["qwen3-235b-prefill"])
    assert np.array_equal(d.x, p.x[:32])
    assert not d.b13.any() and not d.b2.any()


def test_distributions():
    li = make_inputs(custom_shape(T=512, H=1024, E=16, top_k=2, I=256))
    x = (li.x.astype(np.uint32) << 16).view(np.float32)
    assert abs(x.std() - 1) < 0.01 and abs(li.router_w.std() - 0.05) < 0.001


def test_zipf_skew_observables():
    li = make_inputs(SHAPES["deepseek-v3-skewed"])
    lg = R.router_logits(li.x, li.router_w, li.router_b)
    ids, _ = R.topk_softmax(lg, 8)
    counts = np.bincount(ids.ravel(), minlength=256)
    assert (counts == 0).sum() > 0          # some experts idle
    assert (counts > 2000).sum() > 0        # some experts with more than 2000 tokens
    top = -np.sort(-lg, axis=1)[:, :9]
    assert np.all(top[:, :-1] - top[:, 1:] >= MARGIN)
