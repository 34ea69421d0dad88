"""The parity checks' threaded evaluation of the plain oracle equals the oracle's own forward
bit for bit (CPU: host-drawn layers, all three weight formats)."""
import numpy as np
import pytest

from oracle import moe_ref as R
from synth import custom_shape, make_inputs
from gpu_helpers import OracleExperts, oracle_forward_out


@pytest.mark.parametrize("fmt", ["block", "mxfp8", "mxfp4"])
def test_threaded_oracle_forward_is_the_oracle(fmt):
    shape = custom_shape(T=40, H=192, E=6, top_k=2, I=128, seed=71)
    li = make_inputs(shape)
    ox = OracleExperts.of(shape, li, fmt)
    toks = np.array([0, 3, 17, 39])
    got = oracle_forward_out(li, shape.top_k, shape.I, ox, toks, fmt)
    ref = R.forward(li.x, li.router_w, li.router_b, shape.top_k, shape.I, ox.view(0), ox.view(1),
                    li.b13, ox.view(2), ox.view(3), li.b2, token_subset=toks, fmt=fmt)["out"]
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


def test_shared_oracle_experts():
    """A decode layer's check reuses the quantised experts of its weight draw's checks."""
    a = custom_shape(T=8, H=128, E=3, top_k=1, I=64, seed=72)
    li = make_inputs(a)
    ox = OracleExperts.of(a, li, "block")
    assert OracleExperts.of(a, li, "block") is ox
    assert OracleExperts.of(a, li, "mxfp8") is not ox
