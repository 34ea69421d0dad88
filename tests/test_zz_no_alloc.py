"""The entry point that allocates nothing (moe_forward_noalloc): the same layer as
moe_forward with the library's fixed per-device workspace, for callers that cannot allocate
(graph capture, serving loops).  Two calls in a row, the second smaller, each bit-identical
to moe_forward with a caller-owned workspace (the same kernels on the same inputs), and the
routing tables identical."""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_gemm_amd as moe
from sparse_moe_ffn_gemm_amd import _lib
from synth import SHAPES
from gpu_helpers import GpuLayer, say

pytestmark = pytest.mark.gpu


def _pair(g, T):
    x = g.x[:T].contiguous()
    L = g.layer
    args = (x, L.router_w, L.router_b, L.w13, L.w13_scales, L.b13, L.w2, L.w2_scales, L.b2, L.top_k)
    r_ref = moe.new_routing(T, L.E, L.top_k)
    r_na = moe.new_routing(T, L.E, L.top_k)
    ref = moe.forward(*args, routing=r_ref,
                      workspace=moe.new_workspace(T, L.H, L.E, L.top_k, L.I)).clone()
    got = _lib.forward_noalloc(*args, routing=r_na).clone()
    torch.cuda.synchronize()
    return ref, got, r_ref, r_na


@pytest.mark.parametrize("name", ["gpt-oss-20b-decode", "qwen3-235b-decode"])
def test_noalloc_matches_forward_on_two_calls(name):
    g = GpuLayer(SHAPES[name])
    T = g.shape.T
    assert moe.workspace_bytes(T, g.shape.H, g.shape.E, g.shape.top_k, g.shape.I) <= _lib.NOALLOC_BYTES
    for t in (T, T // 4 + 3):                  # the second call smaller (and ragged)
        ref, got, r_ref, r_na = _pair(g, t)
        same = torch.equal(ref, got)
        say(f"noalloc {name} T={t}: out identical {same}")
        assert same
        for k in r_ref:
            assert torch.equal(r_ref[k], r_na[k]), k
