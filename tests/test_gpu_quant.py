"""GPU parity of the quantisers: weight codes/scales and activation codes/scales are
bit-exact against the oracle (same fp32 rule, same rounding)."""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_gemm_amd as moe
from oracle import moe_ref as R
from synth import SHAPES, expert_weights, make_inputs, f32_to_bf16_bits
from gpu_helpers import bf16_dev, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(3, 512, 256), (2, 384, 192), (1, 5760, 2880), (2, 192, 320),
                                   (1, 64, 64)])
def test_weight_quant_bit_exact(shape):
    say(f"weight quant {shape}")
    rng = np.random.default_rng(sum(shape))
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    if shape[1] >= 128 and shape[2] >= 128:
        w[0, :128, :128] = 0.0          # all-zero block -> scale 1, codes 0
    codes, scales = moe.quantize_weights(torch.from_numpy(w).cuda())
    rc, rs = R.quantize_blocks(w)
    assert np.array_equal(scales.cpu().numpy(), rs)
    got = codes.cpu().numpy()
    assert np.array_equal(got, rc), f"{(got != rc).sum()} codes differ"


@pytest.mark.parametrize("name", ["gpt-oss-120b-prefill", "qwen3-235b-prefill", "deepseek-v3-skewed"])
def test_weight_quant_sampled_experts(name):
    shape = SHAPES[name]
    for which in ("w13", "w2"):
        for e in (0, shape.E - 1):
            say(f"weight quant {name} {which} expert {e}")
            w = expert_weights(shape, which, e, "cuda")
            codes, scales = moe.quantize_weights(w)
            rc, rs = R.quantize_blocks(w.cpu().numpy())
            assert np.array_equal(scales.cpu().numpy(), rs)
            assert np.array_equal(codes.cpu().numpy(), rc)


def test_e4m3_conversion_every_bf16_value():
    """Groups whose first element is 448 have scale exactly 1, so the code of every other
    element is the e4m3 rounding of that bf16 value itself: sweep all finite bf16 values
    with |v| <= 448 (ties, subnormals and signed zeros included)."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = (allbits.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    test_bits = allbits[keep]
    per = 127
    n_groups = -(-test_bits.size // per)
    x = np.zeros((n_groups, 128), np.uint16)
    x[:, 0] = f32_to_bf16_bits(np.array([448.0], np.float32))[0]
    flat = np.zeros(n_groups * per, np.uint16)
    flat[:test_bits.size] = test_bits
    x[:, 1:] = flat.reshape(n_groups, per)
    # rows of H = 128 * 4 groups
    pad_rows = (-n_groups) % 4
    x = np.concatenate([x, np.tile(x[:1], (pad_rows, 1))]).reshape(-1, 512)
    say(f"e4m3 sweep over {test_bits.size} bf16 values")
    codes, scales = moe.quantize_activations(bf16_dev(x))
    assert np.all(scales.cpu().numpy() == 1.0)
    ref = R.e4m3_encode((x.astype(np.uint32) << 16).view(np.float32))
    got = codes.cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, [(hex(int(x[i, j])), hex(int(got[i, j])), hex(int(ref[i, j])))
                           for i, j in bad[:10]]


@pytest.mark.parametrize("name", ["tiny", "gpt-oss-20b-decode", "gpt-oss-120b-prefill",
                                  "deepseek-v3-skewed"])
def test_activation_quant_bit_exact(name):
    li = make_inputs(SHAPES[name])
    say(f"activation quant {name}")
    codes, scales = moe.quantize_activations(bf16_dev(li.x))
    x32 = (li.x.astype(np.uint32) << 16).view(np.float32)
    rc, rs = R.quantize_activations(x32)
    assert np.array_equal(scales.cpu().numpy(), rs)
    got = codes.cpu().numpy()
    assert np.array_equal(got, rc), f"{(got != rc).sum()} codes differ"
