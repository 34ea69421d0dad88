"""Values the pages print, checked against the oracle's dispatch tables."""
import os

import numpy as np

from oracle import moe_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, val = line.split()
                vals[key] = float(val)
    return vals


def test_qwen3_prefill_tokens_per_expert():
    g = _read("qwen3_prefill_tokens_per_expert.txt")
    T, E, k = int(g["tokens"]), int(g["experts"]), int(g["top_k"])
    rng = np.random.default_rng(0)
    ids, gates = R.topk_softmax(rng.standard_normal((T, E)), k)
    counts, offsets, perm, inv = R.permute(ids, E)
    assert offsets[-1] == T * k
    assert counts.mean() == g["tokens_per_expert"]
    assert np.allclose(gates.sum(1), 1.0)
