"""Host logic of bench.py (no GPU): the algorithmic byte and flop counts behind the roofline
figures, per weight format, and the refusal of multi-GPU runs."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import custom_shape  # noqa: E402


def _shape(expert_bias=True):
    # H = 192: a K tail of 64 (two 128-blocks, the second half full)
    return custom_shape(T=10, H=192, E=4, top_k=2, I=320, seed=1, expert_bias=expert_bias)


def test_flops_are_format_independent():
    sh = _shape()
    counts = np.array([5, 0, 9, 6])
    for fmt in ("block", "mxfp8", "mxfp4"):
        a = bench.algorithmic(sh, counts, fmt)
        rows = sh.T * sh.top_k
        assert a["gemm1"]["flops"] == 2 * rows * sh.H * 2 * sh.I
        assert a["gemm2"]["flops"] == 2 * rows * sh.I * sh.H
        assert a["active_experts"] == 3                      # an idle expert is never read


def test_weight_bytes_per_format():
    """Per active expert: e4m3 codes one byte per element, e2m1 half a byte; block scales
    4 bytes per 128x128 block, MX scales one byte per 32 elements along K.  The GEMMs'
    algorithmic bytes are their weights only (the intermediates x codes, h and y are
    implementation traffic); the layer adds x, the router and out."""
    sh = _shape(expert_bias=False)
    counts = np.array([1, 1, 0, 0])
    H, I, T, E = sh.H, sh.I, sh.T, sh.E
    exp = {
        "block": (2 * (2 * I * H + 5 * 2 * 4), 2 * (H * I + 2 * 3 * 4)),
        "mxfp8": (2 * (2 * I * H + 2 * I * H // 32), 2 * (H * I + H * I // 32)),
        "mxfp4": (2 * (I * H + 2 * I * H // 32), 2 * (H * I // 2 + H * I // 32)),
    }
    for fmt, (g1, g2) in exp.items():
        a = bench.algorithmic(sh, counts, fmt)
        assert a["gemm1"]["bytes"] == g1, fmt
        assert a["gemm2"]["bytes"] == g2, fmt
        assert a["layer_bytes"] == g1 + g2 + 2 * T * H * 2 + E * H * 4 + E * 4, fmt


def test_roofline_reports_both_fractions_and_leads_by_intensity():
    """The dominant kernel's line carries the FP8-MFMA and the HBM fraction; it leads with
    the matrix cores for a prefill-sized GEMM (intensity near the 625 flop/B ridge) and
    with HBM for a weight stream."""
    from synth import SHAPES
    for name, lead in (("gpt-oss-120b-prefill", "mfma"), ("gpt-oss-20b-decode", "hbm")):
        sh = SHAPES[name]
        counts = np.full(sh.E, sh.T * sh.top_k // sh.E)
        k = bench.algorithmic(sh, counts)["gemm1"]
        r = bench.roofline(k, 1e-3, sh, "block", "gemm1")
        assert r["bound"] == lead
        assert r["mfma_frac"] == round(k["flops"] / 1e-3 / 1e12 / 5000.0, 4)
        assert r["hbm_frac"] == round(k["bytes"] / 1e-3 / 1e9 / 8000.0, 4)
        assert r["frac"] == (r["mfma_frac"] if lead == "mfma" else r["hbm_frac"])


def test_biases_are_read_once_per_active_expert():
    counts = np.array([2, 0, 3, 0])
    with_b = bench.algorithmic(_shape(True), counts, "block")
    without = bench.algorithmic(_shape(False), counts, "block")
    sh = _shape()
    assert with_b["gemm1"]["bytes"] - without["gemm1"]["bytes"] == 2 * (2 * sh.I * 2)
    assert with_b["gemm2"]["bytes"] - without["gemm2"]["bytes"] == 2 * (sh.H * 2)


def test_multi_gpu_runs_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
