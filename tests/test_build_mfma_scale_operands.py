"""Build-time check of the scaled matrix-core instructions of the GEMM kernels.

v_mfma_scale_f32_16x16x128_f8f6f4 reads its two E8M0 scale operands from VGPRs.  The
compiler does not keep its result registers apart from those scale registers (seen with
a result that overwrote the activation scale it still had to read, which gave products
off by powers of two).  The kernels accumulate every scaled MFMA in place, so the result
is the live accumulator, and the row-run tiles keep both scales live past each instruction;
this test compiles the GEMM source and the fused decode kernel (which inlines the row-run
tiles) with the library's flags and checks that no scaled MFMA anywhere in them writes a
register that holds one of its scales.
"""
import os
import re
import subprocess

import pytest

from sparse_moe_ffn_gemm_amd import build as B


def _regs(tok: str):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("source", ["gemm.hip", "fused.hip"])
def test_no_scaled_mfma_result_overlaps_its_scale_operands(tmp_path, source):
    src = os.path.join(B.CSRC, source)
    asm = tmp_path / (source[:-4] + ".s")
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    r = subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", str(asm)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kern, n, bad = None, 0, []
    for line in asm.read_text().splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            kern = m.group(1)
        if "v_mfma_scale_f32" not in line:
            continue
        ops = [o.strip() for o in line.split("op_sel")[0].split(None, 1)[1].split(",")]
        n += 1
        dst, sa, sb = _regs(ops[0]), _regs(ops[4]), _regs(ops[5])
        if dst & (sa | sb):
            bad.append((kern, line.strip()))
    assert n > 0
    assert not bad, bad[:5]
