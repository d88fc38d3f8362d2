"""The division-free e4m3 query quantisation of the MLA kernel
(``quantise8_rcp`` in device.h) rests on one fact: for a bf16 numerator, the
product with the correctly rounded reciprocal, corrected once by the exact
remainder, is the correctly rounded fp32 quotient.  ``csrc/rcp_division_check.c``
checks it over every fp32 divisor significand against every bf16 numerator
significand (2^30 pairs) with the host's IEEE arithmetic; the GPU's fused
multiply-add and multiply round the same way.  The queries' e4m3 codes are then
the oracle's (the e4m3 code of the fp32 quotient q / q_scale, "Xqa decode
kernels", timeline: FP8-Q)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_corrected_reciprocal_quotient_is_correctly_rounded(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "rcp_division_check")
    src = os.path.join(HERE, "csrc", "rcp_division_check.c")
    # -ffp-contract=off: the products and sums round exactly as written
    cmd = [cc, "-O2", "-ffp-contract=off", "-fopenmp", src, "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        cmd.remove("-fopenmp")
        r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    fields = dict(zip(out.stdout.split()[::2], map(int, out.stdout.split()[1::2])))
    assert fields["pairs"] == 2 ** 30
    assert fields["estimate_wrong"] > 0          # the correction is needed
    assert fields["corrected_wrong"] == 0, out.stdout
    assert out.returncode == 0
