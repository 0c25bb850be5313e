"""Host check of the quantize kernels' fast division (Markstein's correction
with the correctly rounded reciprocal of the scale): the C restatement in
tests/host/div_by_scale_check.c is built with gcc and run over every BF16
input at 3,000 scales (1,000 of them a few FP32 units from round values,
where a quotient taken through 1/s alone would round the other way).  The
GPU kernels themselves are checked against the oracle by the exhaustive
quantize tests."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_div_by_scale_matches_ieee_quotient(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.fail("gcc is needed to build the host check")
    exe = str(tmp_path / "div_by_scale_check")
    src = os.path.join(HERE, "host", "div_by_scale_check.c")
    flags = ["-O2", "-ffp-contract=off", "-o", exe, src, "-lm"]
    r = subprocess.run([gcc, "-mfma", *flags], capture_output=True, text=True)
    if r.returncode != 0:   # no FMA instructions: glibc's fmaf is still correctly rounded
        r = subprocess.run([gcc, *flags], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([exe, "3000"], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout
    assert "quotient mismatches 0, code mismatches 0" in out.stdout, out.stdout
