"""The FP8 activation quantiser's quotient (reciprocal, product, FMA
residual, one correction) against the correctly rounded division, over every
bf16 amax / x pair on the kernel's fast path; see quant_division_check.c.
Host only (gcc); the GPU tests then compare the kernel's codes with the
oracle bit for bit."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_quant_division_matches_correct_rounding(tmp_path):
    exe = str(tmp_path / "quant_division_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "quant_division_check.c"), "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert " 0 normal-quotient mismatches, 0 code mismatches" in r.stdout
