"""The quantizer's scale division shortcut (multiply by RN(1/15) plus one
fma correction) against the IEEE binary32 quotient, for every positive
finite binary32 range. Host-only: compiles a small C program with gcc."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_division_by_15_is_correctly_rounded_everywhere():
    src = os.path.join(HERE, "c", "div15_check.c")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "div15")
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                        "-o", exe, src, "-lm"], check=True, capture_output=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True,
                             timeout=600).stdout
    assert "mismatches fp32=0 bf16=0" in out, out
