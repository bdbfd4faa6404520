"""The division the FP8 quantize kernel uses (a reciprocal and one FMA correction,
see csrc/quant_fp8.hip) against correctly rounded float32 division, on the CPU:
``tests/csrc/quant_division_check.c`` built with gcc (glibc's fmaf is correctly
rounded) and run over 2e8 random pairs."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fma_division_gives_the_rounded_quotient(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "quant_division_check")
    subprocess.run([gcc, "-O2", "-o", exe, os.path.join(HERE, "csrc", "quant_division_check.c"), "-lm"],
                   check=True)
    r = subprocess.run([exe, "200000000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "mismatches 0" in r.stdout
