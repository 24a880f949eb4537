"""Host-side checks of arithmetic identities the HIP kernels rely on (no GPU).

The INT8 quantization kernel forms fp32(x / s) without a division per
element (reciprocal once per row, then Markstein's fma correction). The codes
must stay bit-identical to rint(fp32(x / s)), so the identity is checked here
on the host with C's IEEE division and fmaf over random blocks and over
quotients next to every rounding boundary k + 1/2.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_division_free_quotient_is_correctly_rounded(tmp_path):
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", os.path.join(HERE, "host", "quotient_check.c"),
                    "-o", str(exe), "-lm"], check=True)
    res = subprocess.run([str(exe), "20000000"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert " 0 mismatches" in res.stdout
