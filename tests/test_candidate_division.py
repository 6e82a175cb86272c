"""The GPU scale search computes a candidate step's division by 7 as a product and one fma
correction (no IEEE division sequence).  This host check runs that arithmetic in C on every
significand of the binades that matter and requires the correctly rounded quotient each time."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_fma_division_by_7_is_correctly_rounded(tmp_path):
    exe = tmp_path / "div7_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), os.path.join(HERE, "div7_check.c"), "-lm"],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    assert int(out.strip()) == 0
