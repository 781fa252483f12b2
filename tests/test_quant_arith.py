"""The fused kernel forms each activation quotient from a two-term reciprocal (and a power-of-two
rescaling below 2^-64) instead of a division.  tests/native/quant_arith_check.c restates that recipe
in C and checks, over every pair of bf16 amax and bf16 x with |x| <= amax, that the resulting e4m3
code equals the code of the correctly rounded division.  Runs on the CPU in a few seconds."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_quotient_recipe_gives_the_division_codes(tmp_path):
    exe = tmp_path / "quant_arith_check"
    src = os.path.join(HERE, "native", "quant_arith_check.c")
    res = subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
                          src, "-o", str(exe), "-lm"], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "e4m3 code mismatches 0, scale mismatches 0" in run.stdout, run.stdout
