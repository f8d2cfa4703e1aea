"""The routing and selection kernels divide each exponential by its row's sum with
three instructions (a product by the correctly rounded reciprocal, an exact
fma remainder, one fma correction) instead of an IEEE division.  This CPU test
compiles the same three steps in C and checks them against IEEE binary32
division over the callers' domain: every e in [2^-30, 1] for several l, random
pairs, and quotients next to rounding midpoints."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_three_step_quotient_matches_ieee_division(tmp_path):
    exe = str(tmp_path / "quotient_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-mfma", os.path.join(ROOT, "tests", "quotient_check.c"),
                    "-o", exe, "-lm"], check=True, capture_output=True, text=True)
    r = subprocess.run([exe, "4", "30000000", "60000000"], capture_output=True, text=True, timeout=580)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 mismatched" in r.stdout, r.stdout
