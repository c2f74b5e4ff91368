"""The encode kernels replace per-element IEEE division by a per-block
reciprocal plus an FMA correction (Markstein's step).  This CPU test compiles
tests/native/div_identity_check.c, which compares the two bit for bit over
every bf16 significand against every fp32 significand of the divisor (the
three-op sequence is exact under power-of-two scaling while intermediates stay
normal, which the kernels' range test guarantees), plus tiny, subnormal and
signed-zero numerators, and requires zero mismatches."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "div_identity_check.c")
EXE = os.path.join(ROOT, "_build", "div_identity_check")


def test_fma_corrected_quotient_equals_ieee_division():
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-pthread", "-o", EXE, SRC, "-lm"], check=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert " 0 mismatches" in res.stdout
