"""The stochastic E2M1 rounding in the SR encoding kernel is written without
branches on the bits of |q|; tests/native/sr_round_check.c transcribes that
form and compares it with the oracle's rule (orc_e2m1_encode_sr, compiled
from oracle/nvfp4_oracle.c) for every non-NaN fp32 q, each with a hashed
8-bit random, plus every random value at the grid points.  Zero
mismatches required.  (The GPU parity tests then compare the kernel itself
with the oracle.)"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "sr_round_check.c")
ORC = os.path.join(ROOT, "oracle", "nvfp4_oracle.c")
EXE = os.path.join(ROOT, "_build", "sr_round_check")


def test_branch_free_sr_rounding_equals_the_oracle_rule():
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-pthread", "-o", EXE, SRC, ORC,
                    "-lm"], check=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stdout + res.stderr
    assert " 0 mismatches" in res.stdout, res.stdout
