"""Blocks whose scale falls in the E4M3 subnormal range (0 < sf < 2^-6) stay
on the encode kernels' fast path, which takes their code as RNE(sf * 2^9) by
one float addition of 2^23 and their value as code * 2^-9;
tests/native/e4m3_sub_check.c compares both with the oracle's E4M3 encoder
and decoder (compiled from oracle/nvfp4_oracle.c) for every fp32 pattern in
that range.  Zero mismatches required.  (The GPU parity tests' crafted
inputs then compare the kernels themselves with the oracle.)"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "e4m3_sub_check.c")
ORC = os.path.join(ROOT, "oracle", "nvfp4_oracle.c")
EXE = os.path.join(ROOT, "_build", "e4m3_sub_check")


def test_subnormal_scale_code_equals_the_oracle_encoder():
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-o", EXE, SRC, ORC, "-lm",
                    "-lpthread"], check=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert " 0 mismatches" in res.stdout, res.stdout
