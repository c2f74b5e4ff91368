"""Build tests/native/libnvfp4_hwfacts.so, the test-only GPU library that
sweeps the hardware operations the cast's fast path relies on (the tests in
tests/test_gpu_hwfacts.py load it).  Same flags as the product library."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "hwfacts.hip")
LIB = os.path.join(HERE, "libnvfp4_hwfacts.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    sys.path.insert(0, ROOT)
    from nvfp4_block_scaled_bf16_amd.build import FLAGS
    cmd = [HIPCC, *FLAGS, "-o", LIB + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr[-4000:])
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
