"""The cross-workgroup wait protocol (arrival counters with host-issued
bases, zero-first, the grid-wide wait with its published flag words, the
bounded give-up and its error word), checked on a CPU build: tests/native/sync_protocol_check.cpp models
it with one thread per workgroup over many launches that reuse a few slots,
with shuffled start times, and one forced give-up every 20 launches."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "sync_protocol_check.cpp")
EXE = os.path.join(ROOT, "_build", "sync_protocol_check")


def test_wait_protocol_on_cpu_threads():
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    subprocess.run(["g++", "-O2", "-std=c++17", "-pthread", "-o", EXE, SRC], check=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("OK "), res.stdout
