"""GPU parity of both launch schedules of the per-tensor / per-token cast.

The library runs these casts either as two launches (amax, then an encoding
pass that reads x again) or as one resident launch (amax phase, grid-wide
wait, encoding phase with the last tiles of each workgroup still in
registers).  Each test forces one schedule through nvfp4_set_schedule and
compares every output byte with the oracle, guards included.  The resident
cases are chosen to span its work split: runs of one, two (everything kept
in registers), three and four 256-row tiles per workgroup, a run count that
leaves the last band short, ragged last tiles, column strips narrower than
256, and a K too wide for the resident grid (where it falls back to two
launches).
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_bf16_amd as nv
from nvfp4_block_scaled_bf16_amd import workloads as W
from tests.gpu_util import Guarded, assert_bytes_equal, cast_spec, compare_cast, host, quantize_guarded, to_dev
from tests.test_gpu_parity import _crafted

pytestmark = pytest.mark.gpu

SCHEDULES = ["two_pass", "resident"]
# (M, K): with 256 compute units and K = 8192 (32 strips, 8 bands each) the
# runs are ceil(ceil(M / 256) / 8) tiles long
SHAPES = [(16, 16), (48, 1040), (272, 528), (1072, 544), (2048, 48), (64, 8192), (4096, 8192),
          (6096, 8192), (5088, 8192), (8000, 8192), (32, 65552)]


@pytest.fixture
def schedule(request):
    nv.set_schedule(request.param)
    yield request.param
    nv.set_schedule("auto")


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


@pytest.mark.parametrize("schedule", SCHEDULES, indirect=True)
@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
@pytest.mark.parametrize("shape", SHAPES)
def test_schedule_row_and_col(oracle, schedule, mode, shape):
    M, K = shape
    x = W.row_scaled_with_outliers(M, K, 900 + M + K)
    _announce(f"{schedule} quantize mode={mode} shape={shape}")
    out = quantize_guarded(to_dev(x), mode)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, mode))


@pytest.mark.parametrize("schedule", SCHEDULES, indirect=True)
@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
@pytest.mark.parametrize("dirs", [(True, False), (False, True)])
@pytest.mark.parametrize("shape", [(272, 528), (6096, 8192)])
def test_schedule_one_direction(oracle, schedule, mode, dirs, shape):
    M, K = shape
    row, col = dirs
    x = W.row_scaled_with_outliers(M, K, 950 + M)
    _announce(f"{schedule} quantize mode={mode} shape={shape} row={row} col={col}")
    out = quantize_guarded(to_dev(x), mode, rowwise=row, columnwise=col)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, mode, rowwise=row, columnwise=col))


@pytest.mark.parametrize("schedule", SCHEDULES, indirect=True)
@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
def test_schedule_crafted_edges(oracle, schedule, mode):
    """Zeros, subnormals, huge values and blocks on the exact path; tiled up
    so that the resident launch has exact-path steps in kept and re-read
    tiles alike."""
    x = np.tile(_crafted(), (40, 8))   # 2560 x 8192: runs of two tiles
    _announce(f"{schedule} crafted {x.shape} mode={mode}")
    out = quantize_guarded(to_dev(x), mode)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, mode))
    x = np.tile(_crafted(), (100, 8))   # 6400 x 8192: runs of four
    _announce(f"{schedule} crafted {x.shape} mode={mode}")
    out = quantize_guarded(to_dev(x), mode)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, mode))


@pytest.mark.parametrize("schedule", SCHEDULES, indirect=True)
@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
def test_schedule_calibrate_repeated(oracle, schedule, mode):
    """Calls in a row into the same buffers (the arrival counters advance
    from call to call), with the decayed calibration update folded in."""
    M, K = 4112, 8192
    buf = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    ref_buf = np.zeros(1, np.float32)
    out = Guarded(cast_spec(M, K, mode))
    for it, decay in enumerate([0.9, 0.5, 1.0, 0.0, 0.9]):
        x = W.row_scaled_with_outliers(M, K, 970 + it)
        if it == 2:
            x = (x & np.uint16(0x8000)) | ((x & np.uint16(0x7FFF)) >> np.uint16(1))   # smaller amax: decay shows
        _announce(f"{schedule} quantize_calibrate mode={mode} call {it}")
        nv.quantize_calibrate_into(to_dev(x), mode, buf, decay, **out.views)
        torch.cuda.synchronize()
        compare_cast(out, oracle.quantize(x, mode))
        ref_buf = oracle.amax_accumulate(ref_buf, np.array([oracle.amax_tensor(x)], np.float32), decay)
        assert_bytes_equal(host(buf), ref_buf, f"buf after call {it}")


@pytest.mark.parametrize("schedule", SCHEDULES, indirect=True)
def test_schedule_c3_per_token_full(oracle, schedule):
    x = W.c3(3)
    _announce(f"{schedule} C3 16384x8192 per-token row+col (full compare)")
    out = quantize_guarded(to_dev(x), nv.PER_TOKEN)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, nv.PER_TOKEN))


@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
def test_resident_wait_slots_wrap(oracle, mode):
    """140 resident casts queued back to back with no synchronization between
    them (more than twice the 64 wait slots, so every slot's arrival counter
    and flag words are taken again, with larger targets, by later launches),
    each into its own guarded outputs; then every output against the
    oracle."""
    nv.set_schedule("resident")
    try:
        M, K, n = 64, 1024, 140
        _announce(f"resident x{n} mode={mode} {M}x{K}")
        xs = [W.row_scaled_with_outliers(M, K, 5000 + i) for i in range(n)]
        dx = [to_dev(x) for x in xs]
        outs = [Guarded(cast_spec(M, K, mode)) for _ in range(n)]
        for d, o in zip(dx, outs):
            nv.quantize_into(d, mode, **o.views)
        torch.cuda.synchronize()
        for x, o in zip(xs, outs):
            compare_cast(o, oracle.quantize(x, mode))
    finally:
        nv.set_schedule("auto")
