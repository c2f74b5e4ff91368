"""Stream capture: casts recorded into a graph (torch.cuda.CUDAGraph) and
replayed several times, with eager work and synchronizations between the
replays, give the oracle's result on every replay.  On a capturing stream the
library takes launch paths without cross-workgroup waits (their arrival
counts come from the host at each call and would be frozen into the graph);
the outputs are refilled with a canary before each replay, so a replay that
skipped a write would show."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_bf16_amd as nv
from nvfp4_block_scaled_bf16_amd import workloads as W
from tests.gpu_util import CANARY, Guarded, assert_bytes_equal, cast_spec, compare_cast, host, to_dev

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _refill(out):
    for v in out.views.values():
        v.view(torch.uint8).fill_(CANARY)


@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
@pytest.mark.parametrize("shape,dirs", [((4096, 4096), (True, True)), ((272, 528), (True, True)),
                                        ((1072, 544), (False, True)), ((96, 1040), (True, False))])
def test_capture_and_replay(oracle, mode, shape, dirs):
    M, K = shape
    row, col = dirs
    x = W.row_scaled_with_outliers(M, K, 1200 + M)
    _announce(f"capture quantize mode={mode} shape={shape} row={row} col={col}")
    d = to_dev(x)
    out = Guarded(cast_spec(M, K, mode, row, col))
    ref = oracle.quantize(x, mode, rowwise=row, columnwise=col)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.quantize_into(d, mode, **out.views)
    torch.cuda.synchronize()
    for rep in range(3):
        _refill(out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare_cast(out, ref)


def test_capture_calibrate_replays_accumulate(oracle):
    """Each replay applies the decayed update once more: buf follows the
    oracle's accumulate over the replays."""
    M, K = 2048, 8192
    x = W.row_scaled_with_outliers(M, K, 1300)
    _announce("capture quantize_calibrate per-token 2048x8192")
    d = to_dev(x)
    out = Guarded(cast_spec(M, K, nv.PER_TOKEN))
    buf = torch.full((1,), 1e4, dtype=torch.float32, device="cuda:0")
    ref = oracle.quantize(x, nv.PER_TOKEN)
    A = np.array([oracle.amax_tensor(x)], np.float32)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.quantize_calibrate_into(d, nv.PER_TOKEN, buf, 0.5, **out.views)
    torch.cuda.synchronize()
    ref_buf = np.array([1e4], np.float32)
    buf.fill_(1e4)
    for rep in range(4):
        _refill(out)
        g.replay()
        torch.cuda.synchronize()
        compare_cast(out, ref)
        ref_buf = oracle.amax_accumulate(ref_buf, A, 0.5)
        assert_bytes_equal(host(buf), ref_buf, f"buf after replay {rep}")


@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
def test_capture_rht_replays(oracle, mode):
    """The Hadamard-transform cast under capture: a fill launch zeroes its
    amax outputs (no waits), and every replay gives the oracle's result."""
    M, K, mask = 1072, 544, 0xA5C3
    x = W.row_scaled_with_outliers(M, K, 1400)
    _announce(f"capture quantize_rht mode={mode} {M}x{K}")
    d = to_dev(x)
    out = Guarded(cast_spec(M, K, mode, True, True))
    ref = oracle.quantize_rht(x, mode, mask)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.quantize_rht_into(d, mode, mask, **out.views)
    torch.cuda.synchronize()
    for rep in range(3):
        _refill(out)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        compare_cast(out, ref)
