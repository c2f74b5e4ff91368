"""GPU parity of the Hadamard-transform cast (nvfp4_quantize_rht) against the
CPU oracle: bit-exact on every output byte and on the fp32 amax bits.  The
transform's binary32 butterfly, its bf16 rounding, the columnwise amax of the
transformed tensor and the cast are all decided in binary32 on both sides.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_bf16_amd as nv
from nvfp4_block_scaled_bf16_amd import workloads as W
from tests.gpu_util import Guarded, cast_spec, compare_cast, host, to_dev

pytestmark = pytest.mark.gpu

MODES = [nv.PER_TENSOR, nv.PER_TOKEN]
# several 256-column and 128/512-row tiles, ragged tails
SHAPES = [(16, 16), (32, 512), (48, 1040), (272, 528), (1072, 544), (2048, 48), (528, 8208)]
MASKS = [0x0000, 0xFFFF, 0xA5C3]


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _rht_guarded(d, mode, mask, rowwise=True):
    M, K = d.shape
    g = Guarded(cast_spec(M, K, mode, rowwise, True))
    nv.quantize_rht_into(d, mode, mask, **g.views)
    return g


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", SHAPES)
def test_rht_small_shapes(oracle, shape, mode, mask):
    M, K = shape
    x = W.row_scaled_with_outliers(M, K, 300 + M + K)
    _announce(f"rht M={M} K={K} mode={mode} mask={mask:#06x}")
    out = _rht_guarded(to_dev(x), mode, mask)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize_rht(x, mode, mask))


@pytest.mark.parametrize("mode", MODES)
def test_rht_columnwise_only_narrow(oracle, mode):
    # K % 16 != 0 is allowed without rowwise output
    M, K = 96, 24
    x = W.normal(M, K, 77)
    _announce(f"rht columnwise only M={M} K={K}")
    out = _rht_guarded(to_dev(x), mode, 0x1234, rowwise=False)
    torch.cuda.synchronize()
    assert "row_q" not in out
    compare_cast(out, oracle.quantize_rht(x, mode, 0x1234, rowwise=False))


@pytest.mark.parametrize("mode", MODES)
def test_rht_crafted_edges(oracle, mode):
    # zero columns, a column of one repeated value (the transform maps it to a
    # single nonzero per block), subnormal and huge finite values (the exact
    # path), and ties of the bf16 rounding
    M, K = 64, 256
    x = W.normal(M, K, 78).copy()
    x[:, 0:8] = 0
    x[:, 8:16] = W.bf16_from_f32(np.full((M, 8), 3.0, np.float32))
    x[:, 16:24] = W.bf16_from_f32((W.bf16_to_f32(x[:, 16:24]) * np.float32(1e-39)).astype(np.float32))
    x[:, 24:32] = W.bf16_from_f32((W.bf16_to_f32(x[:, 24:32]) * np.float32(1e30)).astype(np.float32))
    tie = np.zeros((16, 8), np.float32)
    tie[0], tie[1] = 1.0, 2.0 ** -8
    x[:16, 32:40] = W.bf16_from_f32(tie)
    _announce(f"rht crafted edges mode={mode}")
    for mask in (0x0000, 0x8001):
        out = _rht_guarded(to_dev(x), mode, mask)
        torch.cuda.synchronize()
        compare_cast(out, oracle.quantize_rht(x, mode, mask))


def test_rht_c3_per_token_full(oracle):
    x = W.c3(0)
    mask = 0xB2E5
    _announce("rht C3 16384x8192 per-token (full compare)")
    out = _rht_guarded(to_dev(x), nv.PER_TOKEN, mask)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize_rht(x, nv.PER_TOKEN, mask))


def test_rht_inverse_through_dequantize(oracle):
    # the consumer's view: dequantize the columnwise output and undo the
    # transform with D H16 / 4; the result tracks x within the NVFP4 error
    M, K = 256, 64
    x = W.row_scaled_with_outliers(M, K, 79)
    mask = 0x0FF0
    out = nv.quantize_rht(to_dev(x), nv.PER_TOKEN, mask, rowwise=False)
    deq = host(nv.dequantize(out["col_q"], out["col_sf"], out["col_amax"], nv.PER_TOKEN)).astype(np.float64)   # [K][M]
    import scipy.linalg
    H = scipy.linalg.hadamard(16).astype(np.float64)
    s = np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(16)])
    back = ((deq.reshape(K, M // 16, 16) @ H.T / 4.0) * s).reshape(K, M).T
    xf = W.bf16_to_f32(x).astype(np.float64)
    err = np.linalg.norm(back - xf) / np.linalg.norm(xf)
    assert err < 0.2


def test_rht_empty_tensor():
    # M == 0: nothing to read; the per-column amax comes back zero (output
    # buffers are non-empty allocations: a NULL pointer means "not requested")
    _announce("rht empty M=0 K=32")
    x = torch.empty((0, 32), dtype=torch.bfloat16, device="cuda:0")
    dummy = lambda dt: torch.full((64,), 7, dtype=dt, device="cuda:0")
    ca = torch.full((32,), 7.0, dtype=torch.float32, device="cuda:0")
    nv.quantize_rht_into(x, nv.PER_TOKEN, 0x1234, col_q=dummy(torch.uint8), col_sf=dummy(torch.uint8), col_amax=ca)
    torch.cuda.synchronize()
    assert not host(ca).any()
