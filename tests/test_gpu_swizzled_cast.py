"""GPU parity of the cast with swizzled scale output (nvfp4_quantize_swizzled)
against the CPU oracle: packed data and amax bit-exact with the ordinary
cast's oracle result, both scale matrices bit-exact with the oracle's swizzle
of the oracle's scales (the rowwise [M][K/16], the columnwise [K][M/16]).
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_bf16_amd as nv
from nvfp4_block_scaled_bf16_amd import workloads as W
from tests.gpu_util import Guarded, assert_bytes_equal, cast_spec, host, to_dev
from tests.test_gpu_parity import _crafted

pytestmark = pytest.mark.gpu

MODES = [nv.PER_TENSOR, nv.PER_TOKEN]
SHAPES = [(128, 128), (256, 384), (384, 1024), (1152, 640), (2048, 2176)]


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _swz_guarded(d, mode, rowwise=True, columnwise=True):
    M, K = d.shape
    g = Guarded(cast_spec(M, K, mode, rowwise, columnwise))   # swizzled matrices: M*K/16 bytes each
    nv.quantize_swizzled_into(d, mode, **g.views)
    return g


def _compare(out, ref, oracle):
    if isinstance(out, Guarded):
        out.check_guards()
    for k in ("row_q", "row_amax", "col_q", "col_amax"):
        if k in ref:
            assert_bytes_equal(host(out[k]).reshape(ref[k].shape), ref[k], k)
    if "row_sf" in ref:
        assert_bytes_equal(host(out["row_sf"]), oracle.swizzle_scales(ref["row_sf"]), "row_sf (swizzled)")
    if "col_sf" in ref:
        assert_bytes_equal(host(out["col_sf"]), oracle.swizzle_scales(ref["col_sf"]), "col_sf (swizzled)")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", SHAPES)
def test_swizzled_cast_shapes(oracle, shape, mode):
    M, K = shape
    x = W.row_scaled_with_outliers(M, K, 500 + M + K)
    _announce(f"swizzled cast M={M} K={K} mode={mode}")
    out = _swz_guarded(to_dev(x), mode)
    torch.cuda.synchronize()
    _compare(out, oracle.quantize(x, mode), oracle)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dirs", [(True, False), (False, True)])
def test_swizzled_cast_one_direction(oracle, mode, dirs):
    M, K = 384, 640
    x = W.normal(M, K, 501)
    _announce(f"swizzled cast one direction {dirs} mode={mode}")
    out = _swz_guarded(to_dev(x), mode, rowwise=dirs[0], columnwise=dirs[1])
    torch.cuda.synchronize()
    _compare(out, oracle.quantize(x, mode, rowwise=dirs[0], columnwise=dirs[1]), oracle)


@pytest.mark.parametrize("mode", MODES)
def test_swizzled_cast_exact_path(oracle, mode):
    # blocks outside the fast path's range take the exact path, which writes
    # its own rowwise scales
    x = _crafted(M=128, K=1024, seed=5)
    _announce(f"swizzled cast crafted edges mode={mode}")
    out = _swz_guarded(to_dev(x), mode)
    torch.cuda.synchronize()
    _compare(out, oracle.quantize(x, mode), oracle)


def test_swizzled_cast_c3_full(oracle):
    x = W.c3(0)
    _announce("swizzled cast C3 16384x8192 per-token (full compare)")
    out = _swz_guarded(to_dev(x), nv.PER_TOKEN)
    torch.cuda.synchronize()
    _compare(out, oracle.quantize(x, nv.PER_TOKEN), oracle)


def test_swizzled_cast_feeds_swizzled_gemm(oracle):
    # the swizzled outputs go straight into the GEMM that reads them, equal
    # bit for bit to the plain cast + plain GEMM
    M, N, K = 256, 384, 512
    xa, xb = W.row_scaled_with_outliers(M, K, 502), W.weight_with_outliers(N, K, 503)
    _announce("swizzled cast -> swizzled GEMM")
    sa = nv.quantize_swizzled(to_dev(xa), nv.PER_TOKEN, columnwise=False)
    sb = nv.quantize_swizzled(to_dev(xb), nv.PER_TOKEN, columnwise=False)
    pa = nv.quantize(to_dev(xa), nv.PER_TOKEN, columnwise=False)
    pb = nv.quantize(to_dev(xb), nv.PER_TOKEN, columnwise=False)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    nv.gemm_swizzled_into(out, sa["row_q"], sa["row_sf"], sa["row_amax"], sb["row_q"], sb["row_sf"], sb["row_amax"])
    plain = nv.gemm(pa["row_q"], pa["row_sf"], pa["row_amax"], pb["row_q"], pb["row_sf"], pb["row_amax"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), plain.view(torch.int32))


def test_swizzled_cast_empty_tensor():
    # output buffers are non-empty allocations (NULL means "not requested")
    _announce("swizzled cast empty M=0 K=128")
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda:0")
    dummy = lambda dt: torch.full((64,), 7, dtype=dt, device="cuda:0")
    ca = torch.full((128,), 7.0, dtype=torch.float32, device="cuda:0")
    nv.quantize_swizzled_into(x, nv.PER_TOKEN, col_q=dummy(torch.uint8), col_sf=dummy(torch.uint8), col_amax=ca)
    torch.cuda.synchronize()
    assert not host(ca).any()
