"""Pins of the oracle's NVFP4 GEMM consumer (CPU only).

The consumer on the per-token recipe page (TransformerEngine PR #3045,
Changes and sequence diagram) multiplies two NVFP4 operands and rescales by
the per-row / per-column outer amax in its epilogue.  The oracle computes it
in binary64 (oracle/nvfp4_oracle.c).  Pinned here against:
  - numpy's float64 matmul of the operands dequantized through the
    separately pinned codec decoders (a different route to the same sum);
  - exact properties: swapping the operands transposes the result, doubling
    an operand's amax doubles it, a zero operand gives zeros, and the bound
    is the same sum taken over absolute values.
"""
import numpy as np
import pytest

import oracle
from nvfp4_block_scaled_bf16_amd import workloads as W

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6], np.float64)


def _deq(q, sf):
    """block values g * D as float64 [R][C] from [R][C/2] bytes and [R][C/16] codes"""
    nib = np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], -1)
    g = np.array([oracle.e2m1_decode(int(n)) for n in range(16)], np.float64)[nib]
    d = np.array([oracle.e4m3_decode(int(c)) for c in range(256)], np.float64)[sf]
    return g * np.repeat(d, 16, axis=1)


def _operand(rows, K, seed, per_row):
    x = W.row_scaled_with_outliers(rows, K, seed)
    out = oracle.quantize(x, oracle.PER_TOKEN if per_row else oracle.PER_TENSOR, columnwise=False)
    return out["row_q"], out["row_sf"], out["row_amax"]


@pytest.mark.parametrize("per_row", [(True, True), (True, False), (False, True), (False, False)])
def test_gemm_matches_float64_matmul(per_row):
    M, N, K = 40, 24, 160
    aq, asf, aa = _operand(M, K, 1, per_row[0])
    bq, bsf, ba = _operand(N, K, 2, per_row[1])
    out, bound = oracle.gemm_nvfp4(aq, asf, aa, bq, bsf, ba)
    Sa = (aa / np.float32(2688)).astype(np.float32).astype(np.float64)
    Sb = (ba / np.float32(2688)).astype(np.float32).astype(np.float64)
    Sa = np.broadcast_to(Sa, (M,)) if Sa.size == 1 else Sa
    Sb = np.broadcast_to(Sb, (N,)) if Sb.size == 1 else Sb
    A, B = _deq(aq, asf), _deq(bq, bsf)
    ref = (A @ B.T) * Sa[:, None] * Sb[None, :]
    mag = (np.abs(A) @ np.abs(B).T) * Sa[:, None] * Sb[None, :]
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-300)
    assert np.allclose(bound, mag, rtol=1e-12, atol=1e-300)
    assert np.all(np.abs(out) <= bound * (1 + 1e-12))


def test_gemm_exact_properties():
    M, N, K = 16, 32, 64
    aq, asf, aa = _operand(M, K, 5, True)
    bq, bsf, ba = _operand(N, K, 6, True)
    ab, _ = oracle.gemm_nvfp4(aq, asf, aa, bq, bsf, ba)
    ba_, _ = oracle.gemm_nvfp4(bq, bsf, ba, aq, asf, aa)
    assert np.array_equal(ab, ba_.T)
    twice, _ = oracle.gemm_nvfp4(aq, asf, aa * np.float32(2), bq, bsf, ba)
    assert np.array_equal(twice, 2 * ab)
    zero, bound = oracle.gemm_nvfp4(np.zeros_like(aq), np.zeros_like(asf), aa, bq, bsf, ba)
    assert not zero.any() and not bound.any()
    with pytest.raises(ValueError):
        oracle.gemm_nvfp4(aq[:, :4], asf[:, :1], aa, bq, bsf, ba)
