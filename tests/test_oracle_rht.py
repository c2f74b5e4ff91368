"""Pins of the oracle's random Hadamard transform (CPU only).

The per-token recipe page lists a random Hadamard transform as an opt-in for
the columnwise direction (TransformerEngine PR #3045, "Changes",
per_token_rht; never on rows).  The oracle reads it as y = (1/4) H16 D x per
16-element columnwise block, D a diagonal of signs from a 16-bit mask,
evaluated as the binary32 butterfly and rounded to bf16.  Pinned against:
  - scipy's Sylvester Hadamard matrix (a library routine): exact equality
    where every partial sum is representable, and the binary32 + bf16
    rounding bound on heavy-tailed data;
  - exact properties: the transform is its own inverse up to D, unit
    vectors map to signed columns of H16 / 4, the sign mask flips inputs,
    ties round to even, norms are preserved (Parseval);
  - the column-block structure of rht_columns and the wiring of
    quantize_rht (rowwise = ordinary cast of x, columnwise = ordinary cast of
    the transformed tensor with its own amax).
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
from nvfp4_block_scaled_bf16_amd import workloads as W

H16 = scipy.linalg.hadamard(16).astype(np.float64)


def _signs(mask):
    return np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(16)])


def _f(b):
    return W.bf16_to_f32(b).astype(np.float64)


def _exact(blocks_f64, mask):
    return (blocks_f64 * _signs(mask)) @ H16.T / 4.0


@pytest.mark.parametrize("mask", [0x0000, 0xFFFF, 0xA5C3, 0x1234])
def test_exact_on_small_integers(mask):
    rng = np.random.Generator(np.random.PCG64(1))
    x = rng.integers(-8, 9, size=(200, 16)).astype(np.float32)
    y = _f(oracle.rht16(W.bf16_from_f32(x), mask))
    assert np.array_equal(y, _exact(x.astype(np.float64), mask))


@pytest.mark.parametrize("mask", [0x0000, 0x9E37])
def test_within_rounding_bound_on_heavy_tails(mask):
    x = W.student_t(64, 256, 7).reshape(-1, 16)
    xf = _f(x)
    y = _f(oracle.rht16(x, mask))
    ex = _exact(xf, mask)
    s = np.abs(xf).sum(axis=1, keepdims=True)
    # butterfly: 4 roundings of partial sums bounded by sum|x|, then / 4;
    # bf16 (8 significant bits): half an ulp, at most 2^-8 relative
    bound = 2.0 ** -24 * s + 2.0 ** -8 * (np.abs(ex) + 2.0 ** -24 * s)
    assert np.all(np.abs(y - ex) <= bound)
    assert np.any(y != 0)


def test_inverse_recovers_input():
    rng = np.random.Generator(np.random.PCG64(2))
    x = rng.integers(-8, 9, size=(50, 16)).astype(np.float64)
    mask = 0x5A3C
    y = _f(oracle.rht16(W.bf16_from_f32(x.astype(np.float32)), mask))
    back = (y @ H16.T / 4.0) * _signs(mask)
    assert np.array_equal(back, x)


def test_unit_vectors_give_signed_hadamard_columns():
    mask = 0x00F0
    e = np.eye(16, dtype=np.float32)
    y = _f(oracle.rht16(W.bf16_from_f32(e), mask))
    for j in range(16):
        assert np.array_equal(y[j], H16[:, j] * _signs(mask)[j] / 4.0)


def test_sign_mask_flips_inputs():
    x = W.normal(8, 16, 3)
    flipped = x.copy()
    mask = 0xC00F
    for j in range(16):
        if (mask >> j) & 1:
            flipped[:, j] ^= np.uint16(0x8000)
    assert np.array_equal(oracle.rht16(x, mask), oracle.rht16(flipped, 0))


def test_ties_round_to_even():
    x = np.zeros((2, 16), np.float32)
    x[0, 0], x[0, 1] = 1.0, 2.0 ** -8          # 1 + 2^-8: halfway, even is 1
    x[1, 0], x[1, 1] = 1.0, 3 * 2.0 ** -8      # 1 + 3*2^-8: halfway, even is 1 + 2^-6
    y = _f(oracle.rht16(W.bf16_from_f32(x), 0))
    assert y[0, 0] == 0.25
    assert y[1, 0] == (1 + 2.0 ** -6) / 4
    assert y[0, 1] == (1 - 2.0 ** -8) / 4       # representable: no rounding


def test_parseval():
    x = W.normal(32, 64, 4).reshape(-1, 16)
    xf, y = _f(x), _f(oracle.rht16(x, 0xBEEF))
    # H16 / 4 is orthonormal: the transform keeps the norm up to rounding
    assert np.allclose((y ** 2).sum(axis=1), (xf ** 2).sum(axis=1), rtol=2.0 ** -6)


def test_rht_columns_block_structure():
    x = W.row_scaled_with_outliers(64, 40, 5)
    mask = 0x0F0F
    y = oracle.rht_columns(x, mask)
    # each 16-row block of each column is one transform
    for r0 in (0, 48):
        for k in (0, 17, 39):
            assert np.array_equal(y[r0:r0 + 16, k], oracle.rht16(x[r0:r0 + 16, k][None], mask)[0])
    # columns are independent: permuting them commutes with the transform
    perm = np.random.Generator(np.random.PCG64(6)).permutation(40)
    assert np.array_equal(oracle.rht_columns(x[:, perm], mask), y[:, perm])
    with pytest.raises(ValueError):
        oracle.rht_columns(x[:40], mask)


@pytest.mark.parametrize("mode", [oracle.PER_TENSOR, oracle.PER_TOKEN])
def test_quantize_rht_wiring(mode):
    x = W.row_scaled_with_outliers(96, 64, 8)
    mask = 0x3C5A
    out = oracle.quantize_rht(x, mode, mask)
    plain = oracle.quantize(x, mode)
    for k in ("row_q", "row_sf", "row_amax"):
        assert np.array_equal(out[k], plain[k])
    yf = _f(oracle.rht_columns(x, mask))
    if mode == oracle.PER_TENSOR:
        assert out["col_amax"][0] == np.float32(np.abs(yf).max())
    else:
        assert np.array_equal(out["col_amax"], np.abs(yf).max(axis=0).astype(np.float32))
    # the columnwise codes decode to the transformed tensor within the
    # NVFP4 step: half the largest E2M1 gap (1) times the block divisor,
    # which is b / 6 up to the E4M3 rounding of the scale (below 7 %)
    deq = oracle.dequantize(out["col_q"], out["col_sf"], out["col_amax"], 64, 96, mode == oracle.PER_TOKEN)
    ref = yf.T
    blk = np.abs(ref).reshape(64, -1, 16).max(axis=2, keepdims=True)
    assert np.all(np.abs(deq.reshape(64, -1, 16) - ref.reshape(64, -1, 16)) <= blk / 6 * 1.0 * 1.07 + 1e-30)
