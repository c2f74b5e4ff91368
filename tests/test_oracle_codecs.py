"""Pins for the oracle's scalar codecs (E4M3 block scale, E2M1 element).

Each is checked against something other than the oracle itself: a
brute-force nearest-value search over every finite code, written from the
format definitions; torch's own float8_e4m3fn conversion (a library routine)
where it applies; and values fixed by the formats themselves.
"""
import numpy as np
import pytest
import torch

from tests import bruteforce as bf


def _around(values, span, step=1):
    """All float32 bit patterns within +/- span ulps of each value."""
    out = []
    for v in values:
        u = int(np.array([v], np.float32).view(np.uint32)[0])
        lo, hi = max(0, u - span), min(0x7F7FFFFF, u + span)
        out.append(np.arange(lo, hi + 1, step, dtype=np.uint32))
    return np.concatenate(out).view(np.float32)


# ------------------------------------------------------------------- E2M1

def _e2m1_brute_vec(q):
    """Vectorised brute force: nearest of the 8 magnitudes, ties to even code."""
    # beyond 2^30 every distance is huge; clamping keeps the ordering of the
    # distances (6 stays nearest) while float64 still resolves them exactly
    a = np.minimum(np.abs(q.astype(np.float64)), 2.0 ** 30)
    grid = np.array(bf.E2M1_GRID)
    d = np.abs(a[:, None] - grid[None, :])
    dmin = d.min(axis=1, keepdims=True)
    tied = d == dmin
    # prefer the even index among tied minima
    even_pref = np.where(tied & (np.arange(8)[None, :] % 2 == 0), 1, 0)
    pick = np.where(even_pref.any(axis=1), even_pref.argmax(axis=1), tied.argmax(axis=1))
    pick = np.where(np.isinf(a), 7, pick)
    sign = np.signbit(q).astype(np.uint8) * 8
    return (sign | pick.astype(np.uint8)).astype(np.uint8)


def test_e2m1_exhaustive_near_every_boundary(oracle):
    grid = bf.E2M1_GRID
    mids = [(grid[i] + grid[i + 1]) / 2 for i in range(7)]
    q = _around(grid[1:] + mids + [2.0 ** -149, 1e-30, 8.0, 12.0, 1e30], span=1 << 15)
    q = np.concatenate([q, [0.0, np.inf], q * -1.0, [-0.0, -np.inf]]).astype(np.float32)
    np.testing.assert_array_equal(oracle.e2m1_encode(q), _e2m1_brute_vec(q))


def test_e2m1_every_exponent_random_mantissa(oracle):
    rng = np.random.default_rng(7)
    exps = np.repeat(np.arange(0, 255, dtype=np.uint32), 2048)
    mant = rng.integers(0, 1 << 23, size=exps.size, dtype=np.uint32)
    sign = rng.integers(0, 2, size=exps.size, dtype=np.uint32) << 31
    q = (sign | (exps << 23) | mant).view(np.float32)
    np.testing.assert_array_equal(oracle.e2m1_encode(q), _e2m1_brute_vec(q))


def test_e2m1_grid_values_and_ties_exact(oracle):
    # every grid value maps to its own code; ties go to the even code
    for c, g in enumerate(bf.E2M1_GRID):
        assert oracle.e2m1_encode(np.array([g], np.float32))[0] == c
        assert oracle.e2m1_encode(np.array([-g], np.float32))[0] == 8 | c
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, c in ties.items():
        assert oracle.e2m1_encode(np.array([t], np.float32))[0] == c, t
    # saturation
    assert oracle.e2m1_encode(np.array([6.5, 1e9, np.inf], np.float32)).tolist() == [7, 7, 7]
    # decode is the inverse on the grid
    for n in range(16):
        g = bf.E2M1_GRID[n & 7]
        assert oracle.e2m1_decode(n) == (-g if n & 8 else g)


# ------------------------------------------------------------------- E4M3

def test_e4m3_decode_matches_torch_for_all_codes(oracle):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        got = oracle.e4m3_decode(c)
        if np.isnan(ref[c]):
            assert np.isnan(got), c
        else:
            assert got == ref[c], (c, got, ref[c])


def test_e4m3_decode_spec_values(oracle):
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert oracle.e4m3_decode(0x38) == 1.0
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6     # smallest normal
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9     # smallest subnormal
    assert oracle.e4m3_decode(0x07) == 7 * 2.0 ** -9  # largest subnormal


def test_e4m3_encode_bruteforce_near_every_code(oracle):
    vals = bf.E4M3_VALUES
    mids = [(vals[i] + vals[i + 1]) / 2 for i in range(126)]
    s = _around(vals[1:] + mids + [464.0, 480.0, 1e6], span=1 << 10, step=3)
    s = np.concatenate([s, np.array([0.0, 2.0 ** -149, 2.0 ** -11, 2.0 ** -10, np.inf], np.float32)])
    got = oracle.e4m3_encode(s)
    # brute force, vectorised over the 127 finite codes
    v = np.array(vals)
    d = np.abs(s.astype(np.float64)[:, None] - v[None, :])
    dmin = d.min(axis=1, keepdims=True)
    tied = d == dmin
    even = tied & (np.arange(127)[None, :] % 2 == 0)
    exp = np.where(even.any(axis=1), even.argmax(axis=1), tied.argmax(axis=1))
    exp = np.where(np.isinf(s), 0x7E, exp)
    np.testing.assert_array_equal(got, exp.astype(np.uint8))


def test_e4m3_encode_matches_torch_cast_below_464(oracle):
    rng = np.random.default_rng(3)
    s = np.concatenate([
        rng.uniform(0, 448, 200000), np.exp2(rng.uniform(-14, 8.8, 200000)),
        np.array(bf.E4M3_VALUES), [(a + b) / 2 for a, b in zip(bf.E4M3_VALUES, bf.E4M3_VALUES[1:])]
    ]).astype(np.float32)
    s = s[s <= 464.0]
    ref = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(s), ref)


def test_e4m3_saturates_and_never_emits_nan(oracle):
    s = np.array([448.0, 449.0, 464.0, 470.0, 1e10, np.inf], np.float32)
    assert oracle.e4m3_encode(s).tolist() == [0x7E] * 6
    rng = np.random.default_rng(5)
    big = np.exp2(rng.uniform(-20, 40, 100000)).astype(np.float32)
    assert oracle.e4m3_encode(big).max() <= 0x7E


@pytest.mark.parametrize("s,code", [(2.0 ** -10, 0x00), (1.5 * 2.0 ** -9, 0x02),
                                    (7.5 * 2.0 ** -9, 0x08), (1.1875, 0x3A), (1.0625, 0x38)])
def test_e4m3_tie_cases(oracle, s, code):
    # ties resolve to the even code (LSB of the mantissa field 0)
    assert oracle.e4m3_encode(np.array([s], np.float32))[0] == code
    assert bf.e4m3_brute(s) == code
