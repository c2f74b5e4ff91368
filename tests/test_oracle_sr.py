"""Pins of the oracle's stochastic-rounding cast (CPU only).

The per-token recipe page (TransformerEngine PR #3045, Changes) lists a
stochastic-rounding variant without saying how randoms are drawn; the
library's definition is in oracle/nvfp4_oracle.c and include/nvfp4.h.  These
tests tie the oracle to things other than itself:
  - its Philox4x32-10 block function against rocRAND's implementation of the
    same published generator (Salmon et al., SC'11), compiled here from the
    ROCm headers;
  - its E2M1 stochastic rounding against the rule evaluated in exact rational
    arithmetic;
  - the exact round-up frequency over all 2^8 values of U, which puts the
    rounding's mean within 2^-8 of a grid step above the quotient;
  - the cast's structure against the deterministic cast: the same amax and
    block scales, and every element code one of the two grid neighbours of
    the exact quotient.
"""
import hashlib
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _philox_reference_binary():
    src = os.path.join(HERE, "native", "philox_ref.cpp")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    tag = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    out_dir = os.path.join(tempfile.gettempdir(), "nvfp4_philox_ref")
    os.makedirs(out_dir, exist_ok=True)
    exe = os.path.join(out_dir, f"philox_ref_{tag}")
    if not os.path.exists(exe):
        tmp = exe + f".{os.getpid()}"
        res = subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-o", tmp, src], capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("building the rocRAND reference failed:\n" + res.stderr[-2000:])
        shutil.move(tmp, exe)
    return exe


def test_philox_matches_rocrand_block_function():
    rng = np.random.default_rng(2024)
    ctr = rng.integers(0, 2**32, size=(1000, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2**32, size=(1000, 2), dtype=np.uint64).astype(np.uint32)
    edge_c = np.array([[0, 0, 0, 0], [2**32 - 1] * 4, [1, 0, 0, 0], [0, 0, 0, 2**31]], np.uint32)
    edge_k = np.array([[0, 0], [2**32 - 1] * 2, [0, 1], [2**31, 0]], np.uint32)
    ctr = np.concatenate([edge_c, ctr])
    key = np.concatenate([edge_k, key])
    lines = "\n".join(" ".join(str(int(v)) for v in list(c) + list(k)) for c, k in zip(ctr, key)) + "\n"
    res = subprocess.run([_philox_reference_binary()], input=lines, capture_output=True, text=True, check=True)
    ref = np.array([[int(t) for t in l.split()] for l in res.stdout.strip().split("\n")], np.uint64).astype(np.uint32)
    got = oracle.philox4x32_10(ctr, key)
    assert ref.shape == got.shape
    bad = np.nonzero((ref != got).any(axis=1))[0]
    assert bad.size == 0, f"Philox blocks differ from rocRAND at {bad[:5]}"


def _sr_rational(q, rnd):
    """The rounding rule in exact arithmetic: lo <= x < hi on the grid,
    up iff x - lo > U * (hi - lo), U = rnd / 2^8 (rnd the 8-bit random)."""
    sign = 8 if np.signbit(q) else 0
    x = Fraction(abs(float(q)))
    if x >= 6:
        return sign | 7
    c = max(i for i, g in enumerate(GRID) if g <= x)
    lo, hi = GRID[c], GRID[c + 1]
    u = Fraction(int(rnd), 2**8)
    return sign | (c + 1 if x - lo > u * (hi - lo) else c)


def test_sr_matches_rational_definition():
    rng = np.random.default_rng(7)
    qs = [0.0, -0.0, 6.0, -6.0, 7.5, 1e30]
    for g in [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5]:
        f = np.float32(g)
        qs += [float(f), float(np.nextafter(f, np.float32(0))), float(np.nextafter(f, np.float32(8)))]
    qs += list(rng.uniform(-7, 7, 3000).astype(np.float32))
    qs += list((rng.standard_normal(500) * 1e-3).astype(np.float32))
    q = np.array(qs, np.float32)
    rnd = rng.integers(0, 256, size=q.size, dtype=np.int64).astype(np.uint8)
    # randoms at the edges, and ones that make U * d land exactly on x - lo
    rnd[:50] = 0
    rnd[50:100] = 255
    got = oracle.e2m1_encode_sr(q, rnd)
    want = np.array([_sr_rational(a, r) for a, r in zip(q, rnd)], np.uint8)
    assert np.array_equal(got, want)
    # ties: U * d == x - lo exactly rounds down, one step of U more rounds up
    for x, lo, d in [(0.25, 0.0, 0.5), (1.25, 1.0, 0.5), (2.5, 2.0, 1.0), (5.0, 4.0, 2.0), (3.75, 3.0, 1.0)]:
        k = int(Fraction(x - lo) / Fraction(d) * 2**8)
        r = np.array([k, k - 1], np.uint8)
        codes = oracle.e2m1_encode_sr(np.array([x, x], np.float32), r)
        base = GRID.index(Fraction(lo))
        assert codes[0] == base and codes[1] == base + 1, (x, codes)


@pytest.mark.parametrize("x", [0.1, 0.3, 0.6, 1.3, 1.9999999, 2.2, 3.7, 4.4, 5.9, 1.0, 4.0])
def test_sr_round_up_count_is_exact(x):
    """Over all 2^8 values of U, rounding up happens exactly
    ceil(2^8 (x - lo) / d) times, so E[code value] lies in [x, x + 2^-8 d)."""
    xf = np.float32(x)
    X = Fraction(float(xf))
    c = max(i for i, g in enumerate(GRID) if g <= X)
    lo, d = GRID[c], GRID[c + 1] - GRID[c]
    t = (X - lo) / d * 2**8
    expect = -((-t.numerator) // t.denominator)   # ceil
    rnd = np.arange(2**8, dtype=np.int64).astype(np.uint8)
    codes = oracle.e2m1_encode_sr(np.full(2**8, xf, np.float32), rnd)
    ups = int(np.count_nonzero(codes == c + 1))
    assert int(np.count_nonzero((codes != c) & (codes != c + 1))) == 0
    assert ups == expect
    mean = lo + d * Fraction(ups, 2**8)
    assert X <= mean < X + d / 2**8


@pytest.mark.parametrize("mode", [oracle.PER_TENSOR, oracle.PER_TOKEN])
def test_sr_cast_against_deterministic_cast(mode):
    from nvfp4_block_scaled_bf16_amd import workloads as W
    x = W.row_scaled_with_outliers(64, 256, 11)
    det = oracle.quantize(x, mode)
    sr = oracle.quantize_sr(x, mode, seed=0x0123456789ABCDEF, offset=5)
    for k in ("row_sf", "col_sf", "row_amax", "col_amax"):
        assert np.array_equal(det[k], sr[k]), k
    # every element code is one of the two grid neighbours of the exact
    # quotient v / r (recomputed here in binary32, one rounding, as defined)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    for direction, v in (("row", xf), ("col", xf.T.copy())):
        amax = det[f"{direction}_amax"]
        A = amax if mode == oracle.PER_TOKEN else np.full(v.shape[0], amax[0], np.float32)
        S = (A / np.float32(2688)).astype(np.float32)
        D = np.array([oracle.e4m3_decode(c) for c in det[f"{direction}_sf"].ravel()], np.float32)
        r = (D.reshape(v.shape[0], -1) * S[:, None]).astype(np.float32)
        rr = np.repeat(r, 16, axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            qv = np.where(rr == 0, np.float32(0), v / rr).astype(np.float32)
        q = sr[f"{direction}_q"]
        nib = np.stack([q & 15, q >> 4], axis=-1).reshape(v.shape)
        mag = np.array([float(g) for g in GRID], np.float64)[nib & 7]
        a = np.abs(qv.astype(np.float64))
        lo = np.array([float(max(g for g in GRID if g <= Fraction(float(t)))) if t < 6 else 6.0 for t in a.ravel()]).reshape(a.shape)
        hi = np.array([float(min([g for g in GRID if g > Fraction(float(t))] or [Fraction(6)])) for t in a.ravel()]).reshape(a.shape)
        assert np.all((mag == lo) | (mag == hi)), direction
        assert np.all(((nib & 8) != 0) == np.signbit(v)), direction


def test_sr_seed_and_offset():
    from nvfp4_block_scaled_bf16_amd import workloads as W
    x = W.row_scaled_with_outliers(32, 128, 3)
    a = oracle.quantize_sr(x, oracle.PER_TOKEN, seed=1, offset=0)
    b = oracle.quantize_sr(x, oracle.PER_TOKEN, seed=1, offset=0)
    c = oracle.quantize_sr(x, oracle.PER_TOKEN, seed=1, offset=1)
    d = oracle.quantize_sr(x, oracle.PER_TOKEN, seed=2, offset=0)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["row_q"], c["row_q"]) and not np.array_equal(a["col_q"], c["col_q"])
    assert not np.array_equal(a["row_q"], d["row_q"])
    with pytest.raises(ValueError):
        oracle.quantize_sr(x, oracle.TILE_16x16, seed=1, offset=0)


@pytest.mark.parametrize("mode", [oracle.PER_TENSOR, oracle.PER_TOKEN])
def test_sr_counter_layout(mode):
    """Every element's random is byte i % 16 of the Philox block with counter
    (i / 16, vector, direction, offset) and key (seed low, seed high), the
    block's four words read as 16 little-endian bytes: rebuild each element's
    code from the two pinned pieces above and compare."""
    from nvfp4_block_scaled_bf16_amd import workloads as W
    M, K, seed, offset = 48, 96, 0xFEDCBA9876543210, 77
    x = W.row_scaled_with_outliers(M, K, 21)
    det = oracle.quantize(x, mode)
    sr = oracle.quantize_sr(x, mode, seed=seed, offset=offset)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32)
    for direction, dflag, v in (("row", 0, xf), ("col", 1, xf.T.copy())):
        n_vec, n = v.shape
        amax = det[f"{direction}_amax"]
        A = amax if mode == oracle.PER_TOKEN else np.full(n_vec, amax[0], np.float32)
        S = (A / np.float32(2688)).astype(np.float32)
        D = np.array([oracle.e4m3_decode(c) for c in det[f"{direction}_sf"].ravel()], np.float32)
        rr = np.repeat((D.reshape(n_vec, -1) * S[:, None]).astype(np.float32), 16, axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            qv = np.where(rr == 0, np.float32(0) * v, v / rr).astype(np.float32)
        vec, i = np.meshgrid(np.arange(n_vec), np.arange(n), indexing="ij")
        ctr = np.stack([i // 16, vec, np.full_like(i, dflag), np.full_like(i, offset)], -1).reshape(-1, 4).astype(np.uint32)
        words = oracle.philox4x32_10(ctr, np.tile(key, (ctr.shape[0], 1)))
        k = (i % 16).ravel()
        rnd = ((words[np.arange(ctr.shape[0]), k // 4] >> (8 * (k % 4)).astype(np.uint32)) & 0xFF).astype(np.uint8)
        want = oracle.e2m1_encode_sr(qv.ravel(), rnd).reshape(n_vec, n)
        zero = (rr == 0)
        want = np.where(zero, np.where(np.signbit(v), 8, 0), want).astype(np.uint8)
        q = sr[f"{direction}_q"]
        got = np.stack([q & 15, q >> 4], axis=-1).reshape(n_vec, n)
        assert np.array_equal(got, want), direction
