"""Exhaustive GPU sweeps of the gfx950 operations the cast's fast path
relies on, run through the library's own device helpers (test-only library
tests/native/libnvfp4_hwfacts.so, built by __graft_entry__.build()):

1. the hardware reciprocal v_rcp_f32 returns RD(1/r) or RU(1/r) -- exactly
   1/r when that is representable -- and the library's rcp_rn / rcp_rd give
   exactly RN(1/r) / RD(1/r), for every fp32 significand at exponents
   spanning [2^-64, 2^64] (the range the fast path uses them in);
2. the scaled FP4 conversion with scale 1.0 gives the CPU oracle's E2M1
   code (round to nearest, ties to the even code, saturating at 6, the sign
   copied, signed zeros and fp32 subnormals included) for every fp32 bit
   pattern that is not a NaN;
3. the packed bf16 conversion rounds every non-NaN fp32 pattern to nearest
   even (the integer rounding written out in the test library).

References: binary64 division on the host is exact enough to decide every
binary32 rounding of 1/r (1/r of a 24-bit significand never lies within
2^-49 relative of a binary32 rounding boundary without being on it); the
oracle's E2M1 encoder is pinned by its own brute-force tests.
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "native", "libnvfp4_hwfacts.so")


@pytest.fixture(scope="module")
def hw():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    p = ctypes.c_void_p
    L.hwf_rcp.argtypes = [ctypes.c_int, p, p, p]
    L.hwf_fp4.argtypes = [ctypes.c_uint64, ctypes.c_uint64, p]
    L.hwf_bf16.argtypes = [p, p]
    return L


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _down(y):
    """Next binary32 value toward zero (positive y)."""
    return (y.view(np.uint32) - np.uint32(1)).view(np.float32)


@pytest.mark.parametrize("e", [-64, -41, -20, -7, -1, 0, 1, 6, 21, 40, 63])
def test_reciprocal_rounding(hw, e):
    n = 1 << 23
    y0, yrn, yrd = (np.empty(n, np.float32) for _ in range(3))
    _announce(f"reciprocal sweep, exponent {e}")
    assert hw.hwf_rcp(e, y0.ctypes.data, yrn.ctypes.data, yrd.ctypes.data) == 0
    m = np.arange(n, dtype=np.uint32)
    r = ((np.uint32(e + 127) << np.uint32(23)) | m).view(np.float32)
    q = 1.0 / r.astype(np.float64)                       # exact to binary64
    rn = q.astype(np.float32)                             # RN to binary32
    # RD: rn when rn <= q, else the next value down
    rd = np.where(rn.astype(np.float64) <= q, rn, _down(rn))
    ru = np.where(rn.astype(np.float64) >= q, rn, np.nextafter(rn, np.float32(np.inf)))
    exact = rn.astype(np.float64) == q
    ok_hw = (y0 == rd) | (y0 == ru)
    assert ok_hw.all(), f"v_rcp_f32 outside [RD, RU] at significand {int(np.argmin(ok_hw)):#x}"
    assert (y0[exact] == rn[exact]).all(), "v_rcp_f32 inexact where 1/r is representable"
    bad = np.nonzero(yrn.view(np.uint32) != rn.view(np.uint32))[0]
    assert bad.size == 0, f"rcp_rn != RN(1/r) at {bad.size} significands, first {int(bad[0]):#x}"
    bad = np.nonzero(yrd.view(np.uint32) != rd.view(np.uint32))[0]
    assert bad.size == 0, f"rcp_rd != RD(1/r) at {bad.size} significands, first {int(bad[0]):#x}"


def test_fp4_conversion_all_patterns(hw, oracle):
    chunk = 1 << 26                                        # fp32 patterns per chunk
    nchunks = (1 << 32) // chunk
    _announce(f"scaled FP4 conversion: all 2^32 fp32 patterns in {nchunks} chunks")

    def one(c):
        start = c * chunk
        got = np.empty(chunk // 2, np.uint8)
        rc = hw.hwf_fp4(start, chunk // 2, got.ctypes.data)
        if rc != 0:
            return f"hwf_fp4 failed ({rc}) at chunk {c}"
        u = np.arange(chunk, dtype=np.uint32) + np.uint32(start)   # start + chunk <= 2^32
        nan = ((u & np.uint32(0x7F800000)) == np.uint32(0x7F800000)) & ((u & np.uint32(0x007FFFFF)) != 0)
        code = oracle.e2m1_encode(u.view(np.float32))
        lo, hi = got & np.uint8(0xF), got >> np.uint8(4)
        bad_lo = (lo != code[0::2]) & ~nan[0::2]
        bad_hi = (hi != code[1::2]) & ~nan[1::2]
        if bad_lo.any() or bad_hi.any():
            i = int(np.argmax(bad_lo)) * 2 if bad_lo.any() else int(np.argmax(bad_hi)) * 2 + 1
            g = lo[i // 2] if i % 2 == 0 else hi[i // 2]
            return f"pattern {int(u[i]):#010x}: hardware {int(g):#x}, oracle {int(code[i]):#x}"
        return None

    # the GPU calls are serialized by the runtime; the host checks overlap
    with ThreadPoolExecutor(max_workers=8) as ex:
        errors = [e for e in ex.map(one, range(nchunks)) if e]
    assert not errors, errors[:4]


def test_bf16_conversion_all_patterns(hw):
    _announce("packed bf16 conversion: all 2^32 fp32 patterns")
    bad = ctypes.c_ulonglong(0)
    first = ctypes.c_uint32(0)
    assert hw.hwf_bf16(ctypes.byref(bad), ctypes.byref(first)) == 0
    assert bad.value == 0, f"{bad.value} mismatches, the smallest at pattern {first.value:#010x}"
