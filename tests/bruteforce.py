"""Pure-Python brute-force quantizer used to pin the C oracle.

Independent of the oracle: the E4M3 and E2M1 codes are found by searching
every finite code for the nearest value (ties to the even code), with the
code tables written from the format definitions (OCP FP8 E4M3: bias 7,
3 mantissa bits, max 448; E2M1: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).
The fp32 steps of the cast use numpy float32 scalars, i.e. single IEEE
binary32 operations, in the order the per-token recipe page and the
Model-Optimizer review of the FP8 block scale imply:
S = A/2688, sf = (b/6)/S, r = D*S, q = v/r.
Slow by design; only for small inputs.
"""
import math

import numpy as np

F = np.float32

E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e4m3_value(code: int) -> float:
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return m * 2.0 ** -9
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_VALUES = [e4m3_value(c) for c in range(127)]  # 0x00..0x7E, all finite


def nearest_code(x: float, values) -> int:
    """argmin |x - values[c]|, ties to the even code index."""
    best, bestd = None, None
    for c, v in enumerate(values):
        d = abs(x - v)
        if bestd is None or d < bestd or (d == bestd and c % 2 == 0 and best % 2 == 1):
            best, bestd = c, d
    return best


def e4m3_brute(s: float) -> int:
    # clamping huge values keeps the distance ordering exact in doubles
    return nearest_code(min(float(s), 2.0 ** 30), E4M3_VALUES)


def e2m1_brute(q: float) -> int:
    sign = 8 if math.copysign(1.0, q) < 0 else 0
    a = min(abs(float(q)), 2.0 ** 30)
    return sign | nearest_code(a, E2M1_GRID)


def bf16_value(bits: int) -> np.float32:
    return np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]


def quantize_vector_brute(v, A):
    """v: sequence of float32 values (n % 16 == 0); A: float32 outer amax."""
    v = [F(x) for x in v]
    A = F(A)
    S = F(A / F(2688.0))
    nibbles, scales = [], []
    for j in range(len(v) // 16):
        blk = v[16 * j:16 * j + 16]
        if S == F(0.0):
            code, r = 0, F(0.0)
        else:
            b = max(abs(x) for x in blk)
            sf = F(F(b / F(6.0)) / S)
            code = e4m3_brute(float(sf))
            r = F(F(E4M3_VALUES[code]) * S)
        scales.append(code)
        for x in blk:
            if r == F(0.0):
                nibbles.append(8 if math.copysign(1.0, float(x)) < 0 else 0)
            else:
                with np.errstate(over="ignore", divide="ignore"):
                    q = F(x / r)
                nibbles.append(e2m1_brute(float(q)))
    packed = [nibbles[2 * i] | (nibbles[2 * i + 1] << 4) for i in range(len(nibbles) // 2)]
    return np.array(packed, np.uint8), np.array(scales, np.uint8)


def amax_brute(vals) -> np.float32:
    m = F(0.0)
    for x in vals:
        if abs(F(x)) > m:
            m = abs(F(x))
    return m


def quantize_brute(x_bits: np.ndarray, mode: int):
    """Whole-tensor brute force on a bf16-bit matrix (small sizes only)."""
    M, K = x_bits.shape
    xf = [[bf16_value(int(x_bits[m, k])) for k in range(K)] for m in range(M)]
    out = {}
    if mode == 2:
        A = amax_brute([xf[m][k] for m in range(M) for k in range(K)])
        S = F(A / F(2688.0))
        row_q = np.zeros((M, K // 2), np.uint8)
        col_q = np.zeros((K, M // 2), np.uint8)
        row_sf = np.zeros((M, K // 16), np.uint8)
        col_sf = np.zeros((K, M // 16), np.uint8)
        nib = np.zeros((M, K), np.uint8)
        for I in range(M // 16):
            for J in range(K // 16):
                tile = [xf[16 * I + a][16 * J + b] for a in range(16) for b in range(16)]
                if S == F(0.0):
                    code, r = 0, F(0.0)
                else:
                    bmax = amax_brute(tile)
                    code = e4m3_brute(float(F(F(bmax / F(6.0)) / S)))
                    r = F(F(E4M3_VALUES[code]) * S)
                for a in range(16):
                    for b in range(16):
                        xv = xf[16 * I + a][16 * J + b]
                        if r == F(0.0):
                            n = 8 if math.copysign(1.0, float(xv)) < 0 else 0
                        else:
                            with np.errstate(over="ignore", divide="ignore"):
                                n = e2m1_brute(float(F(xv / r)))
                        nib[16 * I + a, 16 * J + b] = n
                    row_sf[16 * I:16 * I + 16, J] = code
                    col_sf[16 * J:16 * J + 16, I] = code
        row_q[:] = nib[:, 0::2] | (nib[:, 1::2] << 4)
        col_q[:] = nib.T[:, 0::2] | (nib.T[:, 1::2] << 4)
        out.update(row_q=row_q, row_sf=row_sf, col_q=col_q, col_sf=col_sf,
                   row_amax=np.full(M, A, np.float32), col_amax=np.full(K, A, np.float32))
        return out
    rows = [xf[m] for m in range(M)]
    cols = [[xf[m][k] for m in range(M)] for k in range(K)]
    if mode == 0:
        A = amax_brute([v for r in rows for v in r])
        ra = [A] * M
        ca = [A] * K
        out["row_amax"] = np.array([A], np.float32)
        out["col_amax"] = np.array([A], np.float32)
    else:
        ra = [amax_brute(r) for r in rows]
        ca = [amax_brute(c) for c in cols]
        out["row_amax"] = np.array(ra, np.float32)
        out["col_amax"] = np.array(ca, np.float32)
    rq, rs = zip(*[quantize_vector_brute(rows[m], ra[m]) for m in range(M)])
    cq, cs = zip(*[quantize_vector_brute(cols[k], ca[k]) for k in range(K)])
    out["row_q"], out["row_sf"] = np.stack(rq), np.stack(rs)
    out["col_q"], out["col_sf"] = np.stack(cq), np.stack(cs)
    return out
