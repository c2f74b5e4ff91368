"""Seeded synthetic inputs for the bf16 -> NVFP4 cast.

This module only draws random tensors and rounds them to bf16; it holds none
of the quantization arithmetic, so both the HIP path's tests/benchmark and
the CPU oracle can take their inputs from it.

Every tensor is drawn in float32 with numpy's PCG64, in fixed chunks of
``CHUNK_ROWS`` rows whose generators are spawned from ``SeedSequence(seed)``
(so the bytes do not depend on how many threads draw them), then rounded to
bf16 with round-to-nearest-even.  Tensors are returned as numpy ``uint16``
arrays of bf16 bit patterns, row-major.

Workloads (shapes and value distributions stand in for the activations,
MoE expert batches and weights the per-token recipe page talks about):

* ``c1``  per-tensor rowwise, 256 x 1024, N(0, 1), seed 1001.
* ``c2``  per-token row+col, 4096 x 4096: row r is N(0,1) * exp(u_r) with
          u_r ~ N(0, 1.5); 0.1 % of entries (uniform, without replacement)
          become +/-50 * exp(u_r) with a fair random sign; seed 1002.
* ``c3``  16384 x 8192 Student-t (df = 3, unit scale), seed 3000 + t for
          iteration t = 0..15.
* ``c4``  grouped MoE: 64 experts, counts = 128 * Multinomial(256, uniform),
          so they sum to 32768 and may be zero; expert scale s_e ~ U(0.5, 4);
          rows N(0, 1) * s_e, hidden 4096; seed 4004.
* ``c5``  8192 x 28672 weight, N(0, 0.02) with round(0.0005 * M * K)
          entries set to +/-1.0; seed 5005.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK_ROWS = 256


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns, nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def sha256(b: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(b).tobytes()).hexdigest()


def _chunked(seed: int, M: int, K: int, draw) -> np.ndarray:
    """Fill an M x K float32 array chunk by chunk; ``draw(gen, rows, K)``."""
    out = np.empty((M, K), np.float32)
    n = (M + CHUNK_ROWS - 1) // CHUNK_ROWS
    kids = np.random.SeedSequence(seed).spawn(max(n, 1))

    def work(i):
        r0 = i * CHUNK_ROWS
        r1 = min(M, r0 + CHUNK_ROWS)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        out[r0:r1] = draw(g, r1 - r0, K)

    if n > 0:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n)))
    return out


def normal(M: int, K: int, seed: int, sigma: float = 1.0) -> np.ndarray:
    f = _chunked(seed, M, K, lambda g, r, k: g.standard_normal((r, k), dtype=np.float32))
    if sigma != 1.0:
        f *= np.float32(sigma)
    return bf16_from_f32(f)


def student_t(M: int, K: int, seed: int, df: float = 3.0) -> np.ndarray:
    f = _chunked(seed, M, K, lambda g, r, k: g.standard_t(df, size=(r, k)).astype(np.float32))
    return bf16_from_f32(f)


def row_scaled_with_outliers(M: int, K: int, seed: int, row_sigma: float = 1.5,
                             outlier_frac: float = 0.001, outlier_mult: float = 50.0) -> np.ndarray:
    """N(0,1) * exp(u_r), u_r ~ N(0, row_sigma); a fraction of entries set to
    +/- outlier_mult * exp(u_r)."""
    z = _chunked(seed, M, K, lambda g, r, k: g.standard_normal((r, k), dtype=np.float32))
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    u = g.normal(0.0, row_sigma, size=M)
    fac = np.exp(u).astype(np.float32)
    z *= fac[:, None]
    n_out = int(round(outlier_frac * M * K))
    if n_out > 0:
        pos = g.choice(M * K, size=n_out, replace=False)
        sign = np.where(g.integers(0, 2, size=n_out) == 1, 1.0, -1.0).astype(np.float32)
        rows = pos // K
        z.reshape(-1)[pos] = sign * np.float32(outlier_mult) * fac[rows]
    return bf16_from_f32(z)


def weight_with_outliers(M: int, K: int, seed: int, sigma: float = 0.02,
                         outlier_frac: float = 0.0005, outlier_val: float = 1.0) -> np.ndarray:
    z = _chunked(seed, M, K, lambda g, r, k: g.standard_normal((r, k), dtype=np.float32))
    z *= np.float32(sigma)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    n_out = int(round(outlier_frac * M * K))
    if n_out > 0:
        pos = g.choice(M * K, size=n_out, replace=False)
        sign = np.where(g.integers(0, 2, size=n_out) == 1, 1.0, -1.0).astype(np.float32)
        z.reshape(-1)[pos] = sign * np.float32(outlier_val)
    return bf16_from_f32(z)


def moe_counts(seed: int, experts: int = 64, chunks: int = 256, align: int = 128) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2])))
    return (g.multinomial(chunks, [1.0 / experts] * experts) * align).astype(np.int64)


def moe_batch(seed: int, K: int = 4096, experts: int = 64, chunks: int = 256,
              align: int = 128, scale_lo: float = 0.5, scale_hi: float = 4.0):
    """Returns (x [sum(counts), K] bf16 bits, counts int64[experts])."""
    counts = moe_counts(seed, experts, chunks, align)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3])))
    scales = g.uniform(scale_lo, scale_hi, size=experts).astype(np.float32)
    T = int(counts.sum())
    z = _chunked(seed, T, K, lambda gg, r, k: gg.standard_normal((r, k), dtype=np.float32))
    row_scale = np.repeat(scales, counts)
    z *= row_scale[:, None]
    return bf16_from_f32(z), counts


def nvfp4_operand(rows: int, K: int, seed: int, per_row: bool = True):
    """Random NVFP4 operand bytes for the GEMM consumer: q [rows][K/2] with
    every nibble uniform over the 16 codes, sf [rows][K/16] uniform over the
    finite E4M3 codes 0x00..0x7E, amax ([rows] or [1]) log-uniform over
    [2^-4, 2^12].  Raw codes, not a cast of any tensor: they span the whole
    range of block scales (subnormal to 448) and element values."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    q = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    sf = rng.integers(0, 0x7F, size=(rows, K // 16), dtype=np.uint8)
    amax = np.exp2(rng.uniform(-4.0, 12.0, size=rows if per_row else 1)).astype(np.float32)
    return q, sf, amax


# ------------------------------------------------------------ named configs

def c1():
    return normal(256, 1024, 1001)


def c2():
    return row_scaled_with_outliers(4096, 4096, 1002)


def c3(t: int = 0):
    return student_t(16384, 8192, 3000 + t)


def c4():
    return moe_batch(4004)


def c5():
    return weight_with_outliers(8192, 28672, 5005)
