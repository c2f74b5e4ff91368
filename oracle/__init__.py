"""CPU oracle for the bf16 -> NVFP4 block-scaled cast (numpy front end).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` import this package; the product library
never does.  It shares no code with the HIP path: the arithmetic lives in
``nvfp4_oracle.c`` (plain C, one IEEE binary32 op per step), loaded here with
ctypes.  Inputs are bf16 bit patterns held as numpy ``uint16`` arrays.

Modes: 0 = per-tensor outer amax, 1 = per-token (per-row amax for rowwise
output, per-column amax for columnwise output), 2 = 16x16 tiles with the
per-tensor amax, emitted in the per-token layout.  See ``nvfp4_oracle.c`` for
the step-by-step definition and the pages each step follows.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libnvfp4_oracle.so")
_lib = None

PER_TENSOR, PER_TOKEN, TILE_16x16 = 0, 1, 2

_p = ctypes.c_void_p
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "orc_e4m3_encode_array": (None, [_p, _i64, _p]),
        "orc_e2m1_encode_array": (None, [_p, _i64, _p]),
        "orc_e4m3_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "orc_e2m1_decode": (ctypes.c_float, [ctypes.c_uint8]),
        "orc_quantize_vector": (None, [_p, _i64, ctypes.c_float, _p, _p]),
        "orc_amax_tensor": (ctypes.c_float, [_p, _i64, _i64, _i64]),
        "orc_amax_rows": (None, [_p, _i64, _i64, _i64, _p]),
        "orc_amax_cols": (None, [_p, _i64, _i64, _i64, _p]),
        "orc_encode_rowwise": (ctypes.c_int, [_p, _i64, _i64, _i64, ctypes.c_int, _p, _p, _p]),
        "orc_encode_colwise": (ctypes.c_int, [_p, _i64, _i64, _i64, ctypes.c_int, _p, _p, _p]),
        "orc_quantize": (ctypes.c_int, [_p, _i64, _i64, ctypes.c_int, _p, _p, _p, _p, _p, _p]),
        "orc_quantize_grouped": (ctypes.c_int, [_p, _i64, ctypes.c_int32, _p, _p, _p, _p, _p, _p, _p]),
        "orc_dequantize": (ctypes.c_int, [_p, _p, _p, _i64, _i64, ctypes.c_int, _p]),
        "orc_amax_accumulate": (None, [_p, _p, _i64, ctypes.c_float]),
        "orc_amax_accumulate_reduce": (None, [_p, _p, _i64, ctypes.c_float]),
        "orc_philox4x32_10_array": (None, [_p, _p, _i64, _p]),
        "orc_e2m1_encode_sr_array": (None, [_p, _p, _i64, _p]),
        "orc_quantize_vector_sr": (None, [_p, _i64, ctypes.c_float, _p, _p, ctypes.c_uint64, ctypes.c_uint32,
                                          ctypes.c_uint32, ctypes.c_uint32]),
        "orc_quantize_sr": (ctypes.c_int, [_p, _i64, _i64, ctypes.c_int, _p, _p, _p, _p, _p, _p,
                                           ctypes.c_uint64, ctypes.c_uint32]),
        "orc_gemm_nvfp4": (ctypes.c_int, [_p, _p, _p, ctypes.c_int, _p, _p, _p, ctypes.c_int, _i64, _i64, _i64,
                                          _p, _p]),
        "orc_rht16": (None, [_p, ctypes.c_uint32, _p]),
        "orc_swizzled_size": (_i64, [_i64, _i64]),
        "orc_swizzle_scales": (ctypes.c_int, [_p, _i64, _i64, _p]),
        "orc_unswizzle_scales": (ctypes.c_int, [_p, _i64, _i64, _p]),
        "orc_rht_columns": (ctypes.c_int, [_p, _i64, _i64, ctypes.c_uint32, _p]),
        "orc_quantize_per_token_threads": (ctypes.c_int, [_p, _i64, _i64, ctypes.c_int, _p, _p, _p, _p, _p, _p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _bf16(x):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (numpy uint16)")
    return x


# ------------------------------------------------------------------ codecs

def e4m3_encode(s):
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(s.shape, np.uint8)
    _load().orc_e4m3_encode_array(_ptr(s), s.size, _ptr(out))
    return out


def e2m1_encode(q):
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.empty(q.shape, np.uint8)
    _load().orc_e2m1_encode_array(_ptr(q), q.size, _ptr(out))
    return out


def e4m3_decode(code):
    return float(_load().orc_e4m3_decode(int(code)))


def e2m1_decode(nibble):
    return float(_load().orc_e2m1_decode(int(nibble)))


def quantize_vector(v, A):
    v = np.ascontiguousarray(v, dtype=np.float32)
    n = v.size
    q = np.empty(n // 2, np.uint8)
    sf = np.empty(n // 16, np.uint8)
    _load().orc_quantize_vector(_ptr(v), n, float(np.float32(A)), _ptr(q), _ptr(sf))
    return q, sf


# -------------------------------------------------------------------- amax

def amax_tensor(x):
    x = _bf16(x)
    M, K = x.shape
    return np.float32(_load().orc_amax_tensor(_ptr(x), M, K, K))


def amax_rows(x):
    x = _bf16(x)
    M, K = x.shape
    out = np.empty(M, np.float32)
    _load().orc_amax_rows(_ptr(x), M, K, K, _ptr(out))
    return out


def amax_cols(x):
    x = _bf16(x)
    M, K = x.shape
    out = np.empty(K, np.float32)
    _load().orc_amax_cols(_ptr(x), M, K, K, _ptr(out))
    return out


# ------------------------------------------------------------------ casts

def encode_rowwise(x, amax, per_vector, ld=None, rows=None, cols=None):
    """Rowwise encode with caller-supplied outer amax (scalar or per row).

    ``x`` may be a view into a wider row-major array when ``ld`` is given
    (used by the CPU baseline to split work into bands)."""
    amax = np.ascontiguousarray(np.atleast_1d(amax), dtype=np.float32)
    if ld is None:
        x = _bf16(x)
        M, K = x.shape
        ld = K
        base = x
        off = 0
    else:
        base, off = x
        M, K = rows, cols
    q = np.empty((M, K // 2), np.uint8)
    sf = np.empty((M, K // 16), np.uint8)
    rc = _load().orc_encode_rowwise(base.ctypes.data + 2 * off, M, K, ld, int(per_vector),
                                    _ptr(amax), _ptr(q), _ptr(sf))
    if rc != 0:
        raise ValueError("oracle: rowwise needs K % 16 == 0")
    return q, sf


def encode_colwise(x, amax, per_vector, ld=None, rows=None, cols=None):
    """Columnwise encode (quantization of the transpose) with caller amax."""
    amax = np.ascontiguousarray(np.atleast_1d(amax), dtype=np.float32)
    if ld is None:
        x = _bf16(x)
        M, K = x.shape
        ld = K
        base = x
        off = 0
    else:
        base, off = x
        M, K = rows, cols
    q = np.empty((K, M // 2), np.uint8)
    sf = np.empty((K, M // 16), np.uint8)
    rc = _load().orc_encode_colwise(base.ctypes.data + 2 * off, M, K, ld, int(per_vector),
                                    _ptr(amax), _ptr(q), _ptr(sf))
    if rc != 0:
        raise ValueError("oracle: columnwise needs M % 16 == 0")
    return q, sf


def quantize(x, mode, rowwise=True, columnwise=True):
    """Whole cast; returns a dict with row_q/row_sf/row_amax and/or col_*."""
    x = _bf16(x)
    M, K = x.shape
    out = {}
    if rowwise:
        out["row_q"] = np.empty((M, K // 2), np.uint8)
        out["row_sf"] = np.empty((M, K // 16), np.uint8)
        out["row_amax"] = np.empty(1 if mode == PER_TENSOR else M, np.float32)
    if columnwise:
        out["col_q"] = np.empty((K, M // 2), np.uint8)
        out["col_sf"] = np.empty((K, M // 16), np.uint8)
        out["col_amax"] = np.empty(1 if mode == PER_TENSOR else K, np.float32)
    g = out.get
    rc = _load().orc_quantize(_ptr(x), M, K, int(mode),
                              _ptr(g("row_q")), _ptr(g("row_sf")), _ptr(g("row_amax")),
                              _ptr(g("col_q")), _ptr(g("col_sf")), _ptr(g("col_amax")))
    if rc != 0:
        raise ValueError("oracle: shape not supported by this mode")
    return out


def quantize_per_token_threads(x, nthreads):
    """The per-token row + column cast with rows and columns split over
    nthreads threads (the same per-vector routines; for timing the oracle on
    all host cores).  Same outputs as quantize(x, PER_TOKEN)."""
    x = _bf16(x)
    M, K = x.shape
    out = {"row_q": np.empty((M, K // 2), np.uint8), "row_sf": np.empty((M, K // 16), np.uint8),
           "row_amax": np.empty(M, np.float32), "col_q": np.empty((K, M // 2), np.uint8),
           "col_sf": np.empty((K, M // 16), np.uint8), "col_amax": np.empty(K, np.float32)}
    g = out.get
    rc = _load().orc_quantize_per_token_threads(_ptr(x), M, K, int(nthreads), _ptr(g("row_q")), _ptr(g("row_sf")),
                                                _ptr(g("row_amax")), _ptr(g("col_q")), _ptr(g("col_sf")),
                                                _ptr(g("col_amax")))
    if rc != 0:
        raise ValueError("oracle: bad arguments")
    return out


# ----------------------------------------------------- stochastic rounding

def philox4x32_10(ctr, key):
    """Philox4x32-10 blocks: ctr uint32 [n, 4], key uint32 [n, 2] -> [n, 4]."""
    ctr = np.ascontiguousarray(ctr, np.uint32).reshape(-1, 4)
    key = np.ascontiguousarray(key, np.uint32).reshape(-1, 2)
    if len(ctr) != len(key):
        raise ValueError("one key per counter")
    out = np.empty_like(ctr)
    _load().orc_philox4x32_10_array(_ptr(ctr), _ptr(key), len(ctr), _ptr(out))
    return out


def e2m1_encode_sr(q, rnd):
    """Stochastic E2M1 codes of float32 quotients q with 8-bit randoms rnd."""
    q = np.ascontiguousarray(q, np.float32).ravel()
    rnd = np.asarray(rnd)
    if rnd.dtype != np.uint8:
        raise ValueError("rnd: one uint8 random per quotient")
    rnd = np.ascontiguousarray(rnd).ravel()
    if q.shape != rnd.shape:
        raise ValueError("one random per quotient")
    out = np.empty(q.shape, np.uint8)
    _load().orc_e2m1_encode_sr_array(_ptr(q), _ptr(rnd), q.size, _ptr(out))
    return out


def quantize_vector_sr(v, A, seed, vec, direction, offset):
    v = np.ascontiguousarray(v, np.float32)
    q = np.empty(v.size // 2, np.uint8)
    sf = np.empty(v.size // 16, np.uint8)
    _load().orc_quantize_vector_sr(_ptr(v), v.size, float(A), _ptr(q), _ptr(sf), int(seed), int(vec),
                                   int(direction), int(offset))
    return q, sf


def quantize_sr(x, mode, seed, offset, rowwise=True, columnwise=True):
    """Stochastic-rounding cast (per-tensor or per-token); same outputs as
    quantize()."""
    x = _bf16(x)
    M, K = x.shape
    out = {}
    if rowwise:
        out["row_q"] = np.empty((M, K // 2), np.uint8)
        out["row_sf"] = np.empty((M, K // 16), np.uint8)
        out["row_amax"] = np.empty(1 if mode == PER_TENSOR else M, np.float32)
    if columnwise:
        out["col_q"] = np.empty((K, M // 2), np.uint8)
        out["col_sf"] = np.empty((K, M // 16), np.uint8)
        out["col_amax"] = np.empty(1 if mode == PER_TENSOR else K, np.float32)
    g = out.get
    rc = _load().orc_quantize_sr(_ptr(x), M, K, int(mode),
                                 _ptr(g("row_q")), _ptr(g("row_sf")), _ptr(g("row_amax")),
                                 _ptr(g("col_q")), _ptr(g("col_sf")), _ptr(g("col_amax")),
                                 int(seed), int(offset))
    if rc != 0:
        raise ValueError("oracle: shape or mode not supported by the stochastic-rounding cast")
    return out


# ------------------------------------------------------------ GEMM consumer

def gemm_nvfp4(a_q, a_sf, a_amax, b_q, b_sf, b_amax):
    """out[m][n] = S_a S_b sum_k (gD)_a (gD)_b for NVFP4 operands A [M][K]
    and B [N][K] (16-element blocks along K; amax per row or [1]).  Returns
    (out, bound) in float64, bound = S_a S_b sum_k |term|."""
    a_q, a_sf, b_q, b_sf = (np.ascontiguousarray(t, np.uint8) for t in (a_q, a_sf, b_q, b_sf))
    a_amax = np.ascontiguousarray(a_amax, np.float32)
    b_amax = np.ascontiguousarray(b_amax, np.float32)
    M, K = a_q.shape[0], a_q.shape[1] * 2
    N = b_q.shape[0]
    if b_q.shape[1] * 2 != K or a_sf.shape != (M, K // 16) or b_sf.shape != (N, K // 16):
        raise ValueError("operands must be [M][K/2] / [N][K/2] with [.][K/16] scales")
    out = np.empty((M, N), np.float64)
    bound = np.empty((M, N), np.float64)
    rc = _load().orc_gemm_nvfp4(_ptr(a_q), _ptr(a_sf), _ptr(a_amax), int(a_amax.size == M and M > 1),
                                _ptr(b_q), _ptr(b_sf), _ptr(b_amax), int(b_amax.size == N and N > 1),
                                M, N, K, _ptr(out), _ptr(bound))
    if rc != 0:
        raise ValueError("oracle: K must be a multiple of 16")
    return out, bound


# ------------------------------------------- random Hadamard transform

def rht16(blocks, sign_mask):
    """The transform of bf16 blocks uint16 [n, 16] (each row one block)."""
    blocks = np.ascontiguousarray(blocks, np.uint16).reshape(-1, 16)
    out = np.empty_like(blocks)
    for i in range(len(blocks)):
        _load().orc_rht16(_ptr(blocks[i]), int(sign_mask) & 0xFFFF, _ptr(out[i]))
    return out


def rht_columns(x, sign_mask):
    """bf16 [M, K] (M % 16 == 0): each 16-row block of each column transformed."""
    x = _bf16(x)
    M, K = x.shape
    y = np.empty_like(x)
    if _load().orc_rht_columns(_ptr(x), M, K, int(sign_mask) & 0xFFFF, _ptr(y)) != 0:
        raise ValueError("oracle: M must be a multiple of 16")
    return y


def quantize_rht(x, mode, sign_mask, rowwise=True):
    """Cast with the random Hadamard transform on the columnwise direction:
    rowwise outputs are the ordinary cast of x, columnwise outputs the
    ordinary columnwise cast of rht_columns(x) (its own amax)."""
    out = quantize(x, mode, rowwise=True, columnwise=False) if rowwise else {}
    out.update(quantize(rht_columns(x, sign_mask), mode, rowwise=False, columnwise=True))
    return out


# ------------------------------------------------ swizzled scale layout

def swizzle_scales(sf):
    """Plain scales uint8 [R, nb] -> the GEMM-swizzled layout, 1-D uint8 of
    ceil(R/128)*128 * ceil(nb/4)*4 bytes (padding zero)."""
    sf = np.ascontiguousarray(sf, np.uint8)
    R, nb = sf.shape
    out = np.empty(int(_load().orc_swizzled_size(R, nb)), np.uint8)
    _load().orc_swizzle_scales(_ptr(sf), R, nb, _ptr(out))
    return out


def unswizzle_scales(sw, R, nb):
    """Inverse of swizzle_scales: the [R, nb] plain scales."""
    sw = np.ascontiguousarray(sw, np.uint8).ravel()
    if sw.size != int(_load().orc_swizzled_size(R, nb)):
        raise ValueError("swizzled buffer has the wrong size")
    sf = np.empty((R, nb), np.uint8)
    _load().orc_unswizzle_scales(_ptr(sw), R, nb, _ptr(sf))
    return sf


def quantize_grouped(x, counts, rowwise=True, columnwise=True):
    x = _bf16(x)
    T, K = x.shape
    counts = np.ascontiguousarray(counts, dtype=np.int64)
    G = counts.size
    if int(counts.sum()) != T:
        raise ValueError("oracle: counts must sum to the row count")
    out = {}
    if rowwise:
        out["row_q"] = np.empty((T, K // 2), np.uint8)
        out["row_sf"] = np.empty((T, K // 16), np.uint8)
        out["row_amax"] = np.empty(T, np.float32)
    if columnwise:
        out["col_q"] = np.empty(T * K // 2, np.uint8)
        out["col_sf"] = np.empty(T * K // 16, np.uint8)
        out["col_amax"] = np.empty((G, K), np.float32)
    g = out.get
    rc = _load().orc_quantize_grouped(_ptr(x), K, G, _ptr(counts),
                                      _ptr(g("row_q")), _ptr(g("row_sf")), _ptr(g("row_amax")),
                                      _ptr(g("col_q")), _ptr(g("col_sf")), _ptr(g("col_amax")))
    if rc != 0:
        raise ValueError("oracle: bad grouped shape")
    return out


def dequantize(q, sf, amax, R, C, amax_per_row):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sf = np.ascontiguousarray(sf, dtype=np.uint8)
    amax = np.ascontiguousarray(np.atleast_1d(amax), dtype=np.float32)
    out = np.empty((R, C), np.float32)
    rc = _load().orc_dequantize(_ptr(q), _ptr(sf), _ptr(amax), R, C, int(amax_per_row), _ptr(out))
    if rc != 0:
        raise ValueError("oracle: dequantize needs C % 16 == 0")
    return out


def amax_accumulate(buf, obs, decay):
    buf = np.array(buf, dtype=np.float32, copy=True)
    obs = np.ascontiguousarray(obs, dtype=np.float32)
    assert buf.shape == obs.shape
    _load().orc_amax_accumulate(_ptr(buf), _ptr(obs), buf.size, float(np.float32(decay)))
    return buf


def amax_accumulate_reduce(buf, obs_vec, decay):
    buf = np.array(np.atleast_1d(buf), dtype=np.float32, copy=True)
    obs_vec = np.ascontiguousarray(obs_vec, dtype=np.float32)
    _load().orc_amax_accumulate_reduce(_ptr(buf), _ptr(obs_vec), obs_vec.size,
                                       float(np.float32(decay)))
    return buf
