"""bf16 -> NVFP4 block-scaled cast on AMD MI355X (gfx950).

Thin Python binding of ``libnvfp4.so`` (the C ABI declared in
``include/nvfp4.h``).  This module only marshals arguments: it allocates the
output tensors with torch on the input's device, passes raw device pointers
and the current HIP stream, and raises on a non-OK status.  Every step of the
cast runs in the library's HIP kernels; there is no fallback, so a missing or
unloadable library is an error.

Layouts (see the header): rowwise ``row_q`` [M, K/2] uint8 (element 2i in the
low nibble), ``row_sf`` [M, K/16] E4M3 codes, ``row_amax`` fp32; columnwise
(the quantization of the transpose) ``col_q`` [K, M/2], ``col_sf`` [K, M/16],
``col_amax``.
"""
from __future__ import annotations

import ctypes
import os

import torch

PER_TENSOR, PER_TOKEN, TILE_16x16 = 0, 1, 2
SCHEDULE_AUTO, SCHEDULE_TWO_PASS, SCHEDULE_RESIDENT = 0, 1, 2
_SCHEDULES = {"auto": SCHEDULE_AUTO, "two_pass": SCHEDULE_TWO_PASS, "resident": SCHEDULE_RESIDENT}
_MODES = {"per_tensor": PER_TENSOR, "per_token": PER_TOKEN, "tile_16x16": TILE_16x16,
          PER_TENSOR: PER_TENSOR, PER_TOKEN: PER_TOKEN, TILE_16x16: TILE_16x16}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4.so")

EXPORTS = ("nvfp4_abi_version", "nvfp4_last_error", "nvfp4_quantize", "nvfp4_quantize_rowwise",
           "nvfp4_quantize_columnwise", "nvfp4_amax", "nvfp4_encode", "nvfp4_quantize_grouped",
           "nvfp4_dequantize", "nvfp4_amax_accumulate", "nvfp4_amax_accumulate_reduce",
           "nvfp4_trace_encode", "nvfp4_quantize_calibrate", "nvfp4_quantize_sr", "nvfp4_gemm",
           "nvfp4_gemm_grouped", "nvfp4_quantize_rht", "nvfp4_swizzle_scales",
           "nvfp4_gemm_swizzled", "nvfp4_quantize_swizzled", "nvfp4_set_schedule",
           "nvfp4_test_fail_next_wait")

STATUS = {0: "OK", 1: "EINVAL", 2: "ESHAPE", 3: "EALIGN", 4: "EDEVICE"}

_lib = None


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"nvfp4 {STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libnvfp4.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, i32, f32, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_int
    sig = {
        "nvfp4_abi_version": (ctypes.c_int, []),
        "nvfp4_last_error": (ctypes.c_char_p, []),
        "nvfp4_quantize": (st, [p, i64, i64, st, p, p, p, p, p, p, p]),
        "nvfp4_quantize_rowwise": (st, [p, i64, i64, st, p, p, p, p]),
        "nvfp4_quantize_columnwise": (st, [p, i64, i64, st, p, p, p, p]),
        "nvfp4_amax": (st, [p, i64, i64, st, p, p, p]),
        "nvfp4_encode": (st, [p, i64, i64, st, p, p, p, p, p, p, p]),
        "nvfp4_quantize_grouped": (st, [p, i64, i32, p, p, p, p, p, p, p, p]),
        "nvfp4_dequantize": (st, [p, p, p, i64, i64, st, ctypes.c_int, p, p]),
        "nvfp4_amax_accumulate": (st, [p, p, i64, f32, p]),
        "nvfp4_amax_accumulate_reduce": (st, [p, p, i64, f32, p]),
        "nvfp4_trace_encode": (st, [p, p]),
        "nvfp4_quantize_calibrate": (st, [p, i64, i64, st, p, p, p, p, p, p, p, f32, p]),
        "nvfp4_quantize_sr": (st, [p, i64, i64, st, p, p, p, p, p, p, ctypes.c_uint64, ctypes.c_uint32, p]),
        "nvfp4_gemm": (st, [p, p, p, ctypes.c_int, p, p, p, ctypes.c_int, i64, i64, i64, p, p]),
        "nvfp4_gemm_grouped": (st, [p, p, p, ctypes.c_int, p, p, p, ctypes.c_int, i32, p, i64, i64, p, p]),
        "nvfp4_quantize_rht": (st, [p, i64, i64, st, ctypes.c_uint32, p, p, p, p, p, p, p]),
        "nvfp4_swizzle_scales": (st, [p, i64, i64, p, p]),
        "nvfp4_quantize_swizzled": (st, [p, i64, i64, st, p, p, p, p, p, p, p]),
        "nvfp4_gemm_swizzled": (st, [p, p, p, ctypes.c_int, p, p, p, ctypes.c_int, i64, i64, i64, p, p]),
        "nvfp4_set_schedule": (st, [st]),
        "nvfp4_test_fail_next_wait": (st, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise NVFP4Error(status, lib().nvfp4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _input(x):
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D bfloat16 CUDA tensor")
    return x


def _mode(mode):
    try:
        return _MODES[mode]
    except KeyError:
        raise ValueError(f"unknown scaling mode {mode!r}") from None


def _u8(shape, dev):
    return torch.empty(shape, dtype=torch.uint8, device=dev)


def _f32(shape, dev):
    return torch.empty(shape, dtype=torch.float32, device=dev)


def _amax_len(mode, n):
    return 1 if mode == PER_TENSOR else n


def _check_buf(t, dtype, numel, device, name, min_numel=None):
    """Reject a caller tensor the library would misread: wrong dtype, another
    device, not contiguous, or an element count other than the layout's
    (numel; None skips that check, min_numel then gives a lower bound)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    # an empty layout accepts any buffer (the library writes nothing there,
    # and a non-empty allocation keeps the pointer non-NULL: NULL means "not
    # requested")
    if numel is not None and numel > 0 and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements (got {t.numel()})")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements (got {t.numel()})")


def _check_dir(name, q, sf, amax, dev, q_n, sf_n, amax_n):
    """A direction's three outputs: all None (not requested) or all given
    with the layout's sizes.  Sizes are checked only where the shape is one
    the library accepts (q_n None otherwise), so that the library's own
    shape error reaches the caller."""
    given = [t is not None for t in (q, sf, amax)]
    if not any(given):
        return
    if not all(given):
        raise ValueError(f"{name}: q, sf and amax must all be given (or all None)")
    _check_buf(q, torch.uint8, q_n, dev, f"{name}_q")
    _check_buf(sf, torch.uint8, sf_n, dev, f"{name}_sf")
    _check_buf(amax, torch.float32, amax_n, dev, f"{name}_amax")


def _check_cast_outputs(x, mode, row_q=None, row_sf=None, row_amax=None, col_q=None, col_sf=None, col_amax=None):
    """Sizes of nvfp4_quantize's outputs (header layout): rowwise [M][K/2],
    [M][K/16], amax [1] (per tensor) or [M]; columnwise [K][M/2], [K][M/16],
    amax [1] or [K]."""
    M, K = x.shape
    dev = x.device
    rok, cok = K % 16 == 0, M % 16 == 0 and K % 8 == 0
    _check_dir("row", row_q, row_sf, row_amax, dev, M * (K // 2) if rok else None, M * (K // 16) if rok else None,
               _amax_len(mode, M) if rok else None)
    _check_dir("col", col_q, col_sf, col_amax, dev, K * (M // 2) if cok else None, K * (M // 16) if cok else None,
               _amax_len(mode, K) if cok else None)


def quantize(x: torch.Tensor, mode="per_token", rowwise: bool = True, columnwise: bool = True) -> dict:
    """Whole cast (one read of x for both directions)."""
    x = _input(x)
    mode = _mode(mode)
    M, K = x.shape
    dev = x.device
    out = {}
    if rowwise:
        out.update(row_q=_u8((M, K // 2), dev), row_sf=_u8((M, K // 16), dev), row_amax=_f32(_amax_len(mode, M), dev))
    if columnwise:
        out.update(col_q=_u8((K, M // 2), dev), col_sf=_u8((K, M // 16), dev), col_amax=_f32(_amax_len(mode, K), dev))
    g = out.get
    _check(lib().nvfp4_quantize(_ptr(x), M, K, mode, _ptr(g("row_q")), _ptr(g("row_sf")), _ptr(g("row_amax")),
                                _ptr(g("col_q")), _ptr(g("col_sf")), _ptr(g("col_amax")), _stream(dev)))
    return out


def quantize_sr(x: torch.Tensor, mode="per_token", seed: int = 0, offset: int = 0, rowwise: bool = True,
                columnwise: bool = True) -> dict:
    """Whole cast with stochastic rounding of the element codes (per-tensor or
    per-token scaling); the same seed and offset give the same bytes."""
    x = _input(x)
    mode = _mode(mode)
    M, K = x.shape
    dev = x.device
    out = {}
    if rowwise:
        out.update(row_q=_u8((M, K // 2), dev), row_sf=_u8((M, K // 16), dev), row_amax=_f32(_amax_len(mode, M), dev))
    if columnwise:
        out.update(col_q=_u8((K, M // 2), dev), col_sf=_u8((K, M // 16), dev), col_amax=_f32(_amax_len(mode, K), dev))
    quantize_sr_into(x, mode, seed, offset, **out)
    return out


def quantize_sr_into(x, mode, seed: int, offset: int, row_q=None, row_sf=None, row_amax=None, col_q=None,
                     col_sf=None, col_amax=None):
    """Stochastic-rounding cast into caller-provided buffers."""
    x = _input(x)
    M, K = x.shape
    _check_cast_outputs(x, _mode(mode), row_q, row_sf, row_amax, col_q, col_sf, col_amax)
    _check(lib().nvfp4_quantize_sr(_ptr(x), M, K, _mode(mode), _ptr(row_q), _ptr(row_sf), _ptr(row_amax),
                                   _ptr(col_q), _ptr(col_sf), _ptr(col_amax), ctypes.c_uint64(seed & (2**64 - 1)),
                                   ctypes.c_uint32(offset & 0xFFFFFFFF), _stream(x.device)))


def quantize_rht(x: torch.Tensor, mode="per_token", sign_mask: int = 0, rowwise: bool = True) -> dict:
    """Cast with the random Hadamard transform (16-point, signs from the
    16-bit mask) applied to the columnwise direction only; rowwise outputs
    are the ordinary cast's."""
    x = _input(x)
    mode = _mode(mode)
    M, K = x.shape
    dev = x.device
    out = {}
    if rowwise:
        out.update(row_q=_u8((M, K // 2), dev), row_sf=_u8((M, K // 16), dev), row_amax=_f32(_amax_len(mode, M), dev))
    out.update(col_q=_u8((K, M // 2), dev), col_sf=_u8((K, M // 16), dev), col_amax=_f32(_amax_len(mode, K), dev))
    quantize_rht_into(x, mode, sign_mask, **out)
    return out


def quantize_rht_into(x, mode, sign_mask: int, col_q, col_sf, col_amax, row_q=None, row_sf=None, row_amax=None):
    """Hadamard-transform cast into caller-provided buffers."""
    x = _input(x)
    M, K = x.shape
    _check_cast_outputs(x, _mode(mode), row_q, row_sf, row_amax, col_q, col_sf, col_amax)
    _check(lib().nvfp4_quantize_rht(_ptr(x), M, K, _mode(mode), ctypes.c_uint32(sign_mask), _ptr(row_q),
                                    _ptr(row_sf), _ptr(row_amax), _ptr(col_q), _ptr(col_sf), _ptr(col_amax),
                                    _stream(x.device)))


def quantize_into(x, mode, row_q=None, row_sf=None, row_amax=None, col_q=None, col_sf=None, col_amax=None):
    """Whole cast into caller-provided buffers (no allocation)."""
    x = _input(x)
    M, K = x.shape
    _check_cast_outputs(x, _mode(mode), row_q, row_sf, row_amax, col_q, col_sf, col_amax)
    _check(lib().nvfp4_quantize(_ptr(x), M, K, _mode(mode), _ptr(row_q), _ptr(row_sf), _ptr(row_amax),
                                _ptr(col_q), _ptr(col_sf), _ptr(col_amax), _stream(x.device)))


def quantize_calibrate_into(x, mode, buf, decay: float, row_q=None, row_sf=None, row_amax=None,
                            col_q=None, col_sf=None, col_amax=None):
    """Whole cast into caller-provided buffers plus the decayed calibration
    update buf[0] = max(buf[0] * decay, tensor amax) (fp32 tensor of one
    element on the same device)."""
    x = _input(x)
    M, K = x.shape
    _check_buf(buf, torch.float32, None, x.device, "buf", min_numel=1)
    _check_cast_outputs(x, _mode(mode), row_q, row_sf, row_amax, col_q, col_sf, col_amax)
    _check(lib().nvfp4_quantize_calibrate(_ptr(x), M, K, _mode(mode), _ptr(row_q), _ptr(row_sf), _ptr(row_amax),
                                          _ptr(col_q), _ptr(col_sf), _ptr(col_amax), _ptr(buf),
                                          ctypes.c_float(decay), _stream(x.device)))


def prepare_quantize(x, mode, buf=None, decay: float = 0.0, row_q=None, row_sf=None, row_amax=None,
                     col_q=None, col_sf=None, col_amax=None):
    """quantize_into (or, with buf, quantize_calibrate_into) validated and
    marshalled once: returns a function of no arguments that issues the same
    call on the stream current now.  For loops that repeat one call on fixed
    buffers, where the per-call Python checks would cost more than the
    kernels of a small tensor."""
    x = _input(x)
    M, K = x.shape
    m = _mode(mode)
    _check_cast_outputs(x, m, row_q, row_sf, row_amax, col_q, col_sf, col_amax)
    L = lib()
    ptrs = (_ptr(row_q), _ptr(row_sf), _ptr(row_amax), _ptr(col_q), _ptr(col_sf), _ptr(col_amax))
    if buf is None:
        fn, args = L.nvfp4_quantize, (_ptr(x), M, K, m) + ptrs + (_stream(x.device),)
    else:
        _check_buf(buf, torch.float32, None, x.device, "buf", min_numel=1)
        fn, args = L.nvfp4_quantize_calibrate, (_ptr(x), M, K, m) + ptrs + (_ptr(buf), ctypes.c_float(decay),
                                                                           _stream(x.device))
    keep = (x, buf, row_q, row_sf, row_amax, col_q, col_sf, col_amax)   # alive while the call is

    def call():
        st = fn(*args)
        if st != 0:
            _check(st)
    call.keep = keep
    return call


def quantize_rowwise(x, mode="per_token"):
    x = _input(x)
    mode = _mode(mode)
    M, K = x.shape
    q, sf, a = _u8((M, K // 2), x.device), _u8((M, K // 16), x.device), _f32(_amax_len(mode, M), x.device)
    _check(lib().nvfp4_quantize_rowwise(_ptr(x), M, K, mode, _ptr(q), _ptr(sf), _ptr(a), _stream(x.device)))
    return {"row_q": q, "row_sf": sf, "row_amax": a}


def quantize_columnwise(x, mode="per_token"):
    x = _input(x)
    mode = _mode(mode)
    M, K = x.shape
    q, sf, a = _u8((K, M // 2), x.device), _u8((K, M // 16), x.device), _f32(_amax_len(mode, K), x.device)
    _check(lib().nvfp4_quantize_columnwise(_ptr(x), M, K, mode, _ptr(q), _ptr(sf), _ptr(a), _stream(x.device)))
    return {"col_q": q, "col_sf": sf, "col_amax": a}


def amax(x, mode="per_token", rowwise=True, columnwise=True):
    """Outer amax only (split form, first half)."""
    x = _input(x)
    mode = _mode(mode)
    M, K = x.shape
    ra = _f32(_amax_len(mode, M), x.device) if rowwise else None
    ca = _f32(_amax_len(mode, K), x.device) if columnwise else None
    _check(lib().nvfp4_amax(_ptr(x), M, K, mode, _ptr(ra), _ptr(ca), _stream(x.device)))
    return {"row_amax": ra, "col_amax": ca}


def encode(x, mode="per_token", row_amax=None, col_amax=None):
    """Block scales + E2M1 data from caller-supplied amax (split form): fp32
    values, finite and >= 0, [1] per tensor or [M] / [K] per token."""
    x = _input(x)
    M, K = x.shape
    out = {}
    if row_amax is not None:
        out.update(row_q=_u8((M, K // 2), x.device), row_sf=_u8((M, K // 16), x.device))
    if col_amax is not None:
        out.update(col_q=_u8((K, M // 2), x.device), col_sf=_u8((K, M // 16), x.device))
    encode_into(x, mode, row_amax, col_amax, **out)
    return out


def encode_into(x, mode, row_amax=None, col_amax=None, row_q=None, row_sf=None, col_q=None, col_sf=None):
    """:func:`encode` into caller-provided buffers (rowwise [M][K/2],
    [M][K/16]; columnwise [K][M/2], [K][M/16])."""
    x = _input(x)
    mode = _mode(mode)
    M, K = x.shape
    dev = x.device
    if row_amax is not None:
        _check_buf(row_amax, torch.float32, _amax_len(mode, M), dev, "row_amax")
    if col_amax is not None:
        _check_buf(col_amax, torch.float32, _amax_len(mode, K), dev, "col_amax")
    rok, cok = K % 16 == 0, M % 16 == 0 and K % 8 == 0
    for name, t, n in (("row_q", row_q, M * (K // 2) if rok else None), ("row_sf", row_sf, M * (K // 16) if rok else None),
                       ("col_q", col_q, K * (M // 2) if cok else None), ("col_sf", col_sf, K * (M // 16) if cok else None)):
        if t is not None:
            _check_buf(t, torch.uint8, n, dev, name)
    _check(lib().nvfp4_encode(_ptr(x), M, K, mode, _ptr(row_amax), _ptr(col_amax), _ptr(row_q),
                              _ptr(row_sf), _ptr(col_q), _ptr(col_sf), _stream(dev)))


def quantize_grouped(x, counts, rowwise=True, columnwise=True):
    """Grouped (MoE) per-token cast; counts: host sequence of per-expert rows."""
    x = _input(x)
    T, K = x.shape
    G = len(list(counts))
    dev = x.device
    out = {}
    if rowwise:
        out.update(row_q=_u8((T, K // 2), dev), row_sf=_u8((T, K // 16), dev), row_amax=_f32(T, dev))
    if columnwise:
        out.update(col_q=_u8(T * K // 2, dev), col_sf=_u8(T * K // 16, dev), col_amax=_f32((G, K), dev))
    quantize_grouped_into(x, counts, **out)
    return out


def quantize_grouped_into(x, counts, row_q=None, row_sf=None, row_amax=None, col_q=None, col_sf=None,
                          col_amax=None):
    """Grouped cast into caller-provided buffers: rowwise [T][K/2], [T][K/16],
    [T]; columnwise slabs T*K/2 and T*K/16 bytes, col_amax [G][K]."""
    x = _input(x)
    T, K = x.shape
    counts_t = torch.as_tensor(list(counts), dtype=torch.int64).contiguous()
    G = counts_t.numel()
    dev = x.device
    ok = K % 16 == 0
    _check_dir("row", row_q, row_sf, row_amax, dev, T * (K // 2) if ok else None, T * (K // 16) if ok else None,
               T if ok else None)
    _check_dir("col", col_q, col_sf, col_amax, dev, T * (K // 2) if ok else None, T * (K // 16) if ok else None,
               G * K if ok else None)
    _check(lib().nvfp4_quantize_grouped(_ptr(x), K, G, ctypes.c_void_p(counts_t.data_ptr()),
                                        _ptr(row_q), _ptr(row_sf), _ptr(row_amax),
                                        _ptr(col_q), _ptr(col_sf), _ptr(col_amax), _stream(dev)))


def dequantize(q, sf, amax, mode="per_token", out_dtype=torch.float32):
    """[R, C] from q [R, C/2], sf [R, C/16] and amax ([R] for per-token
    scaling, [1] otherwise): fp32, or bf16 as the round-to-nearest-even of
    the fp32 value (out_dtype=torch.bfloat16)."""
    mode = _mode(mode)
    if q.dim() != 2 or q.dtype != torch.uint8 or not q.is_cuda or not q.is_contiguous():
        raise ValueError("q must be a contiguous 2-D uint8 CUDA tensor [R, C/2]")
    R, C2 = q.shape
    C = 2 * C2
    _check_buf(sf, torch.uint8, R * (C // 16), q.device, "sf")
    _check_buf(amax, torch.float32, R if mode == PER_TOKEN else None, q.device, "amax", min_numel=1)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
    out = torch.empty((R, C), dtype=out_dtype, device=q.device)
    _check(lib().nvfp4_dequantize(_ptr(q), _ptr(sf), _ptr(amax), R, C, mode, int(out_dtype == torch.bfloat16),
                                  _ptr(out), _stream(q.device)))
    return out


def _operand(q, sf, amax, name):
    if q.dim() != 2 or q.dtype != torch.uint8:
        raise ValueError(f"{name}_q must be a 2-D uint8 tensor [rows, K/2]")
    rows, K = q.shape[0], 2 * q.shape[1]
    if sf.numel() != rows * (K // 16) or amax.numel() not in (1, rows):
        raise ValueError(f"{name}_sf must hold rows*K/16 codes and {name}_amax 1 or rows values")
    return rows, K, int(amax.numel() == rows and rows != 1)


def gemm_into(out, a_q, a_sf, a_amax, b_q, b_sf, b_amax):
    """out [M, N] fp32 = S_a(m) S_b(n) sum_k (g D)_a[m][k] (g D)_b[n][k] for
    NVFP4 operands a_q [M, K/2] / a_sf [M, K/16] and b_q [N, K/2] / b_sf
    [N, K/16]; each amax is one value (per tensor) or one per row."""
    M, K, apr = _operand(a_q, a_sf, a_amax, "a")
    N, Kb, bpr = _operand(b_q, b_sf, b_amax, "b")
    if K != Kb:
        raise ValueError(f"contraction sizes differ: {K} vs {Kb}")
    if tuple(out.shape) != (M, N) or out.dtype != torch.float32:
        raise ValueError("out must be fp32 [M, N]")
    _check(lib().nvfp4_gemm(_ptr(a_q), _ptr(a_sf), _ptr(a_amax), apr, _ptr(b_q), _ptr(b_sf), _ptr(b_amax), bpr,
                            M, N, K, _ptr(out), _stream(a_q.device)))
    return out


def swizzled_size(R: int, nb: int) -> int:
    """Bytes of the GEMM-swizzled layout of an [R, nb] scale matrix."""
    return (R + 127) // 128 * 128 * ((nb + 3) // 4 * 4)


def swizzle_scales(sf):
    """Plain scales uint8 [R, nb] -> the GEMM-swizzled layout (1-D uint8)."""
    if sf.dim() != 2 or sf.dtype != torch.uint8:
        raise ValueError("sf must be a 2-D uint8 tensor [R, nb]")
    R, nb = sf.shape
    out = _u8(swizzled_size(R, nb), sf.device)
    _check(lib().nvfp4_swizzle_scales(_ptr(sf.contiguous()), R, nb, _ptr(out), _stream(sf.device)))
    return out


def quantize_swizzled(x: torch.Tensor, mode="per_token", rowwise: bool = True, columnwise: bool = True) -> dict:
    """Whole cast with both scale outputs in the GEMM-swizzled layout (1-D
    uint8 of M*K/16 bytes each; M and K multiples of 128)."""
    x = _input(x)
    mode = _mode(mode)
    M, K = x.shape
    dev = x.device
    out = {}
    if rowwise:
        out.update(row_q=_u8((M, K // 2), dev), row_sf=_u8(M * K // 16, dev), row_amax=_f32(_amax_len(mode, M), dev))
    if columnwise:
        out.update(col_q=_u8((K, M // 2), dev), col_sf=_u8(M * K // 16, dev), col_amax=_f32(_amax_len(mode, K), dev))
    quantize_swizzled_into(x, mode, **out)
    return out


def quantize_swizzled_into(x, mode, row_q=None, row_sf=None, row_amax=None, col_q=None, col_sf=None, col_amax=None):
    """Swizzled-scale cast into caller-provided buffers."""
    x = _input(x)
    M, K = x.shape
    # the swizzled scale matrices hold M*K/16 bytes each (M, K % 128 == 0)
    _check_cast_outputs(x, _mode(mode), row_q, row_sf, row_amax, col_q, col_sf, col_amax)
    _check(lib().nvfp4_quantize_swizzled(_ptr(x), M, K, _mode(mode), _ptr(row_q), _ptr(row_sf), _ptr(row_amax),
                                         _ptr(col_q), _ptr(col_sf), _ptr(col_amax), _stream(x.device)))


def gemm_swizzled_into(out, a_q, a_sw, a_amax, b_q, b_sw, b_amax):
    """:func:`gemm_into` with both operands' scales in the swizzled layout
    (1-D, as :func:`swizzle_scales` returns them)."""
    if a_q.dim() != 2 or b_q.dim() != 2:
        raise ValueError("a_q and b_q must be 2-D [rows, K/2]")
    M, K, N = a_q.shape[0], 2 * a_q.shape[1], b_q.shape[0]
    if 2 * b_q.shape[1] != K:
        raise ValueError("contraction sizes differ")
    if a_sw.numel() != swizzled_size(M, K // 16) or b_sw.numel() != swizzled_size(N, K // 16):
        raise ValueError("swizzled scales have the wrong size")
    if tuple(out.shape) != (M, N) or out.dtype != torch.float32:
        raise ValueError("out must be fp32 [M, N]")
    apr = int(a_amax.numel() == M and M != 1)
    bpr = int(b_amax.numel() == N and N != 1)
    _check(lib().nvfp4_gemm_swizzled(_ptr(a_q), _ptr(a_sw), _ptr(a_amax), apr, _ptr(b_q), _ptr(b_sw),
                                     _ptr(b_amax), bpr, M, N, K, _ptr(out), _stream(a_q.device)))
    return out


def gemm(a_q, a_sf, a_amax, b_q, b_sf, b_amax):
    """Allocate out and run :func:`gemm_into`."""
    return gemm_into(_f32((a_q.shape[0], b_q.shape[0]), a_q.device), a_q, a_sf, a_amax, b_q, b_sf, b_amax)


def gemm_grouped_into(out, a_q, a_sf, a_amax, b_q, b_sf, b_amax, counts):
    """Per expert e: out[rows of e] = A_e x B_e^T (see :func:`gemm_into`).
    a_q [T, K/2] / a_sf [T, K/16] / a_amax ([T] or [1]) hold the experts'
    rows back to back, counts[e] rows each; b_q [G, N, K/2], b_sf
    [G, N, K/16], b_amax [G, N] (per row) or [G] (one per expert)."""
    counts_t = torch.as_tensor(counts, dtype=torch.int64).cpu().contiguous()
    G = counts_t.numel()
    T, K, apr = _operand(a_q, a_sf, a_amax, "a")
    if int(counts_t.sum()) != T:
        raise ValueError("counts must sum to the rows of a_q")
    if b_q.dim() != 3 or b_q.shape[0] != G or 2 * b_q.shape[2] != K:
        raise ValueError("b_q must be [G, N, K/2]")
    N = b_q.shape[1]
    if b_sf.numel() != G * N * (K // 16) or b_amax.numel() not in (G, G * N):
        raise ValueError("b_sf must hold G*N*K/16 codes and b_amax G or G*N values")
    bpr = int(b_amax.numel() == G * N and N != 1)
    if tuple(out.shape) != (T, N) or out.dtype != torch.float32:
        raise ValueError("out must be fp32 [T, N]")
    _check(lib().nvfp4_gemm_grouped(_ptr(a_q), _ptr(a_sf), _ptr(a_amax), apr, _ptr(b_q), _ptr(b_sf), _ptr(b_amax),
                                    bpr, G, ctypes.c_void_p(counts_t.data_ptr()), N, K, _ptr(out),
                                    _stream(a_q.device)))
    return out


def gemm_grouped(a_q, a_sf, a_amax, b_q, b_sf, b_amax, counts):
    """Allocate out and run :func:`gemm_grouped_into`."""
    out = _f32((a_q.shape[0], b_q.shape[1]), a_q.device)
    return gemm_grouped_into(out, a_q, a_sf, a_amax, b_q, b_sf, b_amax, counts)


def amax_accumulate(buf, observed, decay: float):
    """In place: buf = max(buf * decay, observed), fp32."""
    _check_buf(buf, torch.float32, None, buf.device if isinstance(buf, torch.Tensor) else None, "buf")
    _check_buf(observed, torch.float32, buf.numel(), buf.device, "observed")
    _check(lib().nvfp4_amax_accumulate(_ptr(buf), _ptr(observed), buf.numel(), float(decay), _stream(buf.device)))
    return buf


def amax_accumulate_reduce(buf, observed, decay: float):
    """In place: buf[0] = max(buf[0] * decay, max(observed))."""
    _check_buf(buf, torch.float32, None, buf.device if isinstance(buf, torch.Tensor) else None, "buf", min_numel=1)
    _check_buf(observed, torch.float32, None, buf.device, "observed")
    _check(lib().nvfp4_amax_accumulate_reduce(_ptr(buf), _ptr(observed), observed.numel(), float(decay),
                                              _stream(buf.device)))
    return buf


def trace_encode(before, after):
    """Bracket the next encoding-kernel launch on this thread with two events
    (torch.cuda.Event, or raw hipEvent_t handles as ints); None, None cancels.
    A torch event that was never recorded has no handle yet, so it is recorded
    once here on the current stream to create it."""
    def handle(ev):
        if ev is None:
            return None
        if isinstance(ev, int):
            return ctypes.c_void_p(ev)
        if ev.cuda_event == 0:
            ev.record()
        return ctypes.c_void_p(ev.cuda_event)
    _check(lib().nvfp4_trace_encode(handle(before), handle(after)))


def set_schedule(schedule):
    """nvfp4_set_schedule: "auto", "two_pass" or "resident" (or the ints 0..2)
    for the per-tensor and per-token casts whose amax the call measures;
    results are identical, only the launches differ."""
    v = _SCHEDULES.get(schedule, schedule)
    if v not in (0, 1, 2):
        raise ValueError(f"unknown schedule {schedule!r}")
    _check(lib().nvfp4_set_schedule(v))
