"""C ABI checks that need no GPU: the library loads, exports every function
include/nvfp4.h declares, and its host-side validation rejects bad arguments
with the documented status before anything is launched (only argument sets
that fail validation are passed here)."""
import ctypes
import os
import re

import pytest

import nvfp4_block_scaled_bf16_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, EINVAL, ESHAPE, EALIGN = 0, 1, 2, 3
FAKE = 0x10000  # an aligned address that is never dereferenced: validation fails first


def declared():
    with open(HEADER) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"NVFP4_API\s+[\w\s\*]*?\b(nvfp4_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared() == sorted(nv.EXPORTS)


def test_library_loads_and_exports_every_symbol():
    L = nv.lib()
    for name in declared():
        assert hasattr(L, name), name
    assert L.nvfp4_abi_version() == 3


def _q(*args):
    return nv.lib().nvfp4_quantize(*args)


P = ctypes.c_void_p


def test_quantize_validation():
    L = nv.lib()
    f = P(FAKE)
    # no direction requested
    assert _q(f, 16, 16, 1, None, None, None, None, None, None, None) == EINVAL
    assert b"direction" in L.nvfp4_last_error()
    # partial direction
    assert _q(f, 16, 16, 1, f, None, f, None, None, None, None) == EINVAL
    # bad mode
    assert _q(f, 16, 16, 7, f, f, f, None, None, None, None) == EINVAL
    # negative size
    assert _q(f, -16, 16, 1, f, f, f, None, None, None, None) == EINVAL
    # rowwise needs K % 16
    assert _q(f, 16, 24, 1, f, f, f, None, None, None, None) == ESHAPE
    # columnwise needs M % 16 and K % 8
    assert _q(f, 20, 16, 1, None, None, None, f, f, f, None) == ESHAPE
    assert _q(f, 16, 12, 1, None, None, None, f, f, f, None) == ESHAPE
    # 16x16 tiles need both
    assert _q(f, 16, 24, 2, None, None, None, f, f, f, None) == ESHAPE
    # K at the encoding kernel's limit (2^25)
    assert _q(f, 16, 1 << 25, 1, f, f, f, None, None, None, None) == ESHAPE
    assert b"K must be below" in L.nvfp4_last_error()
    # NULL input
    assert _q(None, 16, 16, 1, f, f, f, None, None, None, None) == EINVAL
    # misaligned input / outputs / amax
    assert _q(P(FAKE + 2), 16, 16, 1, f, f, f, None, None, None, None) == EALIGN
    assert _q(f, 16, 16, 1, P(FAKE + 8), f, f, None, None, None, None) == EALIGN
    assert _q(f, 16, 16, 1, f, f, P(FAKE + 2), None, None, None, None) == EALIGN


def test_other_entry_points_validation():
    L = nv.lib()
    f = P(FAKE)
    assert L.nvfp4_quantize_rowwise(f, 16, 16, 1, None, f, f, None) == EINVAL
    assert L.nvfp4_quantize_columnwise(f, 16, 16, 1, f, None, f, None) == EINVAL
    assert L.nvfp4_amax(f, 16, 16, 2, f, f, None) == EINVAL          # tiles not accepted
    assert L.nvfp4_amax(f, 16, 16, 1, None, None, None) == EINVAL
    assert L.nvfp4_amax(f, 16, 12, 1, f, None, None) == ESHAPE
    assert L.nvfp4_encode(f, 16, 16, 2, f, None, f, f, None, None, None) == EINVAL
    assert L.nvfp4_encode(f, 16, 16, 1, None, None, f, f, None, None, None) == EINVAL
    assert L.nvfp4_dequantize(f, f, f, 4, 24, 1, 0, f, None) == ESHAPE
    assert L.nvfp4_dequantize(None, f, f, 4, 32, 1, 0, f, None) == EINVAL
    assert L.nvfp4_dequantize(f, f, f, 4, 32, 3, 0, f, None) == EINVAL      # unknown mode
    assert L.nvfp4_dequantize(f, f, f, 4, 32, -1, 1, f, None) == EINVAL
    assert L.nvfp4_dequantize(f, f, f, 4, 32, 1, 1, P(FAKE + 8), None) == EALIGN   # out needs 16 bytes
    assert L.nvfp4_dequantize(f, f, f, 0, 32, 1, 1, None, None) == OK        # empty: nothing to do
    assert L.nvfp4_amax_accumulate(f, f, 4, ctypes.c_float(1.5), None) == EINVAL
    assert L.nvfp4_amax_accumulate(f, f, 4, ctypes.c_float(-0.1), None) == EINVAL
    assert L.nvfp4_amax_accumulate(f, f, 4, ctypes.c_float(float("nan")), None) == EINVAL
    assert L.nvfp4_amax_accumulate(f, f, -1, ctypes.c_float(0.5), None) == EINVAL
    assert L.nvfp4_amax_accumulate_reduce(None, f, 4, ctypes.c_float(0.5), None) == EINVAL


def test_quantize_calibrate_validation():
    L = nv.lib()
    f = P(FAKE)
    q = L.nvfp4_quantize_calibrate
    assert q(f, 16, 16, 1, f, f, f, None, None, None, None, ctypes.c_float(0.9), None) == EINVAL   # no buf
    assert q(f, 16, 16, 1, f, f, f, None, None, None, P(FAKE + 2), ctypes.c_float(0.9), None) == EALIGN
    assert q(f, 16, 16, 1, f, f, f, None, None, None, f, ctypes.c_float(1.5), None) == EINVAL
    assert q(f, 16, 16, 1, f, f, f, None, None, None, f, ctypes.c_float(float("nan")), None) == EINVAL
    # the cast's own checks still apply
    assert q(f, 16, 24, 1, f, f, f, None, None, None, f, ctypes.c_float(0.9), None) == ESHAPE
    assert q(f, 16, 16, 1, None, None, None, None, None, None, f, ctypes.c_float(0.9), None) == EINVAL


def test_quantize_sr_validation():
    L = nv.lib()
    f = P(FAKE)
    q = L.nvfp4_quantize_sr
    seed, off = ctypes.c_uint64(1), ctypes.c_uint32(0)
    assert q(f, 16, 16, 2, f, f, f, None, None, None, seed, off, None) == EINVAL   # 16x16 tiles: not offered
    assert b"stochastic" in L.nvfp4_last_error()
    assert q(f, 1 << 32, 16, 1, f, f, f, None, None, None, seed, off, None) == ESHAPE   # vector index is 32-bit
    assert q(f, 16, 24, 0, f, f, f, None, None, None, seed, off, None) == ESHAPE
    assert q(f, 16, 16, 1, None, None, None, None, None, None, seed, off, None) == EINVAL
    assert q(P(FAKE + 2), 16, 16, 1, f, f, f, None, None, None, seed, off, None) == EALIGN


def test_gemm_validation():
    L = nv.lib()
    f, g = P(FAKE), L.nvfp4_gemm
    assert g(f, f, f, 1, f, f, f, 1, -1, 16, 16, f, None) == EINVAL
    assert g(f, f, f, 1, f, f, f, 1, 16, 16, 24, f, None) == ESHAPE   # K % 16
    assert b"K % 16" in L.nvfp4_last_error()
    assert g(f, f, f, 1, f, f, f, 1, 1 << 40, 1 << 40, 16, f, None) == ESHAPE   # tile count
    assert g(None, None, None, 1, None, None, None, 1, 0, 16, 16, None, None) == 0   # M == 0: nothing
    assert g(None, f, f, 1, f, f, f, 1, 16, 16, 16, f, None) == EINVAL
    assert g(None, None, f, 1, None, None, f, 1, 16, 16, 0, None, None) == EINVAL   # out NULL
    assert g(P(FAKE + 8), f, f, 1, f, f, f, 1, 16, 16, 16, f, None) == EALIGN
    assert g(f, f, f, 1, f, f, f, 1, 16, 16, 16, P(FAKE + 2), None) == EALIGN


def test_gemm_grouped_validation():
    L = nv.lib()
    f, g = P(FAKE), L.nvfp4_gemm_grouped
    counts = (ctypes.c_int64 * 3)(16, 0, 32)
    assert g(f, f, f, 1, f, f, f, 1, -1, counts, 16, 16, f, None) == EINVAL
    assert g(f, f, f, 1, f, f, f, 1, 3, None, 16, 16, f, None) == EINVAL
    assert g(f, f, f, 1, f, f, f, 1, 3, counts, 16, 24, f, None) == ESHAPE   # K % 16
    neg = (ctypes.c_int64 * 2)(16, -1)
    assert g(f, f, f, 1, f, f, f, 1, 2, neg, 16, 16, f, None) == ESHAPE
    zeros = (ctypes.c_int64 * 2)(0, 0)
    assert g(None, None, None, 1, None, None, None, 1, 2, zeros, 16, 16, None, None) == 0   # no rows
    assert g(f, f, f, 1, f, f, f, 1, 3, counts, 16, 16, None, None) == EINVAL
    assert g(P(FAKE + 8), f, f, 1, f, f, f, 1, 3, counts, 16, 16, f, None) == EALIGN


def test_quantize_rht_validation():
    L = nv.lib()
    f, q = P(FAKE), L.nvfp4_quantize_rht
    assert q(f, 16, 16, 2, 0, None, None, None, f, f, f, None) == EINVAL   # 16x16 tiles: not offered
    assert b"per-tensor and per-token" in L.nvfp4_last_error()
    assert q(f, 16, 16, 1, 1 << 16, None, None, None, f, f, f, None) == EINVAL   # mask has 16 bits
    assert q(f, 16, 16, 1, 0, f, f, f, None, None, None, None) == EINVAL   # columnwise output required
    assert q(f, 24, 16, 1, 0, None, None, None, f, f, f, None) == ESHAPE   # M % 16
    assert q(f, 16, 24, 1, 0, f, f, f, f, f, f, None) == ESHAPE   # K % 16 with rowwise output
    assert q(f, 65536 * 128, 16, 1, 0, None, None, None, f, f, f, None) == ESHAPE
    assert q(P(FAKE + 2), 16, 16, 1, 0, None, None, None, f, f, f, None) == EALIGN


def test_swizzle_and_swizzled_gemm_validation():
    L = nv.lib()
    f = P(FAKE)
    assert L.nvfp4_swizzle_scales(f, -1, 4, f, None) == EINVAL
    assert L.nvfp4_swizzle_scales(None, 0, 4, None, None) == 0   # nothing to do
    assert L.nvfp4_swizzle_scales(None, 4, 4, f, None) == EINVAL
    assert L.nvfp4_swizzle_scales(f, 4, 4, P(FAKE + 2), None) == EALIGN
    g = L.nvfp4_gemm_swizzled
    assert g(f, f, f, 1, f, f, f, 1, 16, 16, 24, f, None) == ESHAPE
    assert g(f, P(FAKE + 2), f, 1, f, f, f, 1, 16, 16, 16, f, None) == EALIGN   # swizzled scales 4-aligned
    assert g(f, f, f, 1, f, f, f, 1, 0, 16, 16, None, None) == 0


def test_quantize_swizzled_validation():
    L = nv.lib()
    f, q = P(FAKE), L.nvfp4_quantize_swizzled
    assert q(f, 128, 128, 2, f, f, f, f, f, f, None) == EINVAL   # 16x16 tiles: not offered
    assert q(f, 144, 128, 1, f, f, f, f, f, f, None) == ESHAPE   # M % 128
    assert q(f, 128, 144, 1, f, f, f, f, f, f, None) == ESHAPE   # K % 128
    assert q(f, 128, 128, 1, f, P(FAKE + 2), f, None, None, None, None) == EALIGN
    assert q(f, 1 << 20, 1 << 15, 1, f, f, f, None, None, None, None) == ESHAPE   # M * K / 16 >= 2^31


def test_trace_encode_validation():
    L = nv.lib()
    assert L.nvfp4_trace_encode(P(FAKE), None) == EINVAL
    assert b"trace" in L.nvfp4_last_error()
    assert L.nvfp4_trace_encode(None, P(FAKE)) == EINVAL
    assert L.nvfp4_trace_encode(None, None) == 0   # cancels; nothing pending


def test_set_schedule_validation():
    L = nv.lib()
    assert L.nvfp4_set_schedule(3) == EINVAL
    assert b"schedule" in L.nvfp4_last_error()
    assert L.nvfp4_set_schedule(-1) == EINVAL
    for v in (1, 2, 0):   # ends on the default
        assert L.nvfp4_set_schedule(v) == 0
    with pytest.raises(ValueError):
        nv.set_schedule("fastest")


def test_grouped_validation():
    L = nv.lib()
    f = P(FAKE)
    bad = (ctypes.c_int64 * 3)(16, 8, 0)
    assert L.nvfp4_quantize_grouped(f, 32, 3, bad, f, f, f, f, f, f, None) == ESHAPE
    neg = (ctypes.c_int64 * 2)(16, -16)
    assert L.nvfp4_quantize_grouped(f, 32, 2, neg, f, f, f, f, f, f, None) == ESHAPE
    good = (ctypes.c_int64 * 2)(16, 32)
    assert L.nvfp4_quantize_grouped(f, 24, 2, good, f, f, f, None, None, None, None) == ESHAPE
    assert L.nvfp4_quantize_grouped(f, 32, -1, good, f, f, f, None, None, None, None) == EINVAL
    assert L.nvfp4_quantize_grouped(f, 32, 2, None, f, f, f, None, None, None, None) == EINVAL


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        nv.quantize(torch.zeros(16, 16, dtype=torch.bfloat16))


def test_binding_validates_caller_buffers():
    """The *_into wrappers check every caller tensor against the header's
    layout before calling the library (checked here with the helpers they
    call, on host tensors, since the wrappers themselves need a GPU)."""
    import torch
    M, K = 32, 64
    x = torch.zeros(M, K, dtype=torch.bfloat16)
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8)
    f32 = lambda n: torch.zeros(n, dtype=torch.float32)
    good = dict(row_q=u8(M * K // 2), row_sf=u8(M * K // 16), row_amax=f32(M),
                col_q=u8(K * M // 2), col_sf=u8(K * M // 16), col_amax=f32(K))
    nv._check_cast_outputs(x, nv.PER_TOKEN, **good)                      # accepted
    nv._check_cast_outputs(x, nv.PER_TENSOR, **dict(good, row_amax=f32(1), col_amax=f32(1)))
    bad_cases = [
        dict(good, row_amax=f32(1)),                                      # per-token row amax must be [M]
        dict(good, col_amax=f32(M)),                                      # [K], not [M]
        dict(good, row_q=u8(M * K // 2 - 1)),                             # short data buffer
        dict(good, col_sf=u8(K * M // 16 + 16)),                          # wrong scale count
        dict(good, row_amax=torch.zeros(M, dtype=torch.float64)),         # amax read as raw fp32 bits
        dict(good, row_q=torch.zeros(M * K, dtype=torch.uint8)[::2]),    # not contiguous
        dict(good, col_q=None),                                           # a direction half given
        dict(good, row_sf=torch.zeros(M * K // 16, dtype=torch.uint8, device="meta")),   # another device
    ]
    for kw in bad_cases:
        with pytest.raises(ValueError):
            nv._check_cast_outputs(x, nv.PER_TOKEN, **kw)
    with pytest.raises(ValueError):
        nv._check_cast_outputs(x, nv.PER_TENSOR, **good)                 # per-tensor amax is [1]
    # a shape the library rejects is left to the library (ESHAPE), not the size check
    nv._check_cast_outputs(torch.zeros(M, 40, dtype=torch.bfloat16), nv.PER_TOKEN,
                           row_q=u8(1), row_sf=u8(1), row_amax=f32(1))
    with pytest.raises(ValueError):
        nv._check_buf(f32(3), torch.float32, 4, torch.device("cpu"), "buf")
    nv._check_buf(f32(3), torch.float32, None, torch.device("cpu"), "buf", min_numel=1)
    with pytest.raises(ValueError):
        nv._check_buf(f32(0), torch.float32, None, torch.device("cpu"), "buf", min_numel=1)
