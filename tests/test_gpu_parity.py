"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact on every output byte (packed E2M1 data, E4M3 scale codes) and on
the fp32 amax bit patterns.  Every output buffer sits between canary-filled guard regions
(tests/gpu_util.py): the guards must survive the call and the buffer is
compared in full, so an unwritten byte or a write past an end fails.
Small shapes span several workgroup tiles and a ragged tail; the full-size workloads are compared in full where the oracle
finishes in seconds, otherwise on sampled rows / columns / tiles that the
oracle computes one by one, plus the complete amax vectors.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_bf16_amd as nv
from nvfp4_block_scaled_bf16_amd import workloads as W
from tests.gpu_util import (Guarded, assert_bytes_equal, cast_spec, compare_cast, grouped_spec, host,
                            quantize_guarded, to_dev)

pytestmark = pytest.mark.gpu

MODES = [nv.PER_TENSOR, nv.PER_TOKEN, nv.TILE_16x16]
# several 512-column tiles and 64/256-row tiles, with ragged tails
SHAPES = [(16, 16), (32, 512), (48, 1040), (272, 528), (1072, 544), (64, 8192), (2048, 48)]


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _x(M, K, seed):
    return W.row_scaled_with_outliers(M, K, seed)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", SHAPES)
def test_cast_small_shapes(oracle, mode, shape):
    M, K = shape
    x = _x(M, K, 100 + M + K)
    _announce(f"quantize mode={mode} shape={shape}")
    out = quantize_guarded(to_dev(x), mode)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, mode))


@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
def test_rowwise_only_ragged_rows(oracle, mode):
    x = _x(37, 96, 7)
    _announce(f"rowwise 37x96 mode={mode}")
    d = to_dev(x)
    out = Guarded(cast_spec(37, 96, mode, True, False))
    nv._check(nv.lib().nvfp4_quantize_rowwise(nv._ptr(d), 37, 96, mode, nv._ptr(out["row_q"]), nv._ptr(out["row_sf"]),
                                              nv._ptr(out["row_amax"]), nv._stream(d.device)))
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, mode, rowwise=True, columnwise=False))


@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
def test_columnwise_only_narrow(oracle, mode):
    x = _x(48, 24, 8)
    _announce(f"columnwise 48x24 mode={mode}")
    d = to_dev(x)
    out = Guarded(cast_spec(48, 24, mode, False, True))
    nv._check(nv.lib().nvfp4_quantize_columnwise(nv._ptr(d), 48, 24, mode, nv._ptr(out["col_q"]), nv._ptr(out["col_sf"]),
                                                 nv._ptr(out["col_amax"]), nv._stream(d.device)))
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, mode, rowwise=False, columnwise=True))


def _crafted(M=64, K=1024, seed=3):
    """Zeros, negative zeros, bf16 subnormals, huge values, exact grid ties,
    blocks whose scale rounds to a subnormal or to zero."""
    rng = np.random.default_rng(seed)
    f = rng.standard_normal((M, K)).astype(np.float32)
    f[0] = 0.0
    f[1, :64] = -0.0
    f[2, 5] = 2688.0
    f[2, 16:32] = 1e-4
    f[2, 32:48] = 3e-7
    f[3] = (rng.integers(-12, 13, K) * 0.25).astype(np.float32)   # exact ties with S = 1
    f[3, 0] = 2688.0
    f[4] = np.float32(2.0 ** -130) * rng.integers(-3, 4, K)       # bf16 subnormals
    f[5] = np.float32(3.0e38) * rng.choice([-1.0, 1.0], K).astype(np.float32)
    f[6, ::2] = -0.0
    f[7] = rng.standard_normal(K).astype(np.float32) * np.float32(1e-38)
    f[:, 7] = 0.0
    f[:, 9] = -0.0
    f[8:24, 100] = 6.0 * 448.0
    # negative bf16 subnormals inside blocks whose scale is normal: their
    # quotients are fp32 subnormals (or round to -0) in both directions
    sub = np.float32(-(2.0 ** -130))
    f[9, 0:16:3] = sub
    f[9, 17] = np.float32(-(2.0 ** -133))
    f[16:32, 300] = rng.standard_normal(16).astype(np.float32)
    f[20, 300] = sub
    f[23, 300] = np.float32(-(2.0 ** -127))
    return W.bf16_from_f32(f)


@pytest.mark.parametrize("mode", MODES)
def test_crafted_edges(oracle, mode):
    x = _crafted()
    _announce(f"crafted 64x1024 mode={mode}")
    out = quantize_guarded(to_dev(x), mode)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, mode))


def test_all_zero_and_single_row(oracle):
    for shape in [(16, 32), (1, 16)]:
        x = np.zeros(shape, np.uint16)
        x.reshape(-1)[3] = 0x8000
        for mode in (nv.PER_TENSOR, nv.PER_TOKEN):
            _announce(f"zeros {shape} mode={mode}")
            col = shape[0] % 16 == 0
            out = quantize_guarded(to_dev(x), mode, rowwise=True, columnwise=col)
            torch.cuda.synchronize()
            compare_cast(out, oracle.quantize(x, mode, rowwise=True, columnwise=col))


def _encode_guarded(d, mode, ra, ca):
    M, K = d.shape
    spec = {k: v for k, v in cast_spec(M, K, mode).items() if not k.endswith("amax")}
    out = Guarded(spec)
    nv.encode_into(d, mode, torch.from_numpy(ra).cuda(), torch.from_numpy(ca).cuda(), **out.views)
    torch.cuda.synchronize()
    out.check_guards()
    return out


def _compare_encode(oracle, x, out, ra, ca, per_token):
    q, sf = oracle.encode_rowwise(x, ra, per_token)
    assert_bytes_equal(host(out["row_q"]).reshape(q.shape), q, "row_q")
    assert_bytes_equal(host(out["row_sf"]).reshape(sf.shape), sf, "row_sf")
    q, sf = oracle.encode_colwise(x, ca, per_token)
    assert_bytes_equal(host(out["col_q"]).reshape(q.shape), q, "col_q")
    assert_bytes_equal(host(out["col_sf"]).reshape(sf.shape), sf, "col_sf")


def test_encode_with_supplied_amax_saturates(oracle):
    x = _x(64, 512, 9)
    d = to_dev(x)
    true_r, true_c = oracle.amax_rows(x), oracle.amax_cols(x)
    for fr, fc in [(1 / 64.0, 1 / 16.0), (3.0, 0.5), (1.0, 1.0)]:
        ra = (true_r * np.float32(fr)).astype(np.float32)
        ca = (true_c * np.float32(fc)).astype(np.float32)
        _announce(f"encode per-token factors {fr} {fc}")
        _compare_encode(oracle, x, _encode_guarded(d, nv.PER_TOKEN, ra, ca), ra, ca, True)
    # per-tensor with different rowwise / columnwise scalars
    ra = np.array([oracle.amax_tensor(x) * np.float32(0.25)], np.float32)
    ca = np.array([oracle.amax_tensor(x) * np.float32(2.0)], np.float32)
    _announce("encode per-tensor, different scalars")
    _compare_encode(oracle, x, _encode_guarded(d, nv.PER_TENSOR, ra, ca), ra, ca, False)


def test_encode_with_supplied_zero_amax(oracle):
    """A supplied amax of 0 over nonzero data (delayed scaling from a
    zero-initialised calibration buffer) gives scale code 0 and sign-only
    nibbles for that vector, as S == 0 does in the oracle."""
    x = _x(64, 512, 19)
    d = to_dev(x)
    ra, ca = oracle.amax_rows(x).copy(), oracle.amax_cols(x).copy()
    ra[[0, 5, 31, 32, 63]] = 0.0
    ca[[0, 7, 8, 255, 256, 511]] = 0.0
    _announce("encode per-token with zero entries in the supplied amax")
    _compare_encode(oracle, x, _encode_guarded(d, nv.PER_TOKEN, ra, ca), ra, ca, True)
    z = np.zeros(1, np.float32)
    _announce("encode per-tensor with a supplied amax of 0")
    _compare_encode(oracle, x, _encode_guarded(d, nv.PER_TENSOR, z, z), z, z, False)
    ok = np.array([oracle.amax_tensor(x)], np.float32)
    _announce("encode per-tensor: rowwise amax 0, columnwise the tensor's")
    _compare_encode(oracle, x, _encode_guarded(d, nv.PER_TENSOR, z, ok), z, ok, False)


@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
def test_split_amax(oracle, mode):
    x = _x(272, 1040, 10)
    _announce(f"amax 272x1040 mode={mode}")
    out = nv.amax(to_dev(x), mode)
    torch.cuda.synchronize()
    if mode == nv.PER_TOKEN:
        assert_bytes_equal(host(out["row_amax"]), oracle.amax_rows(x), "row_amax")
        assert_bytes_equal(host(out["col_amax"]), oracle.amax_cols(x), "col_amax")
    else:
        A = np.array([oracle.amax_tensor(x)], np.float32)
        assert_bytes_equal(host(out["row_amax"]), A, "row_amax")
        assert_bytes_equal(host(out["col_amax"]), A, "col_amax")


def _grouped_case(counts, K, seed):
    rng = np.random.default_rng(seed)
    T = int(sum(counts))
    scales = rng.uniform(0.5, 4.0, len(counts)).astype(np.float32)
    f = rng.standard_normal((T, K)).astype(np.float32) * np.repeat(scales, counts)[:, None]
    return W.bf16_from_f32(f)


@pytest.mark.parametrize("counts,K", [([32, 0, 16, 48, 0, 16, 128], 96),
                                      ([0, 0, 64], 512),
                                      ([16] * 70 + [0] * 40 + [32] * 30, 48),
                                      ([256, 512, 0, 128], 1040),
                                      ([64, 0, 32, 32] + [128] * 31, 256),
                                      ([64, 0, 32, 32] + [128] * 30 + [144], 512),
                                      ([32, 0, 32, 32, 32] + [128] * 31, 256)])
def test_grouped_small(oracle, counts, K):
    """Grouped casts of a few shapes, among them 128-row encode tiles owned
    by four and by five consecutive table entries with an empty expert among
    them, and a ragged last tile."""
    x = _grouped_case(counts, K, len(counts))
    _announce(f"grouped experts={len(counts)} T={sum(counts)} K={K}")
    out = Guarded(grouped_spec(sum(counts), K, len(counts)))
    nv.quantize_grouped_into(to_dev(x), counts, **out.views)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize_grouped(x, np.array(counts, np.int64)))


def _bf16_rne(f32):
    """Round-to-nearest-even of fp32 values to bf16 bit patterns, written out
    here (a second route to what the library's bf16 output must equal)."""
    u = np.ascontiguousarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _dequant_guarded(q, sf, amax, mode, bf16):
    R, C = q.shape[0], 2 * q.shape[1]
    out = Guarded({"out": (R * C, torch.bfloat16 if bf16 else torch.float32)})
    nv._check(nv.lib().nvfp4_dequantize(nv._ptr(q), nv._ptr(sf), nv._ptr(amax), R, C, mode, int(bf16),
                                        nv._ptr(out["out"]), nv._stream(q.device)))
    torch.cuda.synchronize()
    out.check_guards()
    return host(out["out"].view(torch.int16) if bf16 else out["out"]).reshape(R, C)


def test_dequantize_roundtrip(oracle):
    """fp32 and bf16 outputs of every mode against the oracle's fp32
    dequantization (bf16: its round to nearest-even)."""
    x = W.c1()
    _announce("C1 dequantize, fp32 and bf16 outputs")
    d = to_dev(x)
    out = nv.quantize(d, nv.PER_TENSOR)
    tok = nv.quantize(d, nv.PER_TOKEN)
    til = nv.quantize(d, nv.TILE_16x16)
    torch.cuda.synchronize()
    ref = oracle.quantize(x, nv.PER_TENSOR)
    reft = oracle.quantize(x, nv.PER_TOKEN)
    reftl = oracle.quantize(x, nv.TILE_16x16)
    cases = [
        ("row per-tensor", out, "row", nv.PER_TENSOR, oracle.dequantize(ref["row_q"], ref["row_sf"], ref["row_amax"], 256, 1024, False)),
        ("col per-tensor", out, "col", nv.PER_TENSOR, oracle.dequantize(ref["col_q"], ref["col_sf"], ref["col_amax"], 1024, 256, False)),
        ("row per-token", tok, "row", nv.PER_TOKEN, oracle.dequantize(reft["row_q"], reft["row_sf"], reft["row_amax"], 256, 1024, True)),
        ("col per-token", tok, "col", nv.PER_TOKEN, oracle.dequantize(reft["col_q"], reft["col_sf"], reft["col_amax"], 1024, 256, True)),
        ("row 16x16", til, "row", nv.TILE_16x16, oracle.dequantize(reftl["row_q"], reftl["row_sf"], reftl["row_amax"], 256, 1024, False)),
        ("col 16x16", til, "col", nv.TILE_16x16, oracle.dequantize(reftl["col_q"], reftl["col_sf"], reftl["col_amax"], 1024, 256, False)),
    ]
    for name, o, dr, mode, exp in cases:
        assert_bytes_equal(_dequant_guarded(o[dr + "_q"], o[dr + "_sf"], o[dr + "_amax"], mode, False), exp, name + " fp32")
        assert_bytes_equal(_dequant_guarded(o[dr + "_q"], o[dr + "_sf"], o[dr + "_amax"], mode, True).view(np.uint16),
                           _bf16_rne(exp), name + " bf16")
    # the bf16 rounding itself: ties, values just above a tie, large values
    # that round up to the next binade, and signed zeros
    assert list(_bf16_rne(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                                    -0.0, 3.3895e38], np.float32))) == [0x3F80, 0x3F82, 0x3F81, 0x8000, 0x7F7F]


@pytest.mark.parametrize("decay", [0.0, 0.9, 1.0])
def test_accumulate(oracle, decay):
    rng = np.random.default_rng(int(decay * 10) + 1)
    obs = (np.abs(rng.standard_normal((12, 1000))) * np.exp(rng.normal(0, 2, (12, 1)))).astype(np.float32)
    buf = torch.zeros(1000, dtype=torch.float32, device="cuda:0")
    sbuf = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    ref = np.zeros(1000, np.float32)
    sref = np.zeros(1, np.float32)
    _announce(f"accumulate decay={decay}")
    for t in range(12):
        o = torch.from_numpy(obs[t]).cuda()
        nv.amax_accumulate(buf, o, decay)
        nv.amax_accumulate_reduce(sbuf, o, decay)
        ref = oracle.amax_accumulate(ref, obs[t], decay)
        sref = oracle.amax_accumulate_reduce(sref, obs[t], decay)
    torch.cuda.synchronize()
    assert_bytes_equal(host(buf), ref, "buf")
    assert_bytes_equal(host(sbuf), sref, "sbuf")


@pytest.mark.parametrize("mode,shape,dirs", [(nv.PER_TOKEN, (272, 528), (True, True)),
                                             (nv.PER_TOKEN, (96, 1040), (True, False)),
                                             (nv.PER_TOKEN, (48, 24), (False, True)),
                                             (nv.PER_TENSOR, (272, 528), (True, True)),
                                             (nv.TILE_16x16, (64, 512), (False, True))])
def test_quantize_calibrate_matches_cast_then_accumulate(oracle, mode, shape, dirs):
    """The folded calibration update equals the oracle's decayed accumulate
    of the tensor amax, over several calls, and the cast is unchanged."""
    M, K = shape
    row, col = dirs
    _announce(f"quantize_calibrate mode={mode} shape={shape} row={row} col={col}")
    buf = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    ref = np.zeros(1, np.float32)
    for it, decay in enumerate([0.9, 0.9, 0.5, 1.0, 0.0, 0.9]):
        x = _x(M, K, 500 + it)
        if it == 3:
            x = (x & np.uint16(0x8000)) | ((x & np.uint16(0x7FFF)) >> np.uint16(1))   # smaller amax: decay shows
        d = to_dev(x)
        out = Guarded(cast_spec(M, K, mode, row, col))
        nv.quantize_calibrate_into(d, mode, buf, decay, **out.views)
        torch.cuda.synchronize()
        exp = oracle.quantize(x, mode, rowwise=row, columnwise=col)
        compare_cast(out, exp)
        A = np.array([oracle.amax_tensor(x)], np.float32)
        ref = oracle.amax_accumulate(ref, A, decay)
        assert_bytes_equal(host(buf), ref, f"buf after call {it}")


def test_quantize_calibrate_empty_tensor(oracle):
    """An empty tensor observes amax 0: buf = max(buf * decay, 0).  (Output
    buffers are non-empty allocations: a NULL pointer means 'direction not
    requested'.)"""
    _announce("quantize_calibrate of a 0 x 32 tensor")
    buf = torch.full((1,), 3.0, dtype=torch.float32, device="cuda:0")
    x = torch.empty(0, 32, dtype=torch.bfloat16, device="cuda:0")
    dummy = lambda dt: torch.empty(16, dtype=dt, device="cuda:0")
    nv.quantize_calibrate_into(x, nv.PER_TOKEN, buf, 0.5, row_q=dummy(torch.uint8), row_sf=dummy(torch.uint8),
                               row_amax=dummy(torch.float32))
    torch.cuda.synchronize()
    assert_bytes_equal(host(buf), np.array([1.5], np.float32), "buf")


def test_trace_encode_brackets_the_encoding_kernel(oracle):
    x = _x(1072, 544, 21)
    _announce("trace_encode events around a per-token cast")
    d = to_dev(x)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nv.trace_encode(a, b)
    out = quantize_guarded(d, nv.PER_TOKEN)
    again = quantize_guarded(d, nv.PER_TOKEN)   # the pair was consumed by the first call
    torch.cuda.synchronize()
    assert a.elapsed_time(b) > 0.0
    compare_cast(out, oracle.quantize(x, nv.PER_TOKEN))
    for k in out.keys():
        assert torch.equal(out[k], again[k]), k
    nv.trace_encode(a, b)
    nv.trace_encode(None, None)   # cancelled: nothing is recorded
    nv.quantize(d, nv.PER_TOKEN)
    torch.cuda.synchronize()


# ------------------------------------------------------- named workloads

def test_c1_per_tensor_rowwise(oracle):
    x = W.c1()
    _announce("C1 256x1024 per-tensor rowwise")
    out = quantize_guarded(to_dev(x), nv.PER_TENSOR, rowwise=True, columnwise=False)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, nv.PER_TENSOR, rowwise=True, columnwise=False))


def test_c2_per_token_full(oracle):
    x = W.c2()
    _announce("C2 4096x4096 per-token row+col")
    d = to_dev(x)
    out = quantize_guarded(d, nv.PER_TOKEN)
    again = quantize_guarded(d, nv.PER_TOKEN)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, nv.PER_TOKEN))
    again.check_guards()
    for k in out.keys():
        assert torch.equal(out[k], again[k]), f"run-to-run difference in {k}"


@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
@pytest.mark.parametrize("M", [12032, 12288])
def test_encode_tile_height_switch(oracle, M, mode):
    """With K = 4096 (16 column tiles), 12032 rows give 752 workgroups of 256
    rows, so the encode pass uses 128-row tiles; 12288 rows give 768 and keep
    256-row tiles.  Both must match the oracle in full, and so must the
    calibrating call's outputs and decayed buffer."""
    x = W.row_scaled_with_outliers(M, 4096, 60 + M)
    _announce(f"{M}x4096 mode={mode} (encode tile-height switch)")
    d = to_dev(x)
    out = quantize_guarded(d, mode)
    buf = torch.full((1,), 2.0, dtype=torch.float32, device="cuda:0")
    cal = Guarded(cast_spec(M, 4096, mode))
    nv.quantize_calibrate_into(d, mode, buf, 0.5, **cal.views)
    torch.cuda.synchronize()
    ref = oracle.quantize(x, mode)
    compare_cast(out, ref)
    compare_cast(cal, ref)
    a = oracle.amax_tensor(x)
    expect = oracle.amax_accumulate(np.array([2.0], np.float32), np.array([a], np.float32), 0.5)
    assert_bytes_equal(host(buf), expect, "decayed buffer")


SR_SHAPES = [(16, 16), (48, 1040), (272, 528), (1072, 544), (2048, 48)]


def _sr_guarded(d, mode, seed, offset, rowwise=True, columnwise=True):
    M, K = d.shape
    g = Guarded(cast_spec(M, K, mode, rowwise, columnwise))
    nv.quantize_sr_into(d, mode, seed, offset, **g.views)
    return g


@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
@pytest.mark.parametrize("shape", SR_SHAPES)
def test_sr_small_shapes(oracle, mode, shape):
    M, K = shape
    x = _x(M, K, 300 + M + K)
    seed, offset = 0x9E3779B97F4A7C15 ^ (M * 131 + K), M + 3 * K
    _announce(f"quantize_sr mode={mode} shape={shape}")
    out = _sr_guarded(to_dev(x), mode, seed, offset)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize_sr(x, mode, seed, offset))


@pytest.mark.parametrize("mode", [nv.PER_TENSOR, nv.PER_TOKEN])
def test_sr_one_direction(oracle, mode):
    x = _x(37, 96, 12)
    _announce(f"quantize_sr rowwise 37x96 mode={mode}")
    out = _sr_guarded(to_dev(x), mode, 5, 6, rowwise=True, columnwise=False)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize_sr(x, mode, 5, 6, rowwise=True, columnwise=False))
    x = _x(48, 24, 13)
    _announce(f"quantize_sr columnwise 48x24 mode={mode}")
    out = _sr_guarded(to_dev(x), mode, 5, 6, rowwise=False, columnwise=True)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize_sr(x, mode, 5, 6, rowwise=False, columnwise=True))


def test_sr_crafted_edges(oracle):
    x = _crafted()
    for mode in (nv.PER_TENSOR, nv.PER_TOKEN):
        _announce(f"quantize_sr crafted mode={mode}")
        out = _sr_guarded(to_dev(x), mode, 123, 4)
        torch.cuda.synchronize()
        compare_cast(out, oracle.quantize_sr(x, mode, 123, 4))


def test_sr_c2_full_and_offsets(oracle):
    x = W.c2()
    d = to_dev(x)
    _announce("quantize_sr C2 4096x4096 per-token, offsets 0 and 1")
    a = _sr_guarded(d, nv.PER_TOKEN, 2024, 0)
    b = _sr_guarded(d, nv.PER_TOKEN, 2024, 0)
    c = _sr_guarded(d, nv.PER_TOKEN, 2024, 1)
    torch.cuda.synchronize()
    compare_cast(a, oracle.quantize_sr(x, nv.PER_TOKEN, 2024, 0))
    compare_cast(c, oracle.quantize_sr(x, nv.PER_TOKEN, 2024, 1))
    b.check_guards()
    for k in a.keys():
        assert torch.equal(a[k], b[k]), f"same seed and offset, different {k}"
    assert not torch.equal(a["row_q"], c["row_q"]) and not torch.equal(a["col_q"], c["col_q"])
    # the scales and amax do not depend on the randoms
    for k in ("row_sf", "col_sf", "row_amax", "col_amax"):
        assert torch.equal(a[k], c[k]), k


def test_sr_c3_per_token_full(oracle):
    x = W.c3(1)
    _announce("quantize_sr C3 16384x8192 per-token (full compare)")
    out = _sr_guarded(to_dev(x), nv.PER_TOKEN, 77, 9)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize_sr(x, nv.PER_TOKEN, 77, 9))


def _sample_vectors(x, out, mode, rows, cols, oracle):
    xf = W.bf16_to_f32(x)
    if mode == nv.PER_TOKEN:
        ra = host(out["row_amax"])
        ca = host(out["col_amax"])
        assert_bytes_equal(ra, oracle.amax_rows(x), "row_amax")
        assert_bytes_equal(ca, oracle.amax_cols(x), "col_amax")
    else:
        A = np.float32(oracle.amax_tensor(x))
        assert_bytes_equal(host(out["row_amax"]), np.array([A], np.float32), "row_amax")
        ra = np.full(x.shape[0], A, np.float32)
        ca = np.full(x.shape[1], A, np.float32)
    rq, rs = host(out["row_q"]), host(out["row_sf"])
    cq, cs = host(out["col_q"]), host(out["col_sf"])
    for r in rows:
        q, sf = oracle.quantize_vector(xf[r], ra[r])
        assert_bytes_equal(rq[r], q, f"row_q[{r}]")
        assert_bytes_equal(rs[r], sf, f"row_sf[{r}]")
    for c in cols:
        q, sf = oracle.quantize_vector(np.ascontiguousarray(xf[:, c]), ca[c])
        assert_bytes_equal(cq[c], q, f"col_q[{c}]")
        assert_bytes_equal(cs[c], sf, f"col_sf[{c}]")


def test_c3_per_token_full(oracle):
    x = W.c3(0)
    _announce("C3 16384x8192 per-token row+col (full compare)")
    out = quantize_guarded(to_dev(x), nv.PER_TOKEN)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, nv.PER_TOKEN))


def test_c3_per_tensor_full(oracle):
    x = W.c3(2)
    _announce("C3 16384x8192 per-tensor row+col (full compare)")
    out = quantize_guarded(to_dev(x), nv.PER_TENSOR)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, nv.PER_TENSOR))


def test_c3_bench_call_full(oracle):
    """The measured step's own call -- quantize_calibrate_into, per-token
    row+col, 16384x8192, decay 0.9 -- on the three inputs the step rotates
    through, three calls in a row into the same buffers: every output in
    full and the decayed buffer after each call."""
    buf = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    ref_buf = np.zeros(1, np.float32)
    out = Guarded(cast_spec(16384, 8192, nv.PER_TOKEN))
    for t in range(3):
        x = W.c3(t)
        _announce(f"C3 bench call (quantize_calibrate per-token), input {t}")
        nv.quantize_calibrate_into(to_dev(x), nv.PER_TOKEN, buf, 0.9, **out.views)
        torch.cuda.synchronize()
        ref = oracle.quantize(x, nv.PER_TOKEN)
        compare_cast(out, ref)
        ref_buf = oracle.amax_accumulate(ref_buf, np.array([ref["row_amax"].max()], np.float32), 0.9)
        assert_bytes_equal(host(buf), ref_buf, f"decayed buffer after call {t}")


def test_c3_sixteen_iterations_with_decay(oracle):
    """Per-tensor and per-token casts of 16 seeded tensors; the per-tensor
    amax (= max of the per-token row amax) feeds buf = max(buf*0.9, A)."""
    rng = np.random.default_rng(33)
    buf = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    buf_tok = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    ref = np.zeros(1, np.float32)
    for t in range(16):
        x = W.c3(t)
        _announce(f"C3 iteration {t}")
        d = to_dev(x)
        pt = nv.quantize(d, nv.PER_TENSOR)
        tok = nv.quantize(d, nv.PER_TOKEN)
        nv.amax_accumulate(buf, pt["row_amax"], 0.9)
        nv.amax_accumulate_reduce(buf_tok, tok["row_amax"], 0.9)
        torch.cuda.synchronize()
        ref = oracle.amax_accumulate(ref, np.array([oracle.amax_tensor(x)], np.float32), 0.9)
        assert_bytes_equal(host(buf), ref, f"decayed buffer after iteration {t}")
        assert_bytes_equal(host(buf_tok), ref, f"decayed buffer (per-token feed) after iteration {t}")
        if t in (0, 15):
            rows = list(rng.choice(16384, 24, replace=False)) + [0, 16383]
            cols = list(rng.choice(8192, 24, replace=False)) + [0, 8191]
            _sample_vectors(x, pt, nv.PER_TENSOR, rows, cols, oracle)
            _sample_vectors(x, tok, nv.PER_TOKEN, rows, cols, oracle)


def test_c4_grouped_moe(oracle):
    x, counts = W.c4()
    assert int(counts.sum()) == 32768 and (counts % 128 == 0).all()
    _announce(f"C4 grouped 64 experts, zero-count experts: {int((counts == 0).sum())}")
    out = Guarded(grouped_spec(int(counts.sum()), x.shape[1], len(counts)))
    nv.quantize_grouped_into(to_dev(x), counts.tolist(), **out.views)
    torch.cuda.synchronize()
    ref = oracle.quantize_grouped(x, counts)
    compare_cast(out, ref)


def test_grouped_many_experts_per_amax_tile(oracle):
    """Thirty-two 16-row experts in each of the first two 512-row tiles of
    the amax pass (4096 x 32768 gives 512 workgroups of 512 rows, so every
    LDS slot of the per-expert column maxima is taken), then 48-row experts
    straddling tile boundaries."""
    counts = [16] * 64 + [48] * 64
    K = 32768
    x = _grouped_case(counts, K, 4097)
    _announce(f"grouped 128 experts (16 and 48 rows), T={sum(counts)} K={K}")
    out = Guarded(grouped_spec(sum(counts), K, len(counts)))
    nv.quantize_grouped_into(to_dev(x), counts, **out.views)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize_grouped(x, np.array(counts, np.int64)))


def test_c5_tile_16x16_full(oracle):
    x = W.c5()
    _announce("C5 8192x28672 16x16 tiles (full compare)")
    out = quantize_guarded(to_dev(x), nv.TILE_16x16)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, nv.TILE_16x16))


# ------------------------------------------- single-pass per-token rowwise

# K values covering every round configuration of the single-pass row kernel
# (4096 columns per round; 1, 2, 4, 8, 16 rounds, whole or with a partial
# last round) and M values with ragged last batches
ROWS_SHAPES = [(37, 4096), (100, 4112), (24, 12288), (40, 16384), (9, 16400), (18, 32768), (3, 65536),
               (5, 40976), (1, 16), (300, 2064)]


@pytest.mark.parametrize("shape", ROWS_SHAPES)
def test_rows_single_pass_rowwise_only(oracle, shape):
    M, K = shape
    x = _x(M, K, 700 + M + K)
    _announce(f"single-pass rowwise per-token M={M} K={K}")
    out = quantize_guarded(to_dev(x), nv.PER_TOKEN, rowwise=True, columnwise=False)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, nv.PER_TOKEN, rowwise=True, columnwise=False))


@pytest.mark.parametrize("shape", [(48, 4096), (112, 4112), (32, 12288), (16, 16384), (4128, 1040), (4112, 8192)])
def test_cast_row_and_col_wide_shapes(oracle, shape):
    """Per-token row + column casts at the widths the single-pass rowwise
    kernel covers in several round configurations (the row + column cast
    itself takes the amax and encoding kernels)."""
    M, K = shape
    x = _x(M, K, 800 + M + K)
    _announce(f"row + col per-token M={M} K={K}")
    out = quantize_guarded(to_dev(x), nv.PER_TOKEN)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(x, nv.PER_TOKEN))


def test_rows_single_pass_crafted(oracle):
    """The exact path of the row kernel: E4M3-subnormal block scales, zero
    rows, huge rows, ties, subnormals (K = 1024: one partial round, 8 rows
    per batch), rowwise only (and the row + column cast on the same data)."""
    x = _crafted()
    for col in (False, True):
        _announce(f"single-pass crafted 64x1024 columnwise={col}")
        out = quantize_guarded(to_dev(x), nv.PER_TOKEN, rowwise=True, columnwise=col)
        torch.cuda.synchronize()
        compare_cast(out, oracle.quantize(x, nv.PER_TOKEN, rowwise=True, columnwise=col))
    # rows whose amax is outside the fast range (the whole row takes the
    # exact path) next to ordinary rows, at K = 8192
    rng = np.random.default_rng(41)
    f = rng.standard_normal((24, 8192)).astype(np.float32)
    f[3] *= np.float32(1e-13)
    f[10] *= np.float32(1e19)
    f[17, :100] = 0.0
    f[17, 100] = np.float32(2.0 ** -126)
    xx = W.bf16_from_f32(f)
    _announce("single-pass crafted 24x8192 (outer amax outside the fast range)")
    out = quantize_guarded(to_dev(xx), nv.PER_TOKEN, rowwise=True, columnwise=False)
    torch.cuda.synchronize()
    compare_cast(out, oracle.quantize(xx, nv.PER_TOKEN, rowwise=True, columnwise=False))


def test_rows_grouped_rowwise_only(oracle):
    counts = [32, 0, 16, 48, 0, 16, 128, 4096]
    K = 4096
    x = _grouped_case(counts, K, 99)
    _announce("grouped rowwise only (single pass)")
    out = Guarded(grouped_spec(sum(counts), K, len(counts), rowwise=True, columnwise=False))
    nv.quantize_grouped_into(to_dev(x), counts, **out.views)
    torch.cuda.synchronize()
    ref = oracle.quantize_grouped(x, np.array(counts, np.int64))
    compare_cast(out, ref, keys=["row_q", "row_sf", "row_amax"])


def test_rows_calibrate_rowwise_only(oracle):
    M, K = 520, 8192
    buf = torch.full((1,), 5.0, dtype=torch.float32, device="cuda:0")
    ref = np.array([5.0], np.float32)
    for it in range(3):
        x = _x(M, K, 900 + it)
        _announce(f"single-pass rowwise calibrate, call {it}")
        out = Guarded(cast_spec(M, K, nv.PER_TOKEN, True, False))
        nv.quantize_calibrate_into(to_dev(x), nv.PER_TOKEN, buf, 0.5, **out.views)
        torch.cuda.synchronize()
        compare_cast(out, oracle.quantize(x, nv.PER_TOKEN, rowwise=True, columnwise=False))
        ref = oracle.amax_accumulate(ref, np.array([oracle.amax_tensor(x)], np.float32), 0.5)
        assert_bytes_equal(host(buf), ref, f"decayed buffer after call {it}")
