"""GPU parity of the NVFP4 GEMM consumer against the CPU oracle.

The kernel sums exact block-value products in fp32 on fp16 matrix cores and
then applies the two outer scales in fp32; the oracle sums in binary64.  The
tolerance follows from that arithmetic: every fp32 addition and the two scale
multiplications round once, each by at most 2^-24 of a magnitude no larger
than S_a S_b sum_k |term| (the oracle's ``bound``), so
    |gpu - exact| <= (K + 2) * 2^-24 * bound  (+ 2^-126 for fp32 underflow).
Where every partial sum is exactly representable (unit scales, E2M1 values)
the result must be bit-exact.  Operands come from the oracle's own cast of
the seeded workload tensors, or are raw seeded codes spanning every block
scale; nothing the oracle reads comes from the GPU.
"""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_bf16_amd as nv
from nvfp4_block_scaled_bf16_amd import workloads as W
from tests.gpu_util import host, to_dev

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _dev(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0") for a in arrays]


def _run(aq, asf, aa, bq, bsf, ba):
    out = nv.gemm(*_dev(aq, asf, aa, bq, bsf, ba))
    torch.cuda.synchronize()
    return host(out).astype(np.float64)


def _check(got, ref, bound, K, name):
    tol = (K + 2) * 2.0 ** -24 * bound + 2.0 ** -126
    err = np.abs(got - ref)
    bad = np.nonzero(err > tol)
    assert not bad[0].size, (f"{name}: {bad[0].size} of {got.size} outside tolerance; first at "
                             f"{bad[0][0], bad[1][0]}: got {got[bad][0]!r} expected {ref[bad][0]!r} "
                             f"tol {tol[bad][0]!r}")


def _cast_operand(rows, K, seed, per_row, oracle):
    x = W.row_scaled_with_outliers(rows, K, seed)
    o = oracle.quantize(x, oracle.PER_TOKEN if per_row else oracle.PER_TENSOR, columnwise=False)
    return o["row_q"], o["row_sf"], o["row_amax"]


# several 128 x 128 tiles with ragged edges; K with a partial 64-step
SHAPES = [(1, 1, 16), (16, 16, 16), (130, 200, 272), (256, 128, 64), (300, 520, 1040), (128, 384, 4096),
          (64, 1000, 48)]


@pytest.mark.parametrize("per_row", [(True, True), (True, False), (False, True), (False, False)])
@pytest.mark.parametrize("shape", SHAPES)
def test_gemm_cast_operands(oracle, shape, per_row):
    M, N, K = shape
    _announce(f"gemm cast operands M={M} N={N} K={K} per_row={per_row}")
    a = _cast_operand(M, K, 11, per_row[0], oracle)
    b = _cast_operand(N, K, 12, per_row[1], oracle)
    ref, bound = oracle.gemm_nvfp4(*a, *b)
    _check(_run(*a, *b), ref, bound, K, "out")


@pytest.mark.parametrize("shape", [(96, 136, 160), (257, 129, 528)])
def test_gemm_raw_codes_every_scale(oracle, shape):
    M, N, K = shape
    _announce(f"gemm raw codes M={M} N={N} K={K}")
    a = W.nvfp4_operand(M, K, 21)
    b = W.nvfp4_operand(N, K, 22, per_row=False)
    ref, bound = oracle.gemm_nvfp4(*a, *b)
    _check(_run(*a, *b), ref, bound, K, "out")


def _offset_copy(t, off):
    """the same bytes, at a device address `off` bytes past an aligned one"""
    buf = torch.zeros(t.numel() + 16, dtype=t.dtype, device=t.device)
    v = buf[off:off + t.numel()].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("off", [1, 2])
def test_gemm_unaligned_plain_scales(off):
    # K % 64 == 0 with plain scales at byte offsets: the byte loads serve
    # them, and the products equal the aligned call's bit for bit, single
    # and grouped
    M, N, K = 300, 260, 256
    _announce(f"gemm plain scales at byte offset {off}, M={M} N={N} K={K}")
    da, db = _dev(*W.nvfp4_operand(M, K, 31)), _dev(*W.nvfp4_operand(N, K, 32, per_row=False))
    ref = host(nv.gemm(*da, *db))
    da[1], db[1] = _offset_copy(da[1], off), _offset_copy(db[1], off)
    got = host(nv.gemm(*da, *db))
    torch.cuda.synchronize()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    counts = np.array([100, 0, 200], np.int64)
    ga, gb = _dev(*W.nvfp4_operand(300, K, 33)), _dev(*_grouped_b(3, N, K, 34, True))
    gref = host(nv.gemm_grouped(*ga, *gb, counts))
    ga[1], gb[1] = _offset_copy(ga[1], off), _offset_copy(gb[1], off)
    ggot = host(nv.gemm_grouped(*ga, *gb, counts))
    torch.cuda.synchronize()
    assert np.array_equal(ggot.view(np.uint32), gref.view(np.uint32))


def test_gemm_exact_when_sums_representable(oracle):
    # unit block scales (E4M3 0x38 = 1.0) and amax = 2688 (S = 1): every
    # product is a multiple of 1/4 below 36 and every partial sum is exact
    M, N, K = 200, 144, 1024
    _announce(f"gemm exact M={M} N={N} K={K}")
    rng = np.random.Generator(np.random.PCG64(31))
    aq = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    bq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    asf = np.full((M, K // 16), 0x38, np.uint8)
    bsf = np.full((N, K // 16), 0x38, np.uint8)
    aa = np.full(M, 2688.0, np.float32)
    ba = np.full(1, 2688.0, np.float32)
    ref, _ = oracle.gemm_nvfp4(aq, asf, aa, bq, bsf, ba)
    got = _run(aq, asf, aa, bq, bsf, ba)
    assert np.array_equal(got, ref)


def test_gemm_k_zero_and_empty():
    _announce("gemm K=0 / M=0")
    a = [np.zeros((5, 0), np.uint8), np.zeros((5, 0), np.uint8), np.ones(5, np.float32)]
    b = [np.zeros((7, 0), np.uint8), np.zeros((7, 0), np.uint8), np.ones(1, np.float32)]
    out = torch.full((5, 7), 3.0, dtype=torch.float32, device="cuda:0")
    nv.gemm_into(out, *_dev(*a), *_dev(*b))
    torch.cuda.synchronize()
    assert not host(out).any()
    e = nv.gemm(*_dev(np.zeros((0, 8), np.uint8), np.zeros((0, 1), np.uint8), np.ones(1, np.float32)),
                *_dev(*W.nvfp4_operand(4, 16, 1)))
    torch.cuda.synchronize()
    assert tuple(e.shape) == (0, 4)


def test_gemm_training_products(oracle):
    # forward Y = X W^T (TN), dgrad dX = dY W (NN: W columnwise), wgrad
    # dW = dY^T X (NT: dY and X columnwise), all from per-token casts
    T, K, N = 256, 192, 320
    _announce(f"gemm TN/NN/NT T={T} K={K} N={N}")
    X = W.row_scaled_with_outliers(T, K, 41)
    Wt = W.weight_with_outliers(N, K, 42)
    dY = W.row_scaled_with_outliers(T, N, 43)
    qx = oracle.quantize(X, oracle.PER_TOKEN)
    qw = oracle.quantize(Wt, oracle.PER_TOKEN)
    qd = oracle.quantize(dY, oracle.PER_TOKEN)

    def row(o):
        return o["row_q"], o["row_sf"], o["row_amax"]

    def col(o, R, C):   # columnwise output of an R x C tensor: C vectors of R
        return o["col_q"].reshape(C, R // 2), o["col_sf"].reshape(C, R // 16), o["col_amax"]

    for name, a, b, kk in (("TN", row(qx), row(qw), K), ("NN", row(qd), col(qw, N, K), N),
                           ("NT", col(qd, T, N), col(qx, T, K), T)):
        ref, bound = oracle.gemm_nvfp4(*a, *b)
        _check(_run(*a, *b), ref, bound, kk, name)


@pytest.mark.parametrize("K", [272, 320])
def test_gemm_large_tiles_ragged(oracle, K):
    # enough output tiles for the 256 x 256 tile shape, with ragged last tiles
    # in both directions; K = 272: a partial last K step (two-load pieces);
    # K = 320: whole 64-wide steps whose last 16-byte scale group (four
    # steps) is partial; sampled blocks including the corner tile
    M, N = 4000, 4100
    _announce(f"gemm 256-tile ragged M={M} N={N} K={K} (sampled)")
    a = W.nvfp4_operand(M, K, 61)
    b = W.nvfp4_operand(N, K, 62, per_row=False)
    out = host(nv.gemm(*_dev(*a), *_dev(*b)))
    torch.cuda.synchronize()
    for r0, c0 in ((0, 0), (M - 80, N - 70), (3800, 0), (0, 3900), (1000, 2000)):
        rs, cs = slice(r0, min(M, r0 + 80)), slice(c0, min(N, c0 + 70))
        ref, bound = oracle.gemm_nvfp4(a[0][rs], a[1][rs], a[2][rs], b[0][cs], b[1][cs], b[2])
        _check(out[rs, cs].astype(np.float64), ref, bound, K, f"block ({r0},{c0})")


def test_gemm_large_tiles_every_tile_written(oracle):
    # 256 x 256 tiles visited in groups of row bands: the output starts as
    # NaN and every element must come back within the bound (ragged M, N)
    M, N, K = 4100, 4000, 128
    _announce(f"gemm 256-tile full compare M={M} N={N} K={K}")
    a = W.nvfp4_operand(M, K, 63)
    b = W.nvfp4_operand(N, K, 64)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    nv.gemm_into(out, *_dev(*a), *_dev(*b))
    torch.cuda.synchronize()
    ref, bound = oracle.gemm_nvfp4(*a, *b)
    got = host(out).astype(np.float64)
    assert np.isfinite(got).all() and np.isfinite(ref).all()
    _check(got, ref, bound, K, "out")


def test_gemm_grouped_large_tiles_every_tile_written(oracle):
    # the grouped kernel on 256 x 256 tiles (eight experts of 1100 rows each):
    # NaN-filled output, full compare
    counts = np.full(8, 1100, np.int64)
    N, K = 2048, 64
    _announce(f"gemm grouped 256-tile full compare counts={counts.tolist()} N={N} K={K}")
    a = W.nvfp4_operand(int(counts.sum()), K, 65)
    b = _grouped_b(counts.size, N, K, 66, True)
    out = torch.full((int(counts.sum()), N), float("nan"), dtype=torch.float32, device="cuda:0")
    nv.gemm_grouped_into(out, *_dev(*a), *_dev(*b), counts)
    torch.cuda.synchronize()
    ref, bound = _grouped_ref(oracle, a, b, counts, True)
    got = host(out).astype(np.float64)
    assert np.isfinite(got).all() and np.isfinite(ref).all()
    _check(got, ref, bound, K, "out")


def test_gemm_full_size_sampled(oracle):
    # the forward product of the 16384 x 8192 activation with an 8192 x 8192
    # weight, in the launch configuration the benchmark times; the oracle
    # computes sampled 64 x 64 blocks (corners, the middle, a random block)
    M, N, K = 16384, 8192, 8192
    _announce(f"gemm full size M={M} N={N} K={K} (sampled)")
    a = W.nvfp4_operand(M, K, 51)
    b = W.nvfp4_operand(N, K, 52)
    out = host(nv.gemm(*_dev(*a), *_dev(*b)))
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(53))
    for r0, c0 in ((0, 0), (M - 64, N - 64), (M // 2 - 32, N // 2 - 32),
                   (int(rng.integers(0, M - 64)), int(rng.integers(0, N - 64)))):
        rs, cs = slice(r0, r0 + 64), slice(c0, c0 + 64)
        ref, bound = oracle.gemm_nvfp4(a[0][rs], a[1][rs], a[2][rs], b[0][cs], b[1][cs], b[2][cs])
        _check(out[rs, cs].astype(np.float64), ref, bound, K, f"block ({r0},{c0})")


# ----------------------------------------------------------------- grouped

def _grouped_ref(oracle, a, b, counts, b_per_row):
    """per group: the oracle's GEMM of the group's rows with its own B"""
    aq, asf, aa = a
    bq, bsf, ba = b
    G, N = bq.shape[0], bq.shape[1]
    refs, bounds = [], []
    off = 0
    for e, c in enumerate(counts):
        rs = slice(off, off + int(c))
        a_am = aa[rs] if aa.size != 1 else aa
        b_am = ba.reshape(G, N)[e] if b_per_row else ba[e:e + 1]
        if c:
            r, bd = oracle.gemm_nvfp4(aq[rs], asf[rs], a_am, bq[e], bsf[e], b_am)
            refs.append(r)
            bounds.append(bd)
        off += int(c)
    return np.concatenate(refs), np.concatenate(bounds)


def _grouped_b(G, N, K, seed, per_row):
    q, sf, amax = zip(*(W.nvfp4_operand(N, K, seed + e, per_row) for e in range(G)))
    return np.stack(q), np.stack(sf), np.concatenate(amax)


def _run_grouped(a, b, counts):
    out = nv.gemm_grouped(*_dev(*a), *_dev(*b), counts)
    torch.cuda.synchronize()
    return host(out).astype(np.float64)


@pytest.mark.parametrize("a_per_row,b_per_row", [(True, True), (True, False), (False, False)])
def test_gemm_grouped_ragged_counts(oracle, a_per_row, b_per_row):
    counts = np.array([5, 0, 130, 16, 0, 64, 257, 1], np.int64)
    N, K = 200, 272
    _announce(f"gemm grouped counts={counts.tolist()} N={N} K={K} per_row={a_per_row},{b_per_row}")
    a = W.nvfp4_operand(int(counts.sum()), K, 71, a_per_row)
    b = _grouped_b(len(counts), N, K, 72, b_per_row)
    ref, bound = _grouped_ref(oracle, a, b, counts, b_per_row)
    _check(_run_grouped(a, b, counts), ref, bound, K, "out")


def test_gemm_grouped_many_groups(oracle):
    # more groups than one launch carries, with empty ones among them
    rng = np.random.Generator(np.random.PCG64(81))
    counts = rng.integers(0, 40, size=300).astype(np.int64)
    counts[[0, 127, 128, 129, 299]] = 0
    N, K = 48, 64
    _announce(f"gemm grouped {counts.size} groups T={int(counts.sum())} N={N} K={K}")
    a = W.nvfp4_operand(int(counts.sum()), K, 82)
    b = _grouped_b(counts.size, N, K, 1000, True)
    ref, bound = _grouped_ref(oracle, a, b, counts, True)
    _check(_run_grouped(a, b, counts), ref, bound, K, "out")


def test_gemm_grouped_moe_cast(oracle):
    # the rowwise output of the oracle's grouped cast of an MoE batch (token
    # counts in multiples of 16, some experts empty) times per-expert weights
    x, counts = W.moe_batch(91, K=256, experts=12, chunks=24, align=16)
    N, K = 96, 256
    _announce(f"gemm grouped MoE cast counts={counts.tolist()}")
    q = oracle.quantize_grouped(x, counts, rowwise=True, columnwise=False)
    a = (q["row_q"], q["row_sf"], q["row_amax"])
    Wts = [W.weight_with_outliers(N, K, 92 + e) for e in range(counts.size)]
    qw = [oracle.quantize(w, oracle.PER_TOKEN, columnwise=False) for w in Wts]
    b = (np.stack([o["row_q"] for o in qw]), np.stack([o["row_sf"] for o in qw]),
         np.concatenate([o["row_amax"] for o in qw]))
    ref, bound = _grouped_ref(oracle, a, b, counts, True)
    _check(_run_grouped(a, b, counts), ref, bound, K, "out")


def test_gemm_grouped_large_tiles_sampled(oracle):
    # enough rows for the 256 x 256 tile shape; sampled blocks in each group
    counts = np.array([1024, 768, 1280, 1024, 512, 1536, 1024, 1024], np.int64)
    N, K = 2048, 512
    _announce(f"gemm grouped 256-tile counts={counts.tolist()} N={N} K={K} (sampled)")
    a = W.nvfp4_operand(int(counts.sum()), K, 101)
    b = _grouped_b(counts.size, N, K, 200, False)
    out = _run_grouped(a, b, counts)
    off = 0
    for e, c in enumerate(counts):
        for r0, c0 in ((off, 0), (off + int(c) - 48, N - 48)):
            rs, cs = slice(r0, r0 + 48), slice(c0, c0 + 48)
            ref, bound = oracle.gemm_nvfp4(a[0][rs], a[1][rs], a[2][rs], b[0][e][cs], b[1][e][cs], b[2][e:e + 1])
            _check(out[rs, cs], ref, bound, K, f"group {e} block ({r0},{c0})")
        off += int(c)


# ---------------------------------------------------- swizzled scale layout

@pytest.mark.parametrize("shape", [(1, 1), (130, 5), (257, 9), (1000, 3), (4096, 512), (8192, 1024)])
def test_swizzle_scales_bit_exact(oracle, shape):
    rng = np.random.Generator(np.random.PCG64(sum(shape)))
    sf = rng.integers(0, 256, size=shape, dtype=np.uint8)
    _announce(f"swizzle scales {shape}")
    got = host(nv.swizzle_scales(_dev(sf)[0]))
    torch.cuda.synchronize()
    assert np.array_equal(got, oracle.swizzle_scales(sf))


def test_swizzle_of_cast_outputs(oracle):
    # the cast's rowwise and columnwise scales, swizzled on the GPU, against
    # the oracle's swizzle of the oracle's cast
    x = W.row_scaled_with_outliers(272, 528, 111)
    _announce("swizzle of the cast's scales 272x528")
    out = nv.quantize(to_dev(x), nv.PER_TOKEN)
    ref = oracle.quantize(x, nv.PER_TOKEN)
    row = host(nv.swizzle_scales(out["row_sf"]))
    col = host(nv.swizzle_scales(out["col_sf"]))
    torch.cuda.synchronize()
    assert np.array_equal(row, oracle.swizzle_scales(ref["row_sf"]))
    assert np.array_equal(col, oracle.swizzle_scales(ref["col_sf"]))


@pytest.mark.parametrize("shape", [(130, 200, 272), (300, 520, 1040), (4000, 4100, 272), (260, 390, 1024), (4000, 4100, 320)])
def test_gemm_swizzled_equals_plain(oracle, shape):
    # same arithmetic: bit-identical to the plain-layout GEMM; the small
    # shape also against the oracle
    M, N, K = shape
    _announce(f"gemm swizzled M={M} N={N} K={K}")
    a = W.nvfp4_operand(M, K, 121)
    b = W.nvfp4_operand(N, K, 122, per_row=False)
    da, db = _dev(*a), _dev(*b)
    plain = nv.gemm(*da, *db)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    asw = _dev(oracle.swizzle_scales(a[1]))[0]
    bsw = _dev(oracle.swizzle_scales(b[1]))[0]
    nv.gemm_swizzled_into(out, da[0], asw, da[2], db[0], bsw, db[2])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), plain.view(torch.int32))
    if M * N * K < 10 ** 9:
        ref, bound = oracle.gemm_nvfp4(*a, *b)
        _check(host(out).astype(np.float64), ref, bound, K, "out")
