"""Pins of the oracle's GEMM-swizzled scale layout (CPU only).

The per-token recipe page emits unswizzled scales and leaves the swizzled
layout to the GEMM (TransformerEngine PR #3045: with_gemm_swizzled_scales
off, with_swizzle=0).  The oracle's reading is the 128-row x 4-block tiled
layout of block-scaled GEMMs, computed there with explicit index
arithmetic.  Pinned here by building the same layout another way (pad,
reshape, transpose with numpy) and by the properties that define it: the
tile of a scale, the 16-byte line per row within 32, the 4-byte slot per
group of 32 rows, the block within the slot, zero padding, and the inverse.
"""
import numpy as np
import pytest

import oracle


def _by_reshape(sf):
    """pad to [Rp][nbp], then axes (row tile, row in 4 groups, row in 32,
    block group, block in 4) -> (row tile, block group, row in 32, row group,
    block in 4), flattened"""
    R, nb = sf.shape
    Rp, nbp = -(-R // 128) * 128, -(-nb // 4) * 4
    p = np.zeros((Rp, nbp), np.uint8)
    p[:R, :nb] = sf
    return p.reshape(Rp // 128, 4, 32, nbp // 4, 4).transpose(0, 3, 2, 1, 4).ravel()


SHAPES = [(1, 1), (32, 4), (128, 4), (130, 5), (257, 9), (512, 64), (1000, 3)]


@pytest.mark.parametrize("shape", SHAPES)
def test_matches_reshape_construction(shape):
    rng = np.random.Generator(np.random.PCG64(sum(shape)))
    sf = rng.integers(1, 256, size=shape, dtype=np.uint8)
    sw = oracle.swizzle_scales(sf)
    assert np.array_equal(sw, _by_reshape(sf))
    assert np.array_equal(oracle.unswizzle_scales(sw, *shape), sf)


def test_defining_properties():
    R, nb = 300, 10
    rng = np.random.Generator(np.random.PCG64(7))
    sf = rng.integers(1, 256, size=(R, nb), dtype=np.uint8)
    sw = oracle.swizzle_scales(sf)
    # size: rows padded to 128, blocks to 4
    assert sw.size == 384 * 12
    pos = {}
    for r in range(R):
        for c in range(nb):
            marker = np.zeros((R, nb), np.uint8)
            marker[r, c] = 1
            pos[r, c] = int(np.flatnonzero(oracle.swizzle_scales(marker))[0]) if (r * nb + c) % 37 == 0 else None
    for (r, c), p in pos.items():
        if p is None:
            continue
        tile, within = divmod(p, 512)
        assert tile == (r // 128) * 3 + c // 4            # 512-byte tiles, row-tile major
        assert within // 16 == r % 32                       # 16-byte line per row within 32
        assert (within % 16) // 4 == (r // 32) % 4          # 4-byte slot per group of 32 rows
        assert within % 4 == c % 4                          # block within the slot
    # and the byte there is that scale
    assert all(sw[p] == sf[r, c] for (r, c), p in pos.items() if p is not None)


def test_padding_is_zero_and_values_move_intact():
    R, nb = 130, 5
    sf = np.full((R, nb), 0xAB, np.uint8)
    sw = oracle.swizzle_scales(sf)
    assert np.count_nonzero(sw == 0xAB) == R * nb
    assert np.count_nonzero(sw == 0) == sw.size - R * nb


def test_refuses_wrong_size():
    with pytest.raises(ValueError):
        oracle.unswizzle_scales(np.zeros(100, np.uint8), 130, 5)
