"""The test-side tile-order helpers against the layout's definition (element
positions computed one by one from the formula in include/fp8moe.h)."""
import numpy as np
import pytest

import tile_layout as tl


@pytest.mark.parametrize("R,C", [(16, 64), (32, 128), (48, 192), (16, 320), (64, 256)])
def test_pack_places_every_element_by_the_formula(R, C):
    rng = np.random.default_rng(R * 1000 + C)
    codes = rng.integers(0, 256, (R, C), dtype=np.uint8)
    flat = tl.pack(codes).reshape(-1)
    CT = (C + 127) // 128
    assert flat.size == R * CT * 128
    for r in range(R):
        for c in range(C):
            assert flat[tl.tile_offset(r, c, C)] == codes[r, c]
    # everything not hit by an element is zero padding (only when C % 128 == 64)
    hit = np.zeros(flat.size, bool)
    hit[[tl.tile_offset(r, c, C) for r in range(R) for c in range(C)]] = True
    assert hit.sum() == R * C
    assert (flat[~hit] == 0).all()


def test_unpack_inverts_pack_with_leading_dims():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, (3, 32, 192), dtype=np.uint8)
    packed = tl.pack(codes)
    assert packed.shape == (3, 2, 2, 2048)
    np.testing.assert_array_equal(tl.unpack(packed, 32, 192), codes)


def test_tile_is_the_mfma_operand_of_a_wave():
    # lane l of a wave reads 16 contiguous bytes from each half of a tile:
    # row l % 16, K bytes 16*(l//16) + [0,16) and 64 + 16*(l//16) + [0,16)
    R, C = 16, 128
    codes = np.arange(R * C, dtype=np.int64).reshape(R, C)
    tile = tl.pack((codes % 251).astype(np.uint8)).reshape(2048)
    for l in range(64):
        lo = tile[l * 16:(l + 1) * 16]
        hi = tile[1024 + l * 16:1024 + (l + 1) * 16]
        k0 = 16 * (l // 16)
        np.testing.assert_array_equal(lo, (codes[l % 16, k0:k0 + 16] % 251).astype(np.uint8))
        np.testing.assert_array_equal(hi, (codes[l % 16, 64 + k0:64 + k0 + 16] % 251).astype(np.uint8))
