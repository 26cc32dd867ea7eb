"""Pins of the oracle's KIVI int8 / int4 encoding (KVBoost page, section 4.5,
Eq. 7, b in {8, 4})."""
import numpy as np
import pytest

from oracle import kivi


def test_key_encoding_bounds(rng):
    pool_cu = np.array([0, 40, 41, 100])
    k = rng.standard_normal((100, 2, 16)).astype(np.float32) * 3
    k[40] = 1.5                                  # one-token chunk: constant groups
    codes, kmin, ksc = kivi.encode_keys(k, pool_cu)
    assert codes.dtype == np.uint8
    dec = kivi.decode_keys(codes, kmin, ksc, pool_cu)
    for c in range(3):
        a, b = pool_cu[c], pool_cu[c + 1]
        blk = k[a:b].astype(np.float64)
        np.testing.assert_array_equal(kmin[c], k[a:b].min(axis=0))
        err = np.abs(dec[a:b] - blk)
        bound = ksc[c].astype(np.float64) / 2 * (1 + 1e-5) + 1e-6 * np.abs(blk).max()
        assert np.all(err <= bound[None])
        # the minimum decodes exactly, the maximum maps to 255
        amin = blk.argmin(axis=0)
        amax = blk.argmax(axis=0)
        for h in range(2):
            for j in range(16):
                assert codes[a + amin[h, j], h, j] == 0
                if ksc[c, h, j] > 0:
                    assert codes[a + amax[h, j], h, j] == 255
    np.testing.assert_array_equal(dec[40], k[40])
    assert np.all(ksc[1] == 0)


def test_value_encoding_bounds(rng):
    v = rng.standard_normal((64, 2, 128)).astype(np.float32)
    v[3, 1] = -0.25
    codes, vmin, vsc = kivi.encode_values(v)
    assert vmin.shape == (64, 2) and vsc.shape == (64, 2)
    dec = kivi.decode_values(codes, vmin, vsc)
    err = np.abs(dec - v.astype(np.float64))
    assert np.all(err <= vsc[..., None].astype(np.float64) / 2 * (1 + 1e-5) + 1e-6)
    np.testing.assert_array_equal(dec[3, 1], v[3, 1])
    assert codes.min() == 0 and codes.max() == 255


def test_encoding_is_affine_in_the_group_range(rng):
    # codes depend only on the position of x inside [min, max]: a group and
    # its image under x -> 2x + 1 (exact in float32 here) get the same codes
    k = (rng.integers(-64, 64, size=(32, 1, 8)) / 8.0).astype(np.float32)
    pool_cu = np.array([0, 32])
    c1, _, _ = kivi.encode_keys(k, pool_cu)
    c2, _, _ = kivi.encode_keys(2 * k + 1, pool_cu)
    np.testing.assert_array_equal(c1, c2)


@pytest.mark.parametrize("bits", [4, 8])
def test_bounds_at_both_widths(rng, bits):
    top = (1 << bits) - 1
    pool_cu = np.array([0, 17, 60])
    k = rng.standard_normal((60, 2, 8)).astype(np.float32)
    codes, kmin, ksc = kivi.encode_keys(k, pool_cu, bits=bits)
    assert codes.max() == top and codes.min() == 0
    dec = kivi.decode_keys(codes, kmin, ksc, pool_cu)
    for c in range(2):
        a, b = pool_cu[c], pool_cu[c + 1]
        np.testing.assert_allclose(ksc[c], (k[a:b].max(0) - k[a:b].min(0)) / np.float32(top),
                                   rtol=1e-6)
        err = np.abs(dec[a:b] - k[a:b].astype(np.float64))
        assert np.all(err <= ksc[c].astype(np.float64) / 2 * (1 + 1e-5) + 1e-6)
    v = rng.standard_normal((30, 2, 16)).astype(np.float32)
    vc, vmin, vsc = kivi.encode_values(v, bits=bits)
    assert vc.max() <= top
    err = np.abs(kivi.decode_values(vc, vmin, vsc) - v.astype(np.float64))
    assert np.all(err <= vsc[..., None].astype(np.float64) / 2 * (1 + 1e-5) + 1e-6)


def test_four_bits_is_a_coarser_grid(rng):
    """The 4-bit code of x is the 8-bit code's grid point rounded to every
    17th level: both place x on [min, max] with 15 and 255 steps, and
    255 = 15 * 17, so code8 / 17 and code4 differ by at most 1/2 + rounding."""
    x = rng.standard_normal((200, 1, 4)).astype(np.float32)
    c8, _, _ = kivi.encode_keys(x, np.array([0, 200]), bits=8)
    c4, _, _ = kivi.encode_keys(x, np.array([0, 200]), bits=4)
    assert np.all(np.abs(c8.astype(float) / 17 - c4.astype(float)) <= 0.5 + 0.5 / 17 + 1e-6)


def test_pack4_layout():
    codes = np.array([[1, 2, 3, 4], [15, 0, 0, 15]], dtype=np.uint8)
    packed = kivi.pack4(codes)
    np.testing.assert_array_equal(packed, np.array([[0x21, 0x43], [0x0F, 0xF0]], dtype=np.uint8))
    np.testing.assert_array_equal(kivi.unpack4(packed), codes)
    with pytest.raises(ValueError):
        kivi.pack4(np.array([16, 0], dtype=np.uint8))
    with pytest.raises(ValueError):
        kivi.levels(2)
