"""Pins of the oracle's KIVI int8 encoding (KVBoost page, section 4.5, Eq. 7)."""
import numpy as np

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
