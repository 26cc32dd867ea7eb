"""Pins of the oracle's rotary embedding and re-positioning (CPU only).

The checks come from outside the oracle's own code path: multiplication by a
complex exponential, the group law of rotations, the relative-offset
property of the KVBoost page (section 3.2, Eq. 3) and that page's worked
case of a key cached at 50 and reused at 1050 via R^1000.
"""
import json
import os

import numpy as np
import pytest

from oracle import rope, fusion

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _complex_rotate(x, pos, freqs):
    """Rotate-half RoPE as complex multiplication: z_j = x_j + i x_{j+d/2}
    times exp(i pos theta_j)."""
    h = x.shape[-1] // 2
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[:, None, None] * freqs[None, None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("d,base", [(64, 1e4), (128, 1e6), (128, 5e5), (8, 10.0)])
def test_frequency_schedule_is_geometric_from_one(d, base):
    f = rope.inverse_frequencies(d, base)
    assert f.shape == (d // 2,)
    assert f[0] == 1.0                                   # base ** 0
    ratio = f[1:] / f[:-1]
    np.testing.assert_allclose(ratio, base ** (-2.0 / d), rtol=1e-13)
    # theta_j * theta_{d/2 - j} = 1 / base for 0 < j < d/2
    j = np.arange(1, d // 2)
    np.testing.assert_allclose(f[j] * f[d // 2 - j], 1.0 / base, rtol=1e-12)


@pytest.mark.parametrize("d,base", [(64, 1e4), (128, 1e6)])
def test_rotation_equals_complex_multiplication(rng, d, base):
    x = rng.standard_normal((37, 3, d))
    pos = rng.integers(0, 40000, size=37)
    ref = _complex_rotate(x, pos, rope.inverse_frequencies(d, base))
    np.testing.assert_allclose(rope.rotate(x, pos, base), ref, rtol=0, atol=1e-12)


def test_single_pair_is_plane_rotation():
    # d = 2: theta_0 = 1, so R(p) is the plane rotation by p radians.
    x = np.array([[[1.0, 0.0]]])
    for p in (0.0, np.pi / 2, np.pi, 1.0):
        y = rope.rotate(x, np.array([p]), 1e4)[0, 0]
        np.testing.assert_allclose(y, [np.cos(p), np.sin(p)], atol=1e-15)


def test_group_law_identity_and_norm(rng):
    d, base = 128, 1e6
    x = rng.standard_normal((50, 2, d))
    a = rng.integers(0, 20000, size=50)
    b = rng.integers(0, 20000, size=50)
    ab = rope.rotate(rope.rotate(x, b, base), a, base)
    np.testing.assert_allclose(ab, rope.rotate(x, a + b, base), atol=1e-11)
    np.testing.assert_allclose(rope.rotate(x, np.zeros(50), base), x, atol=0)
    np.testing.assert_allclose(np.linalg.norm(rope.rotate(x, a, base), axis=-1),
                               np.linalg.norm(x, axis=-1), rtol=1e-13)
    # inverse: R(-a) R(a) = I
    np.testing.assert_allclose(rope.rotate(rope.rotate(x, a, base), -a, base), x, atol=1e-11)


def test_relative_offset_property(rng):
    # KVBoost section 3.2, Eq. 3: q'_s . k'_t depends only on t - s.
    d, base = 128, 1e6
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    for s, t, shift in [(3, 10, 1000), (500, 20, 7), (0, 0, 33000)]:
        d0 = np.sum(rope.rotate(q, [s], base) * rope.rotate(k, [t], base))
        d1 = np.sum(rope.rotate(q, [s + shift], base) * rope.rotate(k, [t + shift], base))
        assert abs(d0 - d1) < 1e-10 * max(1.0, abs(d0))


def test_worked_case_key_at_50_reused_at_1050(rng):
    g = json.load(open(os.path.join(GOLDEN, "kvboost_rope_correction.json")))
    t, target, delta = g["cached_position"], g["reuse_position"], g["correction"]
    assert t + delta == target
    d, base = 128, 1e6
    layer = fusion.Layer(hidden=8, n_q_heads=2, n_kv_heads=2, head_dim=d, rope_base=base)
    k_raw = rng.standard_normal((t + 1, 2, d))
    # chunk cached at local positions 0..t; keys carry R(local position)
    local = np.arange(t + 1)
    pool_k = _complex_rotate(k_raw, local, rope.inverse_frequencies(d, base))
    pool_v = rng.standard_normal((t + 1, 2, d))
    table = np.array([[0, delta, delta, t + 1, 0, 0, 0, 0]], dtype=np.int32)
    fk, fv = fusion.rerotate_stitch(pool_k, pool_v, table, delta + t + 1, layer)
    want = _complex_rotate(k_raw[t:t + 1], [target], rope.inverse_frequencies(d, base))
    np.testing.assert_allclose(fk[target], want[0], atol=1e-10)
    # values move unchanged, rows before the chunk stay empty
    np.testing.assert_array_equal(fv[delta:], pool_v)
    assert not fk[:delta].any() and not fv[:delta].any()
