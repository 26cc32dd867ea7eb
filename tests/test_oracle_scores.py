"""Pins of the oracle's two token scores (CPU only).

Deviation (KVBoost page, section 4.6.2, Algorithm 2): hand-computed
2-vector cases, zero when cached equals fresh, range [0, 2], invariance under
a common rotation.  Attention mass (QCFuse page, section 3.2.1, Eq. 9-10):
brute force with explicit loops, the closed form for zero queries, the
row-sum invariant and a dominant-key case.
"""
import math

import numpy as np
import pytest

from oracle import fusion, rope


def test_deviation_hand_cases():
    e0 = np.array([1.0, 0.0])
    e1 = np.array([0.0, 1.0])
    k = np.array([[e0], [e0], [e0], [e0], [e0]])          # [5 tokens, 1 head, 2]
    kt = np.array([[e0], [e1], [-e0], [2 * e0], [np.zeros(2)]])
    np.testing.assert_allclose(fusion.deviation(k, kt), [0.0, 1.0, 2.0, 0.0, 1.0], atol=1e-15)
    # two heads: one identical, one orthogonal -> 1 - (1 + 0)/2
    k2 = np.array([[e0, e0]])
    kt2 = np.array([[e0, e1]])
    np.testing.assert_allclose(fusion.deviation(k2, kt2), [0.5], atol=1e-15)
    # 45 degrees: 1 - cos(pi/4)
    kt3 = np.array([[[1.0, 1.0]]])
    np.testing.assert_allclose(fusion.deviation(k[:1], kt3), [1 - math.sqrt(0.5)], atol=1e-15)


def test_deviation_invariants(rng):
    a = rng.standard_normal((200, 8, 128))
    b = a + 0.3 * rng.standard_normal(a.shape)
    np.testing.assert_allclose(fusion.deviation(a, a), 0.0, atol=1e-14)
    d = fusion.deviation(a, b)
    assert np.all(d >= 0) and np.all(d <= 2)
    # cos(R a, R b) = cos(a, b): pre- and post-RoPE deviation agree
    pos = rng.integers(0, 30000, size=200)
    np.testing.assert_allclose(fusion.deviation(rope.rotate(a, pos, 1e6), rope.rotate(b, pos, 1e6)), d, atol=1e-12)
    np.testing.assert_allclose(fusion.deviation(a, -a), 2.0, atol=1e-14)


def _mass_brute(q_u, keys, N, Hq, Hkv, sm, n_last):
    U = len(q_u)
    G = Hq // Hkv
    score = [0.0] * N
    query_mass = 0.0
    for i in range(U - n_last, U):
        for h in range(Hq):
            s = []
            for j in range(N + i + 1):
                s.append(sum(q_u[i][h][c] * keys[j][h // G][c] for c in range(len(q_u[i][h]))) * sm)
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            z = sum(e)
            for j in range(N + i + 1):
                if j < N:
                    score[j] += e[j] / z
                else:
                    query_mass += e[j] / z
    return np.array(score), query_mass


@pytest.mark.parametrize("Hq,Hkv,n_last", [(2, 1, 3), (4, 2, 2), (2, 2, 1)])
def test_mass_matches_brute_force(rng, Hq, Hkv, n_last):
    N, U, d = 6, 3, 4
    layer = fusion.Layer(hidden=8, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, rope_base=1e4)
    q_u = rng.standard_normal((U, Hq, d))
    keys = rng.standard_normal((N + U, Hkv, d))
    got = fusion.attention_mass(q_u, keys, N, layer, n_last_q=n_last)
    want, qmass = _mass_brute(q_u.tolist(), keys.tolist(), N, Hq, Hkv, 1 / math.sqrt(d), n_last)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)
    # every (row, head) softmax sums to one
    assert abs(got.sum() + qmass - n_last * Hq) < 1e-12


def test_mass_closed_form_zero_queries(rng):
    # Q = 0 -> uniform softmax over the N + i + 1 visible keys of row i.
    N, U, Hq, Hkv, d = 50, 7, 8, 2, 16
    layer = fusion.Layer(hidden=8, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, rope_base=1e4)
    keys = rng.standard_normal((N + U, Hkv, d))
    got = fusion.attention_mass(np.zeros((U, Hq, d)), keys, N, layer)
    want = sum(Hq / (N + i + 1) for i in range(U))
    np.testing.assert_allclose(got, want, rtol=1e-13)
    got2 = fusion.attention_mass(np.zeros((U, Hq, d)), keys, N, layer, n_last_q=2)
    np.testing.assert_allclose(got2, sum(Hq / (N + i + 1) for i in range(U - 2, U)), rtol=1e-13)


def test_mass_dominant_key(rng):
    # One context key aligned with every query and far larger than the rest
    # takes (almost) all the mass.
    N, U, Hq, Hkv, d = 20, 4, 4, 1, 8
    layer = fusion.Layer(hidden=8, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, rope_base=1e4)
    keys = 0.01 * rng.standard_normal((N + U, Hkv, d))
    keys[13, 0, :] = 100.0
    q_u = np.ones((U, Hq, d))
    got = fusion.attention_mass(q_u, keys, N, layer)
    assert abs(got[13] - U * Hq) < 1e-9
    assert got.argmax() == 13
