"""Pins of the oracle's multi-layer selection signals (CPU only).

QCFuse page, section 3.2.1, Eq. 10 (the score summed over every layer) and
section 3.4.2, Eq. 20 (the sum over a critical layer set); section 2.2.1
(CacheBlend's candidate set narrowed layer by layer).  Checked against the
attention-mass closed form for Q = 0, brute force over tiny inputs, and the
properties nested top-k selections must have.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import fusion, multilayer


def test_layer_sum_closed_form():
    """Q = 0 in every layer: each query row spreads its mass evenly over its
    N + i + 1 visible keys, so I(t) = L * sum_i Hq / (N + i + 1)."""
    g = np.random.default_rng(0)
    N, U, hq, hkv, d, L = 37, 5, 4, 2, 16, 3
    lo = fusion.Layer(64, hq, hkv, d, 1e4)
    per = []
    for l in range(L):
        keys = g.standard_normal((N + U, hkv, d))
        per.append(fusion.attention_mass(np.zeros((U, hq, d)), keys, N, lo))
    want = L * sum(hq / (N + i + 1) for i in range(U))
    np.testing.assert_allclose(multilayer.layer_sum(per), np.full(N, want), rtol=1e-12)
    # a critical subset: two of the three layers
    np.testing.assert_allclose(multilayer.layer_sum(per, [2, 0]), np.full(N, want * 2 / 3),
                               rtol=1e-12)


def test_layer_sum_basic():
    g = np.random.default_rng(1)
    per = [g.random(20) for _ in range(4)]
    np.testing.assert_array_equal(multilayer.layer_sum(per, [1]), per[1])
    np.testing.assert_allclose(multilayer.layer_sum(per, [3, 1, 2]),
                               multilayer.layer_sum(per, [1, 2, 3]), rtol=1e-15)
    with pytest.raises(ValueError):
        multilayer.layer_sum(per, [])


def test_restrict():
    s = np.arange(5.0)
    np.testing.assert_array_equal(multilayer.restrict(s, np.ones(5)), s)
    assert np.isnan(multilayer.restrict(s, np.zeros(5))).all()
    r = multilayer.restrict(s, np.array([1, 0, 1, 0, 0]))
    assert r[0] == 0.0 and r[2] == 2.0 and np.isnan(r[[1, 3, 4]]).all()


def _brute_progressive(per, ks):
    """Exhaustive: at every layer, the k-subset of the candidates whose scores
    (descending, ties to the lower position) rank best."""
    n = len(per[0])
    cand = list(range(n))
    out = []
    for s, k in zip(per, ks):
        best, best_key = None, None
        for sub in itertools.combinations(cand, k):
            key = sorted((-(float(s[i]) + 0.0), i) for i in sub)
            if best_key is None or key < best_key:
                best, best_key = list(sub), key
        out.append(best)
        cand = best
    return out


@pytest.mark.parametrize("seed", range(10))
def test_progressive_brute_force(seed):
    g = np.random.default_rng(10 + seed)
    n = int(g.integers(1, 10))
    L = int(g.integers(1, 4))
    per = [g.integers(-2, 3, size=n).astype(np.float32) for _ in range(L)]
    ks = sorted((int(v) for v in g.integers(0, n + 1, size=L)), reverse=True)
    got = multilayer.progressive_select(per, ks)
    assert [c.tolist() for c in got] == _brute_progressive(per, ks)


def test_progressive_properties():
    g = np.random.default_rng(3)
    n = 500
    per = [g.standard_normal(n).astype(np.float32) for _ in range(4)]
    ks = [400, 250, 250, 100]
    sels = multilayer.progressive_select(per, ks)
    for a, b in zip(sels[:-1], sels[1:]):
        assert np.isin(b, a).all()                      # nested
    assert [len(c) for c in sels] == ks
    # the same scores in every layer: nested top-k is the top-k of the last budget
    same = multilayer.progressive_select([per[0]] * 3, [300, 200, 50])
    np.testing.assert_array_equal(same[-1], fusion.select_topk(per[0], 50))
    # no filtering before the last layer: that layer's own top-k
    free = multilayer.progressive_select(per, [n, n, n, 77])
    np.testing.assert_array_equal(free[-1], fusion.select_topk(per[3], 77))
    with pytest.raises(ValueError):
        multilayer.progressive_select(per[:2], [10, 20])   # budget grows
    with pytest.raises(ValueError):
        multilayer.progressive_select(per[:2], [10])


def test_progressive_candidates_exclude_even_better_scores():
    """A position dropped at layer 1 stays out even if its later score is the
    largest: the filter only narrows."""
    s1 = np.array([5, 4, 3, 2, 1], dtype=np.float32)
    s2 = np.array([0, 0, 0, 0, 9], dtype=np.float32)
    c1, c2 = multilayer.progressive_select([s1, s2], [3, 2])
    assert c1.tolist() == [0, 1, 2] and c2.tolist() == [0, 1]
    assert math.isnan(multilayer.restrict(s2, np.isin(np.arange(5), c1))[4])
