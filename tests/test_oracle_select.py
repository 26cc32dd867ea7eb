"""Pins of the oracle's top-k selection and budget (CPU only).

QCFuse page, section 3.2.1, Eq. 11: P = TopK(I(t), floor(rho N)).
The order rule for ties, signed zeros and NaN is this repository's reading
(the pages are silent): larger first, lower position first on ties, -0 == +0,
NaN last, output ascending.  Checked against a brute-force sort written with
Python's own `sorted` and against the budgets printed in the golden fixture.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import fusion

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute(scores, k):
    def key(i):
        v = float(scores[i])
        if math.isnan(v):
            return (1, 0.0, i)
        return (0, -(v + 0.0), i)
    return sorted(sorted(range(len(scores)), key=key)[:k])


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force(seed):
    g = np.random.default_rng(seed)
    n = int(g.integers(1, 60))
    s = g.integers(-3, 4, size=n).astype(np.float32)        # many ties
    if seed % 3 == 0:
        s[g.integers(0, n)] = np.nan
    if seed % 4 == 1:
        s[s == 0] = -0.0
    k = int(g.integers(0, n + 1))
    got = fusion.select_topk(s, k)
    assert got.tolist() == _brute(s, k)


def test_topk_invariants(rng):
    s = rng.standard_normal(5000).astype(np.float32)
    for k in (0, 1, 1234, 4999, 5000):
        p = fusion.select_topk(s, k)
        assert len(p) == k and len(set(p.tolist())) == k
        assert np.all(np.diff(p) > 0)
        if 0 < k < 5000:
            rest = np.setdiff1d(np.arange(5000), p)
            assert s[p].min() >= s[rest].max()


def test_topk_ties_take_lower_positions():
    s = np.array([1.0, 2.0, 2.0, 2.0, 0.5, 2.0], dtype=np.float32)
    assert fusion.select_topk(s, 2).tolist() == [1, 2]
    assert fusion.select_topk(s, 4).tolist() == [1, 2, 3, 5]
    z = np.array([0.0, -0.0, 0.0, -0.0], dtype=np.float32)
    assert fusion.select_topk(z, 2).tolist() == [0, 1]
    n = np.array([np.nan, -1e30, np.nan, -np.inf], dtype=np.float32)
    assert fusion.select_topk(n, 2).tolist() == [1, 3]
    assert fusion.select_topk(n, 3).tolist() == [0, 1, 3]


def test_topk_rejects_bad_k():
    with pytest.raises(ValueError):
        fusion.select_topk(np.zeros(3, np.float32), 4)


def test_budgets_match_fixture():
    g = json.load(open(os.path.join(GOLDEN, "budgets.json")))
    for c in g["cases"]:
        assert fusion.budget(c["n_ctx"], c["ratio_pct"]) == c["k"], c
        # agrees with floor(rho N) evaluated exactly in rationals
        assert c["k"] == (c["n_ctx"] * c["ratio_pct"]) // 100
