"""Pins of the oracle's static and chunk-segmented selectors (CPU only).

Sources: KVBoost page, section 4.1 (attention-sink tokens) and section 4.6.1,
Algorithm 1 (seam windows of R tokens); QCFuse page, section 2.2.1 (EPIC's
boundary tokens per chunk) and section 3.3.1, Eq. 14 (per-chunk anchors
A_i = TopK(G_i, ceil(r_a |c_i|)), Knorm ranking by key norm).

Each selector is checked against something other than itself: hand-worked
fixtures (tests/golden/static_selectors.json), a membership predicate written
per position, brute force over all subsets of tiny inputs, the rotation
invariance a key-norm score must have, and exact rational arithmetic.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import fusion, rope, selectors

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# key norm
# ----------------------------------------------------------------------------
def test_key_norm_loops():
    g = np.random.default_rng(0)
    k = g.standard_normal((5, 3, 4))
    got = selectors.key_norm(k)
    for t in range(5):
        acc = 0.0
        for h in range(3):
            for j in range(4):
                acc += k[t, h, j] * k[t, h, j]
        assert got[t] == pytest.approx(math.sqrt(acc), rel=1e-14)


def test_key_norm_rotation_invariant():
    g = np.random.default_rng(1)
    k = g.standard_normal((7, 2, 16))
    pos = g.integers(-5000, 5000, size=7)
    rotated = rope.rotate(k, pos, 10000.0)
    np.testing.assert_allclose(selectors.key_norm(rotated), selectors.key_norm(k),
                               rtol=1e-12)


def test_key_norm_zero_and_scale():
    assert np.all(selectors.key_norm(np.zeros((3, 2, 8))) == 0.0)
    assert selectors.key_norm(np.zeros((0, 2, 8))).shape == (0,)
    k = np.zeros((1, 2, 4))
    k[0, 0, 0], k[0, 1, 3] = 3.0, 4.0
    assert selectors.key_norm(k)[0] == 5.0
    k2 = np.random.default_rng(2).standard_normal((4, 2, 8))
    np.testing.assert_allclose(selectors.key_norm(-2.5 * k2), 2.5 * selectors.key_norm(k2),
                               rtol=1e-14)


# ----------------------------------------------------------------------------
# anchor budget
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("n,num,den", [(0, 1, 4), (1, 1, 4), (7, 1, 4), (8, 1, 4),
                                       (100, 15, 100), (101, 15, 100), (5, 0, 3),
                                       (5, 3, 3), (1000, 333, 1000)])
def test_anchor_budget_exact(n, num, den):
    assert selectors.anchor_budget(n, num, den) == math.ceil(Fraction(n * num, den))


def test_anchor_budget_rejects():
    for args in [(5, 1, 0), (5, -1, 4), (5, 5, 4), (-1, 1, 4)]:
        with pytest.raises(ValueError):
            selectors.anchor_budget(*args)


# ----------------------------------------------------------------------------
# static mask
# ----------------------------------------------------------------------------
def _fixtures():
    with open(os.path.join(GOLDEN, "static_selectors.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _fixtures(), ids=lambda c: c["name"])
def test_static_mask_golden(case):
    m = selectors.static_mask(case["n_ctx"], case["chunk_starts"], case["sink"],
                              case["boundary"], case["seam"])
    assert m.dtype == np.uint8 and m.shape == (case["n_ctx"],)
    got = np.flatnonzero(m).tolist()
    if "positions" in case:
        assert got == case["positions"]
    else:
        want = [t for lo, hi in case["positions_ranges"] for t in range(lo, hi)]
        assert got == want
        assert len(got) == case["positions_count"]


def _member(t, starts, sink, boundary, seam):
    if t < sink:
        return True
    for p in starts:
        if p <= t < p + boundary:
            return True
        if p > 0 and p - seam <= t < p:
            return True
    return False


@pytest.mark.parametrize("seed", range(16))
def test_static_mask_membership(seed):
    g = np.random.default_rng(100 + seed)
    n = int(g.integers(1, 80))
    m = int(g.integers(1, 6))
    starts = sorted(set([0] + g.integers(0, n, size=m - 1).tolist()))
    sink, boundary, seam = (int(v) for v in g.integers(0, 12, size=3))
    got = selectors.static_mask(n, starts, sink, boundary, seam)
    want = [1 if _member(t, starts, sink, boundary, seam) else 0 for t in range(n)]
    assert got.tolist() == want


def test_static_mask_seam_cost():
    """Seams far apart pick R positions each (cost O(R N_seams))."""
    for r in (1, 8, 16, 32):
        starts = [0, 200, 400, 600, 800]
        m = selectors.static_mask(1000, starts, 0, 0, r)
        assert int(m.sum()) == r * (len(starts) - 1)


def test_static_mask_rejects_unsorted():
    with pytest.raises(ValueError):
        selectors.static_mask(10, [0, 6, 3], 0, 1, 1)
    with pytest.raises(ValueError):
        selectors.static_mask(10, [0, 11], 0, 1, 1)


# ----------------------------------------------------------------------------
# forced top-k
# ----------------------------------------------------------------------------
def _rank_key(i, s, forced):
    if forced[i]:
        return (0, 0, 0.0, i)
    v = float(s[i])
    if math.isnan(v):
        return (1, 1, 0.0, i)
    return (1, 0, -(v + 0.0), i)


def _brute_forced(s, k, forced):
    """Among all k-subsets, the one whose members' keys, sorted, are
    lexicographically smallest."""
    best, best_key = None, None
    for sub in itertools.combinations(range(len(s)), k):
        key = sorted(_rank_key(i, s, forced) for i in sub)
        if best_key is None or key < best_key:
            best, best_key = list(sub), key
    return best


@pytest.mark.parametrize("seed", range(24))
def test_forced_topk_brute_force(seed):
    g = np.random.default_rng(200 + seed)
    n = int(g.integers(1, 11))
    s = g.integers(-2, 3, size=n).astype(np.float32)
    if seed % 3 == 0:
        s[g.integers(0, n)] = np.nan
    if seed % 5 == 1:
        s[s == 0] = -0.0
    forced = (g.random(n) < 0.3).astype(np.uint8)
    k = int(g.integers(0, n + 1))
    got = selectors.select_topk_forced(s, k, forced)
    assert got.dtype == np.int32
    assert got.tolist() == _brute_forced(s, k, forced)


def test_forced_topk_special_cases():
    g = np.random.default_rng(3)
    s = g.standard_normal(40)
    none = np.zeros(40, dtype=np.uint8)
    for k in (0, 1, 17, 40):
        np.testing.assert_array_equal(selectors.select_topk_forced(s, k, none),
                                      fusion.select_topk(s, k))
    allf = np.ones(40, dtype=np.uint8)
    np.testing.assert_array_equal(selectors.select_topk_forced(s, 5, allf), np.arange(5))
    f = np.zeros(40, dtype=np.uint8)
    f[[3, 30]] = 1
    p = selectors.select_topk_forced(s, 40, f)
    np.testing.assert_array_equal(p, np.arange(40))
    p = selectors.select_topk_forced(s, 10, f)
    assert 3 in p and 30 in p and len(p) == 10
    with pytest.raises(ValueError):
        selectors.select_topk_forced(s, 41, f)


# ----------------------------------------------------------------------------
# segmented top-k
# ----------------------------------------------------------------------------
def _brute_topk(s, k):
    def key(i):
        v = float(s[i])
        return (1, 0.0, i) if math.isnan(v) else (0, -(v + 0.0), i)
    return sorted(sorted(range(len(s)), key=key)[:k])


@pytest.mark.parametrize("seed", range(12))
def test_segmented_brute_force(seed):
    g = np.random.default_rng(300 + seed)
    n = int(g.integers(1, 90))
    s = g.integers(-3, 4, size=n).astype(np.float32)
    if seed % 4 == 0:
        s[g.integers(0, n)] = np.nan
    cuts = sorted(set([0, n] + g.integers(0, n, size=int(g.integers(0, 5))).tolist()))
    starts, lens, ks, want = [], [], [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if g.random() < 0.2:           # gaps between segments are allowed
            continue
        kk = int(g.integers(0, b - a + 1))
        starts.append(a)
        lens.append(b - a)
        ks.append(kk)
        want += [a + i for i in _brute_topk(s[a:b], kk)]
    got = selectors.select_topk_segmented(s, starts, lens, ks)
    assert got.dtype == np.int32
    assert got.tolist() == want


def test_segmented_special_cases():
    s = np.ones(12, dtype=np.float32)
    got = selectors.select_topk_segmented(s, [0, 5, 9], [5, 4, 3], [2, 0, 3])
    assert got.tolist() == [0, 1, 9, 10, 11]
    assert selectors.select_topk_segmented(s, [], [], []).size == 0
    with pytest.raises(ValueError):
        selectors.select_topk_segmented(s, [0, 3], [5, 4], [1, 1])      # overlap
    with pytest.raises(ValueError):
        selectors.select_topk_segmented(s, [0], [5], [6])


def test_segmented_anchor_budget_matches_eq14():
    """A_i sizes follow ceil(r_a |c_i|) per chunk, and no chunk takes another
    chunk's budget even when one chunk holds all the large scores."""
    lens = [37, 64, 5, 130]
    starts = np.cumsum([0] + lens[:-1]).tolist()
    s = np.zeros(sum(lens), dtype=np.float64)
    s[starts[1]:starts[1] + lens[1]] = 100.0 + np.arange(lens[1])
    ks = [selectors.anchor_budget(n, 15, 100) for n in lens]
    got = selectors.select_topk_segmented(s, starts, lens, ks)
    for st, ln, kk in zip(starts, lens, ks):
        inside = got[(got >= st) & (got < st + ln)]
        assert inside.size == kk
