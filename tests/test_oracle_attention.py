"""Pins of the oracle's projection and causal attention (CPU only).

KVBoost page, section 3.1, Eq. 1-2: k = W_K x, v = W_V x; attention of the
query at t over positions <= t with softmax(q K^T / sqrt(d)) V.  Checked
against explicit loops on tiny inputs, a single visible key, zero queries
(uniform average) and the grouped-query head mapping.
"""
import math

import numpy as np
import pytest

from oracle import fusion, rope


def _attn_brute(q, pos, K, V, G):
    M, Hq, d = len(q), len(q[0]), len(q[0][0])
    out = np.zeros((M, Hq, d))
    for r in range(M):
        for h in range(Hq):
            s = [sum(q[r][h][c] * K[j][h // G][c] for c in range(d)) / math.sqrt(d)
                 for j in range(pos[r] + 1)]
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            z = sum(e)
            for j in range(pos[r] + 1):
                for c in range(d):
                    out[r, h, c] += e[j] / z * V[j][h // G][c]
    return out


@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 2), (3, 3)])
def test_attention_matches_brute_force(rng, Hq, Hkv):
    T, d = 9, 4
    layer = fusion.Layer(hidden=8, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, rope_base=1e4)
    K = rng.standard_normal((T, Hkv, d))
    V = rng.standard_normal((T, Hkv, d))
    pos = np.array([0, 2, 3, 7, 8])
    q = rng.standard_normal((len(pos), Hq, d))
    o, lse = fusion.causal_attention(q, pos, K, V, layer)
    np.testing.assert_allclose(o, _attn_brute(q.tolist(), pos.tolist(), K.tolist(), V.tolist(), Hq // Hkv),
                               rtol=1e-12, atol=1e-13)
    # lse = log sum_j exp(s_j)
    r, h = 3, Hq - 1
    s = K[: pos[r] + 1, h // (Hq // Hkv)] @ q[r, h] / math.sqrt(d)
    assert abs(lse[r, h] - math.log(np.exp(s).sum())) < 1e-12


def test_attention_special_cases(rng):
    T, Hq, Hkv, d = 30, 4, 2, 8
    layer = fusion.Layer(hidden=8, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, rope_base=1e4)
    K = rng.standard_normal((T, Hkv, d))
    V = rng.standard_normal((T, Hkv, d))
    # only key 0 visible -> O = V[0]
    o, lse = fusion.causal_attention(rng.standard_normal((1, Hq, d)), [0], K, V, layer)
    for h in range(Hq):
        np.testing.assert_allclose(o[0, h], V[0, h // 2], atol=1e-15)
    # zero query -> mean of the visible values, lse = log(count)
    pos = np.array([4, 17, 29])
    o, lse = fusion.causal_attention(np.zeros((3, Hq, d)), pos, K, V, layer)
    for r, p in enumerate(pos):
        for h in range(Hq):
            np.testing.assert_allclose(o[r, h], V[: p + 1, h // 2].mean(axis=0), atol=1e-14)
            assert abs(lse[r, h] - math.log(p + 1)) < 1e-13


def test_projection_matches_loops_and_is_linear(rng):
    hidden, Hq, Hkv, d = 6, 2, 1, 4
    layer = fusion.Layer(hidden=hidden, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, rope_base=1e4)
    w = rng.standard_normal(((Hq + 2 * Hkv) * d, hidden))
    x = rng.standard_normal((3, hidden))
    pos = np.array([0, 5, 11])
    r = fusion.recompute(x, pos, w, layer)
    # V rows = W_v x by loops; K = R(pos) W_k x by loops
    for n in range(3):
        for c in range(d):
            want_v = sum(w[(Hq + Hkv) * d + c, i] * x[n, i] for i in range(hidden))
            assert abs(r["v"][n, 0, c] - want_v) < 1e-12
    raw_k = np.array([[[sum(w[Hq * d + c, i] * x[n, i] for i in range(hidden)) for c in range(d)]] for n in range(3)])
    np.testing.assert_allclose(r["k"], rope.rotate(raw_k, pos, 1e4), atol=1e-12)
    # linearity in x
    x2 = rng.standard_normal((3, hidden))
    a = fusion.recompute(2 * x - x2, pos, w, layer)
    b, c = fusion.recompute(x, pos, w, layer), fusion.recompute(x2, pos, w, layer)
    for key in ("q", "k", "v"):
        np.testing.assert_allclose(a[key], 2 * b[key] - c[key], atol=1e-12)


def test_fuse_replaces_only_selected_rows(rng):
    fk = rng.standard_normal((10, 2, 4))
    fv = rng.standard_normal((10, 2, 4))
    rows = np.array([1, 4, 9])
    kn, vn = rng.standard_normal((3, 2, 4)), rng.standard_normal((3, 2, 4))
    k2, v2 = fusion.fuse(fk, fv, rows, kn, vn)
    keep = np.setdiff1d(np.arange(10), rows)
    np.testing.assert_array_equal(k2[keep], fk[keep])
    np.testing.assert_array_equal(v2[keep], fv[keep])
    np.testing.assert_array_equal(k2[rows], kn)
    np.testing.assert_array_equal(v2[rows], vn)
    with pytest.raises(ValueError):
        fusion.fuse(fk, fv, np.array([1, 1]), kn[:2], vn[:2])
