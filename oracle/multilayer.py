"""Selection signals that span several layers.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every layer of the fused path computes the same per-layer scores as the
one-layer path (deviation or query-to-context attention mass); the pages use
them across layers in two ways:

  * Summing over layers.  The full-view importance of QCFuse section 3.2.1,
    Eq. 10 (a ProphetKV-style selector) is I(t) = sum over all layers l of
    Attn_l(t); QCFuse's critical-layer view, section 3.4.2, Eq. 20, is the
    same sum over a small layer set L_k.  P = TopK(I, floor(rho N)), Eq. 11.
  * Layer-by-layer filtering.  CacheBlend, as QCFuse section 2.2.1 describes
    it, recomputes a broad candidate set in early layers and keeps, layer by
    layer, the tokens with the largest KV deviation.  Read plainly: the
    candidate set C_0 is every context position, and at layer l the
    selection C_l = TopK over C_{l-1} of that layer's deviation, with
    |C_l| = k_l non-increasing; the last C_l is the layer's P.

Readings (listed with the design notes): scores outside the candidate set
are NaN, which the top-k order ranks below every number, so k_l <= |C_{l-1}|
keeps C_l inside C_{l-1}; the per-layer selections take their decisions on
fp32 scores, like the one-layer selection.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .fusion import select_topk


def layer_sum(per_layer: Sequence[np.ndarray], layers: Optional[Sequence[int]] = None) -> np.ndarray:
    """I(t) = sum over l in `layers` (all by default) of per_layer[l](t),
    float64 ([QCF] Eq. 10; Eq. 20 with layers = L_k).

    Pin: one layer gives that layer's score; Q = 0 in every layer gives the
    closed form sum_l sum_i Hq / (N + i + 1) at every position; the sum is
    the same for any order of the layer list."""
    idx = range(len(per_layer)) if layers is None else layers
    idx = list(idx)
    if not idx:
        raise ValueError("empty layer set")
    out = np.zeros_like(np.asarray(per_layer[idx[0]], dtype=np.float64))
    for l in idx:
        out = out + np.asarray(per_layer[l], dtype=np.float64)
    return out


def restrict(scores: np.ndarray, candidates: np.ndarray) -> np.ndarray:
    """The scores on the candidate set (boolean / 0-1 mask), NaN elsewhere.

    Pin: candidates everywhere returns the scores; none returns all NaN."""
    s = np.asarray(scores, dtype=np.float64).copy()
    s[~np.asarray(candidates).astype(bool)] = np.nan
    return s


def progressive_select(per_layer: Sequence[np.ndarray], ks: Sequence[int]) -> list:
    """C_l = TopK(restrict(per_layer[l], C_{l-1}), ks[l]) with C_0 = every
    position; returns [C_1, C_2, ...] (ascending int32 position arrays).

    Pin: C_l is inside C_{l-1}; every layer given the same scores gives
    TopK(scores, k_last); ks[l] = N for every layer but the last gives the
    last layer's own TopK; brute force over tiny inputs."""
    if len(per_layer) != len(ks) or not ks:
        raise ValueError("one budget per layer")
    n = np.asarray(per_layer[0]).shape[0]
    cand = np.ones(n, dtype=bool)
    out = []
    for l, k in enumerate(ks):
        if not 0 <= k <= int(cand.sum()):
            raise ValueError("budgets must not exceed the previous layer's picks")
        s = restrict(per_layer[l], cand).astype(np.float32)
        sel = select_topk(s, int(k))
        cand = np.zeros(n, dtype=bool)
        cand[sel] = True
        out.append(sel)
    return out
