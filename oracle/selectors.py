"""Static and chunk-segmented selectors that feed the same recompute path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The fused-layer path takes its recompute set P from a selector.  Besides the
scored selectors of S2/S3 (deviation, attention mass), the pages describe
index producers that need no query-time scoring, and one chunk-local ranking
used to build compact anchor views:

  * EPIC's LegoLink rule ([QCF] 2.2.1): a fixed number of boundary tokens
    at the start of every stitched chunk is recomputed.
  * KVBoost's SelectiveRecompute ([KVB] 4.6.1, Algorithm 1): for every seam
    (the start p of a chunk other than the first) the positions
    [max(0, p - R), p) are re-encoded with full preceding context.
  * KVBoost's attention-sink injection ([KVB] 4.1): the first s tokens of
    the prompt are always in the live token set.
  * QCFuse's anchor construction ([QCF] 3.3.1, Eq. 14): per reusable chunk
    c_i, A_i = TopK(G_i, ceil(r_a |c_i|)) under a chunk-local ranking G_i,
    e.g. the Knorm rule that ranks positions by the norm of their cached
    keys.

Readings of points the pages leave open (also listed with the design
notes):
  * Knorm's score is the L2 norm of the token's key over all KV heads and
    channels of the layer; it is rotation invariant, so the per-chunk cache
    and the re-positioned fused cache give the same score.  The direction of
    the ranking is not given; the score is returned as is and the caller
    ranks it (TopK takes the largest), negating it for "smallest norm first".
  * Static picks count against the budget k: TopK with a forced set takes
    every forced position first (the lowest positions if there are more than
    k of them) and fills the rest of the k positions by score.
  * Positions are request-relative context positions 0..N-1; the query
    suffix is never part of these sets (it is always recomputed).
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .fusion import select_topk


def key_norm(keys: np.ndarray) -> np.ndarray:
    """Knorm score per token ([QCF] 3.3.1): sqrt(sum_{h, j} K[t, h, j]^2) over
    a [tokens, Hkv, d] key cache, float64.

    Pin: explicit loops on tiny inputs, invariance under any RoPE rotation of
    the keys, zero keys give zero."""
    k = np.asarray(keys, dtype=np.float64)
    flat = k.reshape(k.shape[0], int(np.prod(k.shape[1:], dtype=np.int64)))
    return np.sqrt(np.sum(flat * flat, axis=1))


def anchor_budget(chunk_len: int, ra_num: int, ra_den: int) -> int:
    """ceil(r_a |c_i|) of [QCF] 3.3.1 Eq. 14 with r_a = ra_num / ra_den, in
    integers (no rounding of r_a |c_i| in floating point)."""
    if ra_den <= 0 or ra_num < 0 or ra_num > ra_den or chunk_len < 0:
        raise ValueError("bad anchor ratio or length")
    return -((-int(chunk_len) * int(ra_num)) // int(ra_den))


def static_mask(n_ctx: int, chunk_starts: Sequence[int], sink: int, boundary: int,
                seam: int) -> np.ndarray:
    """uint8 mask over the N context positions of one request: 1 where a
    static rule picks the position.

    chunk_starts: request positions where the stitched chunks begin (the
    first is 0), ascending.  sink ([KVB] 4.1): positions 0..sink-1.
    boundary ([QCF] 2.2.1, EPIC): the first `boundary` positions of every
    chunk.  seam ([KVB] 4.6.1, Algorithm 1 with R = seam): for every chunk
    start p > 0, positions max(0, p - R) .. p - 1.  Every range is clipped to
    [0, N).

    Pin: hand-worked fixtures (tests/golden/static_selectors.json), the
    count 2 R for two seams far from each other and from the start
    ([KVB] 4.6.1's cost O(R N_seams)), and the zero rule giving an empty set."""
    n = int(n_ctx)
    mask = np.zeros(n, dtype=np.uint8)

    def put(lo: int, hi: int) -> None:
        lo, hi = max(0, lo), min(n, hi)
        if lo < hi:
            mask[lo:hi] = 1

    put(0, sink)
    starts = list(chunk_starts)
    for i, p in enumerate(starts):
        if not 0 <= p <= n or (i and p < starts[i - 1]):
            raise ValueError("chunk starts must be ascending inside [0, N]")
        put(p, p + boundary)
        if p > 0:
            put(p - seam, p)
    return mask


def select_topk_forced(scores: np.ndarray, k: int, forced: np.ndarray) -> np.ndarray:
    """P = forced positions first, then TopK of the rest by score, |P| = k.

    With f = number of forced positions: f >= k keeps the k lowest forced
    positions; otherwise P = forced + TopK(scores restricted to the others,
    k - f) with select_topk's order (larger first, ties to the lower
    position, -0 == +0, NaN last).  Returned ascending (int32).

    Pin: brute force over all k-subsets on tiny inputs (the chosen set is the
    lexicographically best by (forced, score, -position) ranking), no forced
    positions reduce to select_topk, k = N selects everything."""
    s = np.asarray(scores)
    f = np.asarray(forced).astype(bool)
    n = s.shape[0]
    if not 0 <= k <= n or f.shape[0] != n:
        raise ValueError("k or mask size out of range")
    fpos = np.flatnonzero(f)
    if fpos.size >= k:
        return np.sort(fpos[:k]).astype(np.int32)
    rest = np.flatnonzero(~f)
    picked = rest[select_topk(s[rest], k - fpos.size)]
    return np.sort(np.concatenate([fpos, picked])).astype(np.int32)


def select_topk_segmented(scores: np.ndarray, seg_starts: Sequence[int],
                          seg_lens: Sequence[int], seg_k: Sequence[int]) -> np.ndarray:
    """Concatenation over segments (ascending, non-overlapping) of
    seg_start + TopK(scores[seg], k_seg): the per-chunk selection A_i of
    [QCF] 3.3.1 Eq. 14, applied so that no chunk can take another chunk's
    budget.  Positions are relative to the start of `scores`; ascending.

    Pin: per segment it is select_topk itself (checked segment by segment),
    segments of equal scores take their first k_seg positions, and
    k_seg = |segment| selects everything."""
    out = []
    prev_end = 0
    for st, ln, kk in zip(seg_starts, seg_lens, seg_k):
        if st < prev_end or ln < 0 or not 0 <= kk <= ln:
            raise ValueError("segments must be ascending and disjoint, 0 <= k <= len")
        out.append(int(st) + select_topk(np.asarray(scores)[st:st + ln], int(kk)))
        prev_end = st + ln
    if not out:
        return np.zeros(0, dtype=np.int32)
    return np.concatenate(out).astype(np.int32)
