"""Int8-resident fused cache, float64 (test infrastructure).

[KVB] section 4.5, Eq. 7 with b = 8 bits, applied to the fused cache itself:
instead of expanding the cached entries to bf16 when they are re-positioned,
every fused row keeps 8-bit codes, and readers (the scores, the attention)
decode them.  [KVB] section 7.3 (memory budget) is the reason: an 8-bit
cache takes half the bytes of a 16-bit one.

Format: for every fused row t and kv head h, K[t, h, :] and V[t, h, :] are
each d codes with one float32 (min, scale) pair, value = min + code * scale,
the pair stored as stats[t, h] = (min, scale).

Readings of points the pages leave open (also listed with the design notes
of the repository):
  * Grouping.  Eq. 7 takes key statistics per channel over a group of tokens
    and value statistics per token.  A fused row is written on its own - by
    re-positioning (S1) or by fusion (S5, [QCF] 2.1.3 Eq. 7) - so its
    statistics may depend on that row only: keys are grouped per (token,
    head) here, like the values.
  * Encoding arithmetic is that of the KIVI encoder (oracle.kivi): float32,
    range = max - min, scale = range / 255, inv = 255 / range,
    code = round_half_even((x - min) * inv) clamped to [0, 255]; a constant
    group has scale 0 and codes 0.
  * Re-positioned keys: the per-chunk key is decoded exactly, rotated by the
    delta rotation R(pos0) exactly ([KVB] 3.2 Eq. 3), rounded to float32 and
    encoded.
  * Re-positioned values of an 8-bit KIVI per-chunk cache are per-token 8-bit
    groups already: codes and statistics are copied unchanged.  Values of a
    dense per-chunk cache are encoded from their float32 value.
  * Recomputed rows enter the cache as the encoding of their float32 value
    (the serving precision rounds them to bf16 first, as every projection
    output).
  * Rows no chunk covers hold codes 0 and statistics (0, 0), i.e. zeros, as
    the dense fused cache leaves them.

Pins (tests/test_oracle_q8cache.py): the codes lie in [0, 255]; the row
minimum decodes exactly and the maximum maps to 255; every code is the
nearest level (brute force over the neighbouring levels) and codes are
monotone in the value; constant rows decode exactly; values copied from a
KIVI cache are bit-identical; re-positioned keys lie within half a step of
the exact re-positioned key; fusion rewrites exactly the given rows; at
rho = 100% the layer's attention equals attention over the encoded
full-prefill cache, computed without the fusion path.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

from . import fusion, kivi, storage


@dataclasses.dataclass
class Cache:
    """codes [rows, Hkv, d] uint8; stats [rows, Hkv, 2] float32 (min, scale)."""
    k_codes: np.ndarray
    k_stats: np.ndarray
    v_codes: np.ndarray
    v_stats: np.ndarray

    def copy(self) -> "Cache":
        return Cache(self.k_codes.copy(), self.k_stats.copy(), self.v_codes.copy(),
                     self.v_stats.copy())


def encode(x: np.ndarray) -> tuple:
    """x [rows, Hkv, d] (rounded to float32) -> (codes, stats): one 8-bit
    group per (row, head) over its d channels ([KVB] 4.5 Eq. 7, b = 8)."""
    code, mn, sc = kivi._encode_groups(np.asarray(x, dtype=np.float32), axis=2, bits=8)
    stats = np.stack([mn[..., 0], sc[..., 0]], axis=-1).astype(np.float32)
    return code, stats


def decode(codes: np.ndarray, stats: np.ndarray) -> np.ndarray:
    """min + code * scale, float64."""
    st = np.asarray(stats, dtype=np.float64)
    return st[..., 0:1] + np.asarray(codes, dtype=np.float64) * st[..., 1:2]


def decode_k(c: Cache) -> np.ndarray:
    return decode(c.k_codes, c.k_stats)


def decode_v(c: Cache) -> np.ndarray:
    return decode(c.v_codes, c.v_stats)


def empty(rows: int, hkv: int, d: int) -> Cache:
    z8 = np.zeros((rows, hkv, d), dtype=np.uint8)
    zs = np.zeros((rows, hkv, 2), dtype=np.float32)
    return Cache(z8, zs, z8.copy(), zs.copy())


def stitch(chunk_table: np.ndarray, total_rows: int, layer: fusion.Layer,
           pool_k: Optional[np.ndarray] = None, pool_v: Optional[np.ndarray] = None,
           pool_q8: Optional[dict] = None, pool_cu: Optional[np.ndarray] = None) -> Cache:
    """S1 into an int8-resident fused cache ([QCF] 2.1.2 Eq. 4; [KVB] 3.2
    Eq. 3 and 4.5 Eq. 7).

    Per-chunk cache either dense (pool_k, pool_v: float values) or 8-bit KIVI
    (pool_q8: the kivi module's k_codes, k_min, k_scale, v_codes, v_min,
    v_scale, with pool_cu the per-chunk row ranges of the key statistics).
    """
    hkv, d = layer.n_kv_heads, layer.head_dim
    out = empty(total_rows, hkv, d)
    if pool_q8 is not None:
        pk = kivi.decode_keys(pool_q8["k_codes"], pool_q8["k_min"], pool_q8["k_scale"], pool_cu)
    else:
        pk = np.asarray(pool_k, dtype=np.float64)
    # the exact re-positioned keys (and the dense values, unchanged)
    pv_dense = np.zeros_like(pk) if pool_q8 is not None else np.asarray(pool_v, dtype=np.float64)
    fk, fv = fusion.rerotate_stitch(pk, pv_dense, chunk_table, total_rows, layer)
    covered = np.zeros(total_rows, dtype=bool)
    for src, dst, _, n in np.asarray(chunk_table)[:, :4]:
        src, dst, n = int(src), int(dst), int(n)
        covered[dst:dst + n] = True
        if pool_q8 is not None:
            out.v_codes[dst:dst + n] = pool_q8["v_codes"][src:src + n]
            out.v_stats[dst:dst + n, :, 0] = pool_q8["v_min"][src:src + n]
            out.v_stats[dst:dst + n, :, 1] = pool_q8["v_scale"][src:src + n]
    rows = np.nonzero(covered)[0]
    out.k_codes[rows], out.k_stats[rows] = encode(fk[rows])
    if pool_q8 is None:
        out.v_codes[rows], out.v_stats[rows] = encode(fv[rows])
    return out


def fuse(cache: Cache, rows: np.ndarray, k_new: Optional[np.ndarray],
         v_new: Optional[np.ndarray]) -> Cache:
    """KV^Fuse_p = KV^New_p for the given rows ([QCF] 2.1.3 Eq. 7), each new
    row encoded on its own; every other row is unchanged.  Returns a copy."""
    rows = np.asarray(rows, dtype=np.int64)
    if len(np.unique(rows)) != len(rows):
        raise ValueError("destination rows must be unique")
    out = cache.copy()
    if k_new is not None:
        out.k_codes[rows], out.k_stats[rows] = encode(k_new)
    if v_new is not None:
        out.v_codes[rows], out.v_stats[rows] = encode(v_new)
    return out


def fused_layer(x: np.ndarray, w_qkv: np.ndarray, chunk_table: np.ndarray,
                cu_T: Sequence[int], n_ctx: Sequence[int], layer: fusion.Layer,
                k_per_req: Sequence[int], pool_k=None, pool_v=None, pool_q8=None,
                pool_cu=None, forced_sel=None, store: Optional[str] = "bf16",
                attend=None) -> dict:
    """One fused layer with deviation scoring ([KVB] 4.6.2 Algorithm 2 at one
    layer) over an int8-resident fused cache: the steps of
    oracle.fusion.fused_layer in mode "deviation", with the fused cache held
    in the format above.  Scores read the decoded keys; the recomputed rows
    take K from the probe and V from the projection, both at the serving
    precision `store`, and are encoded into the cache; attention reads the
    decoded cache.  `forced_sel` and `attend` as in oracle.fusion.fused_layer.
    """
    def S(a):
        return a if store is None else storage.decode(storage.encode(a, store), store)

    x = np.asarray(x, dtype=np.float64)
    cu_T = [int(v) for v in cu_T]
    n_req = len(cu_T) - 1
    total = cu_T[-1]
    cache = stitch(chunk_table, total, layer, pool_k, pool_v, pool_q8, pool_cu)
    res = {"cache_pic": cache.copy()}
    allpos = np.concatenate([np.arange(cu_T[r + 1] - cu_T[r]) for r in range(n_req)])
    k_probe = S(fusion.recompute(x, allpos, w_qkv, layer, want=("k",))["k"])
    res["k_probe"] = k_probe
    fk = decode_k(cache)
    scores, sels, rows_all, pos_all = [], [], [], []
    for r in range(n_req):
        a, b, N = cu_T[r], cu_T[r + 1], int(n_ctx[r])
        s = fusion.deviation(fk[a:a + N], k_probe[a:a + N])
        scores.append(s)
        if forced_sel is not None:
            sel = np.asarray(forced_sel[r], dtype=np.int32)
        else:
            sel = fusion.select_topk(s.astype(np.float32), int(k_per_req[r]))
        sels.append(sel)
        pos_all.append(np.concatenate([sel, np.arange(N, b - a)]).astype(np.int32))
        rows_all.append((a + pos_all[-1]).astype(np.int32))
    rows = np.concatenate(rows_all)
    pos = np.concatenate(pos_all)
    sizes = [len(p) for p in pos_all]
    starts = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    if attend is None:
        flat = np.arange(len(rows), dtype=np.int64)
    else:
        flat = np.concatenate([starts[r] + np.asarray(attend[r], dtype=np.int64)
                               for r in range(n_req)])
    v_new = S(fusion.recompute(x[rows], pos, w_qkv, layer, want=("v",))["v"])
    k_new = k_probe[rows]
    q = S(fusion.recompute(x[rows[flat]], pos[flat], w_qkv, layer, want=("q",))["q"])
    cache = fuse(cache, rows, k_new, v_new)
    fk, fv = decode_k(cache), decode_v(cache)
    outs, lses = [], []
    qoff = 0
    for r in range(n_req):
        a, b = cu_T[r], cu_T[r + 1]
        idx = np.arange(sizes[r]) if attend is None else np.asarray(attend[r], dtype=np.int64)
        o, l = fusion.causal_attention(q[qoff:qoff + len(idx)], pos_all[r][idx], fk[a:b], fv[a:b],
                                       layer)
        outs.append(o)
        lses.append(l)
        qoff += len(idx)
    res.update(scores=scores, sel=sels, rows=rows, pos=pos, cu_q=starts, attend_flat=flat,
               q=q, k_new=k_new, v_new=v_new, cache=cache,
               out=np.concatenate(outs), lse=np.concatenate(lses))
    return res
