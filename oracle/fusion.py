"""One layer of RAG KV-cache fusion with selective recomputation, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation follows Table 1 of the QCFuse page: a request holds context
C = [c_1; ...; c_m] with N tokens followed by U query tokens (T = N + U);
P is the set of recomputed context positions; KV^PIC the per-chunk caches
built in isolation, KV^New the recomputed entries and KV^Fuse the fused
cache.

Tensor conventions (shared with the library only by documentation):
  x       [sum T, hidden]          fresh hidden state of every request row
  w_qkv   [(Hq + 2 Hkv) d, hidden] rows [Wq; Wk; Wv]; projections are x W^T
                                   ([KVB] section 3.1, Eq. 1: k = W_K x)
  K, V    [rows, Hkv, d]           token-major per-layer cache ([KVB] 3.1)
  Q       [rows, Hq, d]
  query head h reads kv head h // (Hq / Hkv) (grouped-query attention).

Readings of points the pages leave open (each is also listed with the
design notes of the repository):
  * RoPE is the rotate-half form (oracle.rope).
  * Re-positioning a chunk cached at local positions 0..|c|-1 to request
    start g is the delta rotation R(g); values are copied unchanged
    ([QCF] 2.1.2, Eq. 4; [KVB] 3.2's R^1000 example).
  * The deviation score is [KVB] Algorithm 2's delta_t with one layer and the
    Hkv key heads; the fresh keys come from a probe projection of every
    context token at its request position.
  * The attention-mass score normalises every (query token, head) row over
    its whole causal key set (context plus query keys up to itself) and reads
    the mass at context positions, summed over query heads and the last
    n_last_q query tokens ([QCF] 3.2.1, Eq. 9-10 at one layer).
  * The budget is k = floor(rho N) in integer arithmetic, rho in percent.
  * Selection ties go to the lower position; -0 equals +0; NaN ranks last;
    P is returned ascending.  Selection runs on float32-rounded scores.
  * Recomputed rows are P plus all U query rows; in one layer new K/V
    depend only on x, so the fused cache is complete before attention and
    every recomputed row attends over fused rows j <= its position.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

from . import rope, storage


@dataclasses.dataclass(frozen=True)
class Layer:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rope_base: float

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def sm_scale(self) -> float:
        # [KVB] section 3.1, Eq. 2: scores are scaled by 1 / sqrt(d).
        return 1.0 / math.sqrt(self.head_dim)


# ----------------------------------------------------------------------------
# projections
# ----------------------------------------------------------------------------
def split_weights(w_qkv: np.ndarray, layer: Layer):
    d = layer.head_dim
    nq, nk = layer.n_q_heads * d, layer.n_kv_heads * d
    w = np.asarray(w_qkv, dtype=np.float64)
    return w[:nq], w[nq:nq + nk], w[nq + nk:nq + 2 * nk]


def project(x_rows: np.ndarray, w: np.ndarray, n_heads: int, head_dim: int) -> np.ndarray:
    """x W^T reshaped to [n, heads, d] ([KVB] section 3.1, Eq. 1)."""
    y = np.asarray(x_rows, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    return y.reshape(len(x_rows), n_heads, head_dim)


def recompute(x_rows: np.ndarray, pos: np.ndarray, w_qkv: np.ndarray, layer: Layer,
              want=("q", "k", "v")) -> dict:
    """Fresh Q/K/V of rows at request positions `pos` ([QCF] 2.1.3: KV^New
    under the current order and positions).  Q and K carry RoPE at `pos`."""
    wq, wk, wv = split_weights(w_qkv, layer)
    out = {}
    if "q" in want:
        out["q"] = rope.rotate(project(x_rows, wq, layer.n_q_heads, layer.head_dim), pos, layer.rope_base)
    if "k" in want:
        out["k"] = rope.rotate(project(x_rows, wk, layer.n_kv_heads, layer.head_dim), pos, layer.rope_base)
    if "v" in want:
        out["v"] = project(x_rows, wv, layer.n_kv_heads, layer.head_dim)
    return out


def pic_encode(pool_hidden: np.ndarray, pool_pos: np.ndarray, w_qkv: np.ndarray, layer: Layer):
    """Per-chunk cache built in isolation ([QCF] 2.1.2, Eq. 3): keys encoded
    at chunk-local positions starting from zero.  One layer: K = R(t) x W_k^T,
    V = x W_v^T for every cached row at its local position t."""
    r = recompute(pool_hidden, pool_pos, w_qkv, layer, want=("k", "v"))
    return r["k"], r["v"]


# ----------------------------------------------------------------------------
# S1: re-position and stitch
# ----------------------------------------------------------------------------
def rerotate_stitch(pool_k: np.ndarray, pool_v: np.ndarray, chunk_table: np.ndarray,
                    total_rows: int, layer: Layer):
    """KV^PIC(C) = [Pi_1(KV_1^PIC); ...; Pi_m(KV_m^PIC)] ([QCF] 2.1.2, Eq. 4).

    chunk_table rows: (src_row, dst_row, pos0, len, ...).  A key cached at
    local position t moves to request position pos0 + t, which is the delta
    rotation R(pos0) applied to the cached (already rotated) key, because
    R(pos0) R(t) = R(pos0 + t) ([KVB] 3.2, Eq. 3).  Values are stitched in the
    same token order, unchanged.  Rows no chunk covers are left zero.
    """
    hkv, d = pool_k.shape[1], pool_k.shape[2]
    fk = np.zeros((total_rows, hkv, d), dtype=np.float64)
    fv = np.zeros((total_rows, hkv, d), dtype=np.float64)
    for src, dst, pos0, n in np.asarray(chunk_table)[:, :4]:
        src, dst, pos0, n = int(src), int(dst), int(pos0), int(n)
        fk[dst:dst + n] = rope.rotate(pool_k[src:src + n], np.full(n, pos0), layer.rope_base)
        fv[dst:dst + n] = pool_v[src:src + n]
    return fk, fv


# ----------------------------------------------------------------------------
# S2: scores
# ----------------------------------------------------------------------------
def deviation(k_cached: np.ndarray, k_fresh: np.ndarray) -> np.ndarray:
    """delta_t = 1 - (1/H) sum_h cos(K_t^h, K~_t^h)  ([KVB] 4.6.2, Algorithm 2,
    with one layer and H = the key heads).  A zero-norm vector gives cos 0."""
    a = np.asarray(k_cached, dtype=np.float64)
    b = np.asarray(k_fresh, dtype=np.float64)
    dot = np.sum(a * b, axis=-1)
    na = np.sqrt(np.sum(a * a, axis=-1))
    nb = np.sqrt(np.sum(b * b, axis=-1))
    den = na * nb
    with np.errstate(invalid="ignore", divide="ignore"):
        cos = np.where(den > 0, dot / np.where(den > 0, den, 1.0), 0.0)
    return 1.0 - cos.mean(axis=-1)


def attention_mass(q_u: np.ndarray, keys: np.ndarray, n_ctx: int, layer: Layer,
                   n_last_q: Optional[int] = None) -> np.ndarray:
    """Query-to-context attention mass of one request ([QCF] 3.2.1, Eq. 9-10
    at one layer).

    q_u:  [U, Hq, d] rotated queries of the query tokens (positions N..T-1)
    keys: [T, Hkv, d] keys of the request: re-positioned cached keys for
          j < N, fresh query keys for j >= N.
    Query token i attends causally to keys 0..N+i; its softmax is taken over
    that whole row and the mass landing on context position t < N is summed
    over all query heads and the last n_last_q query tokens.
    """
    U = q_u.shape[0]
    nq = U if (n_last_q is None or n_last_q <= 0) else min(n_last_q, U)
    G = layer.group
    score = np.zeros(n_ctx, dtype=np.float64)
    T = n_ctx + U
    i0 = U - nq
    limit = n_ctx + np.arange(i0, U)                     # last visible key per row
    mask = np.arange(T)[None, :] > limit[:, None]        # [nq, T]
    for h in range(layer.n_q_heads):
        s = (q_u[i0:, h, :] @ keys[:T, h // G, :].T) * layer.sm_scale
        s = np.where(mask, -np.inf, s)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        score += p[:, :n_ctx].sum(axis=0)
    return score


# ----------------------------------------------------------------------------
# S3: selection
# ----------------------------------------------------------------------------
def budget(n_ctx: int, ratio_pct: int) -> int:
    """k = floor(rho N) ([QCF] 3.2.1, Eq. 11; [KVB] Algorithm 2), computed in
    integers with rho given in percent."""
    return (int(n_ctx) * int(ratio_pct)) // 100


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """P = TopK(score, k) ([QCF] 3.2.1, Eq. 11).

    Order: larger score first, ties to the lower position, -0 == +0, NaN
    last.  Returns the k chosen positions in ascending order (int32).
    """
    s = np.asarray(scores)
    n = s.shape[0]
    if not 0 <= k <= n:
        raise ValueError("k out of range")
    nan = np.isnan(s)
    clean = np.where(nan, 0.0, s.astype(np.float64)) + 0.0     # -0 -> +0
    order = np.lexsort((np.arange(n), -clean, nan))             # last key first
    return np.sort(order[:k]).astype(np.int32)


# ----------------------------------------------------------------------------
# S5: fuse
# ----------------------------------------------------------------------------
def fuse(fused_k: np.ndarray, fused_v: np.ndarray, rows: np.ndarray,
         k_new: np.ndarray, v_new: np.ndarray):
    """KV^Fuse_p = KV^New_p for p in P, KV^PIC_p otherwise ([QCF] 2.1.3,
    Eq. 7), written back at the same positions.  Returns new arrays."""
    rows = np.asarray(rows, dtype=np.int64)
    if len(np.unique(rows)) != len(rows):
        raise ValueError("destination rows must be unique")
    fk = np.array(fused_k, dtype=np.float64, copy=True)
    fv = np.array(fused_v, dtype=np.float64, copy=True)
    fk[rows] = k_new
    fv[rows] = v_new
    return fk, fv


# ----------------------------------------------------------------------------
# S6: attention of the recomputed rows
# ----------------------------------------------------------------------------
def causal_attention(q: np.ndarray, q_pos: np.ndarray, keys: np.ndarray, values: np.ndarray,
                     layer: Layer):
    """O[r, h] = sum_{j <= pos_r} softmax_j(Q[r,h] . K[j, h//G] / sqrt(d)) V[j, h//G]
    ([KVB] 3.1, Eq. 2; [QCF] 2.1.3: a recomputed token reads prefix
    positions j <= p of the fused cache).  One request: keys/values are that
    request's rows.  Returns (O [M, Hq, d], lse [M, Hq]) with lse the natural
    log-sum-exp of the scaled scores."""
    q = np.asarray(q, dtype=np.float64)
    M = q.shape[0]
    G = layer.group
    pos = np.asarray(q_pos, dtype=np.int64)
    T = int(pos.max()) + 1 if M else 0
    out = np.zeros((M, layer.n_q_heads, layer.head_dim), dtype=np.float64)
    lse = np.zeros((M, layer.n_q_heads), dtype=np.float64)
    if M == 0:
        return out, lse
    mask = np.arange(T)[None, :] > pos[:, None]
    for h in range(layer.n_q_heads):
        s = (q[:, h, :] @ keys[:T, h // G, :].T) * layer.sm_scale
        s = np.where(mask, -np.inf, s)
        mx = s.max(axis=1, keepdims=True)
        p = np.exp(s - mx)
        z = p.sum(axis=1, keepdims=True)
        out[:, h, :] = (p / z) @ values[:T, h // G, :]
        lse[:, h] = (mx + np.log(z))[:, 0]
    return out, lse


# ----------------------------------------------------------------------------
# the whole layer
# ----------------------------------------------------------------------------
def fused_layer(x: np.ndarray, w_qkv: np.ndarray, pool_k: np.ndarray, pool_v: np.ndarray,
                chunk_table: np.ndarray, cu_T: Sequence[int], n_ctx: Sequence[int],
                layer: Layer, mode: str, k_per_req: Sequence[int],
                n_last_q: Optional[int] = None,
                forced_sel: Optional[Sequence[np.ndarray]] = None,
                store: Optional[str] = None,
                attend: Optional[Sequence[np.ndarray]] = None) -> dict:
    """Run the fused layer for a batch of independent requests.

    mode "deviation" ([KVB] Algorithm 2 at one layer): probe K~ for every row,
    score context tokens by key deviation, select, recompute Q and V of the
    selected and query rows, take their K from the probe, fuse, attend.
    mode "attn_mass" ([QCF] 3.2.1 at one layer): compute the query rows,
    place their K/V in the cache, score context tokens by the query-to-context
    attention mass, select, recompute Q/K/V of the selected and query rows,
    fuse, attend.

    mode "none": no scoring; the selection is `forced_sel` (a selector that
    needs no query-time score, e.g. static positions or per-chunk anchors),
    and Q/K/V of the selected and query rows are recomputed as in
    "attn_mass".

    `forced_sel` replaces the selection with given per-request positions
    (used to evaluate the rest of the layer on another selection).

    `store` ("bf16" or "f32", default None) evaluates the layer at a serving
    precision: every tensor a serving stack materialises - cache entries
    written by re-positioning or fusion, the key probe, the projected Q/K/V -
    is rounded to that format (round to nearest even) when it is produced;
    arithmetic between those points stays float64 and the attention output
    and LSE are not rounded.  The QCFuse page runs every strategy in a BF16
    serving stack (section 4.1.1); store="bf16" is that reading.  With
    store=None nothing is rounded.

    `attend` (per request, indices into that request's recomputed rows, i.e.
    its P followed by its U rows) restricts the attention step to those rows:
    "q", "out" and "lse" then hold only them, in that order (their queries
    are the only ones projected), and "attend_flat" gives their indices
    among all recomputed rows.  Every other output is unchanged.
    Returns every intermediate, float64, in flat request-major layouts.
    """
    def S(a):
        return a if store is None else storage.decode(storage.encode(a, store), store)

    x = np.asarray(x, dtype=np.float64)
    cu_T = [int(v) for v in cu_T]
    n_req = len(cu_T) - 1
    total = cu_T[-1]
    fk, fv = rerotate_stitch(pool_k, pool_v, chunk_table, total, layer)
    fk, fv = S(fk), S(fv)
    res = {"fused_k_pic": fk.copy(), "fused_v_pic": fv.copy()}

    scores, sels, rows_all, pos_all = [], [], [], []
    k_probe = None
    if mode == "deviation":
        allpos = np.concatenate([np.arange(cu_T[r + 1] - cu_T[r]) for r in range(n_req)])
        k_probe = S(recompute(x, allpos, w_qkv, layer, want=("k",))["k"])
        res["k_probe"] = k_probe
    elif mode not in ("attn_mass", "none"):
        raise ValueError(mode)
    if mode == "none" and forced_sel is None:
        raise ValueError("mode 'none' takes its selection from forced_sel")

    q_u_all = []
    for r in range(n_req):
        a, b, N = cu_T[r], cu_T[r + 1], int(n_ctx[r])
        if mode == "deviation":
            s = deviation(fk[a:a + N], k_probe[a:a + N])
        elif mode == "none":
            s = None
        else:
            qr = np.arange(a + N, b)
            qpos = np.arange(N, b - a)
            new = {k: S(v) for k, v in recompute(x[qr], qpos, w_qkv, layer).items()}
            fk[qr] = new["k"]
            fv[qr] = new["v"]
            q_u_all.append(new["q"])
            s = attention_mass(new["q"], fk[a:b], N, layer, n_last_q)
        scores.append(s)
        if forced_sel is not None:
            sel = np.asarray(forced_sel[r], dtype=np.int32)
        else:
            sel = select_topk(s.astype(np.float32), int(k_per_req[r]))
        sels.append(sel)
        pos_all.append(np.concatenate([sel, np.arange(N, b - a)]).astype(np.int32))
        rows_all.append((a + pos_all[-1]).astype(np.int32))
    if mode == "attn_mass":
        res["q_u"] = np.concatenate(q_u_all)
        res["fused_k_with_query"] = fk.copy()
        res["fused_v_with_query"] = fv.copy()

    rows = np.concatenate(rows_all)
    pos = np.concatenate(pos_all)
    sizes = [len(p) for p in pos_all]
    starts = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    if attend is None:
        flat = np.arange(len(rows), dtype=np.int64)
    else:
        flat = np.concatenate([starts[r] + np.asarray(attend[r], dtype=np.int64)
                               for r in range(n_req)])
    want_kv = ("v",) if mode == "deviation" else ("k", "v")
    new = {k: S(v) for k, v in recompute(x[rows], pos, w_qkv, layer, want=want_kv).items()}
    if mode == "deviation":
        new["k"] = k_probe[rows]
    new["q"] = S(recompute(x[rows[flat]], pos[flat], w_qkv, layer, want=("q",))["q"])
    fk, fv = fuse(fk, fv, rows, new["k"], new["v"])

    outs, lses = [], []
    qoff = 0
    for r in range(n_req):
        a, b = cu_T[r], cu_T[r + 1]
        idx = np.arange(sizes[r]) if attend is None else np.asarray(attend[r], dtype=np.int64)
        o, l = causal_attention(new["q"][qoff:qoff + len(idx)], pos_all[r][idx], fk[a:b], fv[a:b],
                                layer)
        outs.append(o)
        lses.append(l)
        qoff += len(idx)
    res["attend_flat"] = flat
    res.update(scores=scores, sel=sels, rows=rows, pos=pos, cu_q=starts,
               q=new["q"], k_new=new["k"], v_new=new["v"], fused_k=fk, fused_v=fv,
               out=np.concatenate(outs), lse=np.concatenate(lses))
    return res


def full_prefill(x: np.ndarray, w_qkv: np.ndarray, cu_T: Sequence[int], layer: Layer) -> dict:
    """Full prefill of one layer ([QCF] 2.1.1, Eq. 2): every row's K/V from its
    fresh hidden state at its request position, and causal attention of
    every row.  The reference that rho = 100% must reproduce."""
    x = np.asarray(x, dtype=np.float64)
    cu_T = [int(v) for v in cu_T]
    ks, vs, outs, lses = [], [], [], []
    for r in range(len(cu_T) - 1):
        a, b = cu_T[r], cu_T[r + 1]
        pos = np.arange(b - a)
        new = recompute(x[a:b], pos, w_qkv, layer)
        o, l = causal_attention(new["q"], pos, new["k"], new["v"], layer)
        ks.append(new["k"])
        vs.append(new["v"])
        outs.append(o)
        lses.append(l)
    return {"k": np.concatenate(ks), "v": np.concatenate(vs),
            "out": np.concatenate(outs), "lse": np.concatenate(lses)}
