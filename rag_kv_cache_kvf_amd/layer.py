"""One fused layer on the GPU: buffers plus the ordered libkvfuse calls.

This module sequences the six library calls of the hot path for one batch of
requests and owns the device buffers between them; it computes nothing
itself.  Order (all on one stream, no host synchronisation):

  deviation mode (KVBoost page, section 4.6.2, Algorithm 2 at one layer)
    kvf_recompute_qkv(all rows, K: probe K~) ->
    kvf_rerotate_deviation (re-positioning and the deviation score in one
    pass; with fuse_score=False: kvf_rerotate, then kvf_score(DEVIATION)
    after the probe) -> kvf_select_topk ->
    kvf_recompute_qkv(P+U, Q|V; V straight into the fused cache) ->
    kvf_scatter_kv(K of P+U from the probe) -> kvf_sparse_q_attention
  attention-mass mode (QCFuse page, section 3.2.1 at one layer)
    kvf_rerotate -> kvf_recompute_qkv(U, Q|K; K into the fused cache) ->
    kvf_score(ATTN_MASS) (with fuse_mass: the U-row probe, then
    kvf_rerotate_score_attn_mass, which re-positions the keys inside the
    score's first pass) -> kvf_select_topk ->
    kvf_recompute_qkv(P+U, Q|K|V; K/V into the fused cache) ->
    kvf_sparse_q_attention
  (the recompute call's destination-row output is the scatter of Eq. 7)
  static selection (KVBoost page, sections 4.1 and 4.6.1; QCFuse page,
  section 2.2.1)
    kvf_rerotate -> kvf_select_static -> kvf_select_topk(forced set only) ->
    kvf_recompute_qkv(P+U, Q|K|V into the fused cache) -> kvf_sparse_q_attention
  per-chunk key-norm anchors (QCFuse page, section 3.3.1, Eq. 14)
    kvf_rerotate -> kvf_score(KEY_NORM) -> kvf_select_topk_segmented ->
    kvf_recompute_qkv(P+U, Q|K|V into the fused cache) -> kvf_sparse_q_attention
  A score selector with static rules takes their positions as a forced set
  (kvf_select_static before kvf_select_topk).
  int8-resident fused cache (KVBoost page, section 4.5, Eq. 7 kept by the
  fused cache; section 7.3): the same order with kvf_rerotate_q8_deviation
  (or kvf_rerotate_q8 and kvf_score_q8) and kvf_sparse_q_attention_q8, and the recomputed K/V written
  to compact bf16 rows that kvf_scatter_kv_q8 encodes into the cache.

The per-chunk caches are built ahead of serving (QCFuse page, section 2.1.2,
Eq. 3) either by the caller (`pic=`) or on the GPU by this library's own
projection at chunk-local positions (and its KIVI encoder for 8- or 4-bit caches).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
import torch

from . import kvfuse as kvf
from .synth import Batch as SynthBatch


def _dev(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload a storage-encoded numpy array (float32 or bf16 bits)."""
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def _i32(a, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(device)


def _noop(stream=None):
    return None


class FusedLayerGPU:
    """k_only (default: dense per-request caches): the per-chunk values are
    stitched into the fused cache by the loader (`load()`, ahead of the pass),
    and the pass re-positions the keys only (QCFuse page, section 2.1.2: the
    values keep their token order; only the keys carry the rotation).  With
    k_only False, or for a shared chunk pool or KIVI codes, the pass gathers
    keys and values from the per-chunk caches itself.

    fuse_score (deviation mode): the key probe runs first and the
    re-positioning pass scores every context row as it writes its key
    (kvf_rerotate_deviation, or kvf_rerotate_q8_deviation for the
    int8-resident cache); False keeps the re-positioning and the score
    apart.  fuse_mass (attention-mass mode with keys-only re-positioning,
    off by default): the U-row probe runs first and the score's statistics
    pass re-positions each tile of keys as it reads them
    (kvf_rerotate_score_attn_mass); measured no faster than the two calls
    at the Qwen3-8B and Llama-3-70B shapes."""

    def __init__(self, batch: SynthBatch, ratio_pct: int, device="cuda",
                 pic: Optional[dict] = None, n_last_q: int = 0, mode: Optional[str] = None,
                 k_only: Optional[bool] = None, resident: Optional[str] = None,
                 fuse_score: bool = True, fuse_mass: bool = False):
        wl = batch.wl
        self.q8 = (wl.resident if resident is None else resident) == "q8"
        self.wl = wl
        self.batch = batch
        self.mode = mode or wl.score
        self.selector = wl.selector
        self.rules = tuple(int(v) for v in wl.static_rules)
        if self.selector not in ("score", "static", "anchor"):
            raise ValueError(f"unknown selector {self.selector!r}")
        # the key probe of deviation scoring; other selectors project P+U only
        self.probe = self.selector == "score" and self.mode == "deviation"
        self.mass = self.selector == "score" and self.mode != "deviation"
        # the fused score reduces a row's key within one wave: its lanes (bf16
        # or fp32 cache: Hkv d / 16 rotation units; int8-resident: Hkv d / 8
        # lanes, a row within one 256-thread workgroup) a power of two <= 64
        rl = wl.n_kv_heads * wl.head_dim // (8 if self.q8 else 16)
        self.fuse_dev = (fuse_score and self.probe and wl.head_dim % (32 if self.q8 else 16) == 0
                         and 1 <= rl <= 64 and rl & (rl - 1) == 0)
        self.n_last_q = n_last_q
        self.device = torch.device(device)
        dev = self.device
        L = kvf.Layer(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.dtype)
        self.layer = L
        self.kb = kvf.Batch(batch.cu_T, batch.n_ctx)
        td = L.torch_dtype
        hq, hkv, d = wl.n_q_heads, wl.n_kv_heads, wl.head_dim
        R = batch.n_req
        T_total = batch.total_rows

        self.x = _dev(batch.x, wl.dtype, dev)
        self.w = _dev(batch.w_qkv, wl.dtype, dev)
        self.chunks = _i32(batch.chunk_table, dev)
        self.max_chunk_len = int(batch.chunk_table[:, 3].max())
        max_T = int(np.diff(batch.cu_T).max())
        self.rope_n = max(max_T, self.max_chunk_len)
        self.rope_cos = torch.empty((self.rope_n, d // 2), dtype=torch.float32, device=dev)
        self.rope_sin = torch.empty_like(self.rope_cos)
        kvf.rope_table(wl.rope_base, d, self.rope_n, self.rope_cos, self.rope_sin)

        # per-chunk caches (ahead of serving)
        self.pool_k = self.pool_v = None
        self.kivi = None
        pool_rows = batch.pool_rows
        if pic is not None:
            if "k_codes" in pic:
                self.kivi = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev)
                             for k, v in pic.items()}
            else:
                self.pool_k = _dev(pic["k"], wl.dtype, dev)
                self.pool_v = _dev(pic["v"], wl.dtype, dev)
        else:
            pool_hidden = _dev(batch.pool_hidden, wl.dtype, dev)
            pool_pos = _i32(batch.pool_pos, dev)
            pk = torch.empty((pool_rows, hkv, d), dtype=td, device=dev)
            pv = torch.empty_like(pk)
            kvf.recompute_qkv(L, pool_hidden, None, pool_pos, self.w, kvf.KVF_OUT_K | kvf.KVF_OUT_V,
                              self.rope_cos, self.rope_sin, k_out=pk, v_out=pv)
            if wl.kivi_bits:
                n_pool = len(batch.pool_cu) - 1
                cb = d * wl.kivi_bits // 8               # code bytes per head row
                self.kivi = {
                    "k_codes": torch.empty((pool_rows, hkv, cb), dtype=torch.uint8, device=dev),
                    "v_codes": torch.empty((pool_rows, hkv, cb), dtype=torch.uint8, device=dev),
                    "k_min": torch.empty((n_pool, hkv, d), dtype=torch.float32, device=dev),
                    "k_scale": torch.empty((n_pool, hkv, d), dtype=torch.float32, device=dev),
                    "v_min": torch.empty((pool_rows, hkv), dtype=torch.float32, device=dev),
                    "v_scale": torch.empty((pool_rows, hkv), dtype=torch.float32, device=dev),
                }
                kvf.kivi_encode(L, pk, pv, _i32(batch.pool_cu, dev), self.max_chunk_len, self.kivi)
                del pk, pv
            else:
                self.pool_k, self.pool_v = pk, pv
            del pool_hidden

        # keys-only re-positioning: the values are stitched by load()
        dense = self.kivi is None
        self.k_only = (dense and not wl.pool_chunks and not self.q8) if k_only is None else bool(k_only)
        if self.q8 and (self.k_only or self.mass or wl.dtype != "bf16"):
            raise ValueError("the int8-resident cache takes a bf16 layer, a gathering "
                             "re-positioning and a score other than attention mass")
        if self.k_only and not dense:
            raise ValueError("keys-only re-positioning needs a dense per-chunk cache")
        # attention mass: the keys-only re-positioning rides on the score's pass
        self.fuse_mass = fuse_mass and self.mass and self.k_only and wl.dtype == "bf16"
        if self.k_only:
            src, dst = [], []
            for s0, d0, _, ln in batch.chunk_table[:, :4]:
                src.append(np.arange(s0, s0 + ln, dtype=np.int32))
                dst.append(np.arange(d0, d0 + ln, dtype=np.int32))
            self.stitch_src = _i32(np.concatenate(src), dev)
            self.stitch_dst = _i32(np.concatenate(dst), dev)

        # budgets and buffers
        self.static_mask = None
        self.segs = None
        if self.selector == "static":
            self.k_per_req = kvf.static_counts(self.kb, batch.chunk_table, self.rules)
        elif self.selector == "anchor":
            segs, ks = [], []
            for r in range(R):
                kr = 0
                for p0, ln in batch.chunk_spans(r):
                    kc = kvf.anchor_budget(ln, wl.anchor_pct, 100)
                    segs.append([r, p0, ln, kc, kr, 0, 0, 0])
                    kr += kc
                ks.append(kr)
            self.k_per_req = ks
            self.segs = _i32(np.asarray(segs, dtype=np.int32).reshape(-1, 8), dev)
        else:
            self.k_per_req = [kvf.recompute_budget(int(n), ratio_pct) for n in batch.n_ctx]
        if self.selector == "static" or any(self.rules):
            self.static_mask = torch.zeros(max(int(np.sum(batch.n_ctx)), 1), dtype=torch.uint8,
                                           device=dev)
        self.U = [self.kb.n_query(r) for r in range(R)]
        self.M_per_req = [k + u for k, u in zip(self.k_per_req, self.U)]
        self.cu_q = [0] + list(np.cumsum(self.M_per_req).astype(int))
        M = self.cu_q[-1]
        self.M = M
        n_scores = int(np.sum(batch.n_ctx))
        if self.q8:
            self.fused = kvf.q8_cache(T_total, hkv, d, device=dev)
            self.fused_k = self.fused_v = None
            # the recomputed rows' K (without a probe) and V, compact, before
            # kvf_scatter_kv_q8 encodes them into the cache
            self.k_new = torch.zeros((max(M, 1), hkv, d), dtype=td,
                                     device=dev) if not self.probe else None
            self.v_new = torch.zeros((max(M, 1), hkv, d), dtype=td,
                                     device=dev)
        else:
            self.fused = None
            self.fused_k = torch.zeros((T_total, hkv, d), dtype=td, device=dev)
            self.fused_v = torch.zeros_like(self.fused_k)
        self.scores = torch.zeros(max(n_scores, 1), dtype=torch.float32, device=dev)
        self.sel = torch.zeros(max(sum(self.k_per_req), 1), dtype=torch.int32, device=dev)
        self.rows = torch.zeros(max(M, 1), dtype=torch.int32, device=dev)
        self.pos = torch.zeros(max(M, 1), dtype=torch.int32, device=dev)
        self.q = torch.zeros((max(M, 1), hq, d), dtype=td, device=dev)
        self.out = torch.zeros((max(M, 1), hq, d), dtype=td, device=dev)
        self.lse = torch.zeros((max(M, 1), hq), dtype=torch.float32, device=dev)
        self.sm_scale = 1.0 / math.sqrt(d)
        u_host = np.asarray(batch.query_rows(), dtype=np.int64)
        self.u_rows = _i32(u_host, dev)
        self.u_pos = _i32(batch.query_pos(), dev)
        nU = int(self.u_rows.shape[0])
        # one block of consecutive rows (a single request): the probe reads
        # that slice of x directly, without a row map to gather through
        self.u_span = None
        if nU > 0 and np.all(np.diff(u_host) == 1):
            self.u_span = (int(u_host[0]), int(u_host[0]) + nU)
        self.ws = None
        if self.probe:
            self.all_pos = _i32(batch.all_pos(), dev)
            self.k_probe = torch.zeros((T_total, hkv, d), dtype=td, device=dev)
        elif self.mass:
            self.q_u = torch.zeros((max(nU, 1), hq, d), dtype=td, device=dev)
            nbytes = kvf.score_workspace_size(kvf.KVF_SCORE_ATTN_MASS, L, self.kb, n_last_q)
            self.ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=dev)
        # one projection workspace for every recompute call (they are ordered
        # on the stream), so the stages allocate nothing
        QKV = kvf.KVF_OUT_Q | kvf.KVF_OUT_K | kvf.KVF_OUT_V
        need = [kvf.recompute_workspace_size(L, M, QKV)]
        if self.probe:
            need.append(kvf.recompute_workspace_size(L, T_total, kvf.KVF_OUT_K))
        elif self.mass:
            need.append(kvf.recompute_workspace_size(L, nU, kvf.KVF_OUT_Q | kvf.KVF_OUT_K))
        # zeroed: split projections keep arrival counters at its start
        self.gemm_ws = torch.zeros(max(max(need), 1), dtype=torch.uint8, device=dev)
        # key-split workspace of the attention call: zero-filled once, every
        # call leaves it zeroed
        attn_need = kvf.attention_workspace_size(self.layer, self.kb, self.cu_q)
        self.attn_ws = (torch.zeros(attn_need, dtype=torch.uint8, device=dev)
                        if attn_need > 0 else None)
        self.use_prepared = True
        self._prep = {}

    # ------------------------------------------------------------------ calls
    def _rerotate(self):
        if self.q8 and self.fuse_dev:
            return kvf.rerotate_q8_deviation(self.layer, self.kb, self.chunks, self.max_chunk_len,
                                             self.pool_k, self.pool_v, self.rope_cos, self.rope_sin,
                                             self.fused, self.k_probe, self.scores, kivi=self.kivi)
        if self.q8:
            return kvf.rerotate_q8(self.layer, self.chunks, self.max_chunk_len, self.pool_k, self.pool_v,
                                   self.rope_cos, self.rope_sin, self.fused, kivi=self.kivi)
        if self.fuse_dev:
            return kvf.rerotate_deviation(
                self.layer, self.kb, self.chunks, self.max_chunk_len, self.pool_k,
                None if self.k_only else self.pool_v, self.rope_cos, self.rope_sin, self.fused_k,
                None if self.k_only else self.fused_v, self.k_probe, self.scores, kivi=self.kivi,
                k_only=self.k_only)
        if self.k_only:
            return kvf.rerotate(self.layer, self.chunks, self.max_chunk_len, self.pool_k, None,
                                self.rope_cos, self.rope_sin, self.fused_k, None, k_only=True)
        return kvf.rerotate(self.layer, self.chunks, self.max_chunk_len, self.pool_k, self.pool_v,
                            self.rope_cos, self.rope_sin, self.fused_k, self.fused_v, kivi=self.kivi)

    def load(self):
        """The loader's part ahead of a pass in keys-only mode: the per-chunk
        values stitched into the fused value cache in token order (a row copy
        through kvf_scatter_kv).  A no-op when the pass gathers the values."""
        if not self.k_only:
            return
        kvf.scatter_kv(self.layer, None, None, self.pool_v, self.stitch_src, self.stitch_dst,
                       self.fused_k, self.fused_v, M=int(self.stitch_dst.shape[0]))

    def _k_probe(self):
        return kvf.recompute_qkv(self.layer, self.x, None, self.all_pos, self.w, kvf.KVF_OUT_K,
                                 self.rope_cos, self.rope_sin, k_out=self.k_probe, workspace=self.gemm_ws)

    def _u_probe(self):
        # Q and K of the query rows only: the score reads the query keys (the
        # causal part of each query row) but no values, and the recompute of
        # P + U writes the query rows' K and V before attention reads them
        mask = kvf.KVF_OUT_Q | kvf.KVF_OUT_K
        if self.u_span is not None:
            a, b = self.u_span
            return kvf.recompute_qkv(self.layer, self.x[a:b], None, self.u_pos, self.w, mask,
                                     self.rope_cos, self.rope_sin, q_out=self.q_u, k_out=self.fused_k,
                                     kv_out_row=self.u_rows, workspace=self.gemm_ws)
        return kvf.recompute_qkv(self.layer, self.x, self.u_rows, self.u_pos, self.w, mask,
                                 self.rope_cos, self.rope_sin, q_out=self.q_u, k_out=self.fused_k,
                                 kv_out_row=self.u_rows, workspace=self.gemm_ws)

    def _static_mask(self):
        return kvf.select_static(self.kb, self.chunks, self.rules, self.static_mask)

    def _score(self):
        if self.q8:
            if self.selector == "anchor":
                return kvf.score_q8(kvf.KVF_SCORE_KEY_NORM, self.layer, self.kb, self.fused, None,
                                    self.scores)
            return kvf.score_q8(kvf.KVF_SCORE_DEVIATION, self.layer, self.kb, self.fused, self.k_probe,
                                self.scores)
        if self.selector == "anchor":
            return kvf.score(kvf.KVF_SCORE_KEY_NORM, self.layer, self.kb, self.fused_k, None, None,
                             self.scores)
        elif self.mode == "deviation":
            return kvf.score(kvf.KVF_SCORE_DEVIATION, self.layer, self.kb, self.fused_k, self.k_probe,
                             None, self.scores)
        elif self.fuse_mass:
            return kvf.rerotate_score_attn_mass(self.layer, self.kb, self.chunks, self.max_chunk_len,
                                                self.pool_k, self.rope_cos, self.rope_sin, self.fused_k,
                                                self.q_u, self.scores, self.ws, n_last_q=self.n_last_q)
        else:
            return kvf.score(kvf.KVF_SCORE_ATTN_MASS, self.layer, self.kb, self.fused_k, None, self.q_u,
                             self.scores, self.ws, n_last_q=self.n_last_q)

    def _select(self):
        if self.selector == "anchor":
            return kvf.select_topk_segmented(self.scores, self.kb, self.segs, self.k_per_req, self.sel,
                                             self.rows, self.pos)
        else:
            return kvf.select_topk(None if self.selector == "static" else self.scores, self.kb,
                                   self.k_per_req, self.sel, self.rows, self.pos,
                                   forced=self.static_mask)

    def _recompute(self):
        if self.M == 0:
            return None
        if self.q8:
            # compact K (unless the probe has it) and V rows for kvf_scatter_kv_q8
            mask = kvf.KVF_OUT_Q | kvf.KVF_OUT_V | (0 if self.probe else kvf.KVF_OUT_K)
            return kvf.recompute_qkv(self.layer, self.x, self.rows, self.pos, self.w, mask,
                                     self.rope_cos, self.rope_sin, q_out=self.q, k_out=self.k_new,
                                     v_out=self.v_new, M=self.M, workspace=self.gemm_ws)
        if self.probe:
            # K of these rows is already in the probe
            return kvf.recompute_qkv(self.layer, self.x, self.rows, self.pos, self.w,
                                     kvf.KVF_OUT_Q | kvf.KVF_OUT_V, self.rope_cos, self.rope_sin,
                                     q_out=self.q, v_out=self.fused_v, kv_out_row=self.rows, M=self.M,
                                     workspace=self.gemm_ws)
        else:
            return kvf.recompute_qkv(self.layer, self.x, self.rows, self.pos, self.w,
                                     kvf.KVF_OUT_Q | kvf.KVF_OUT_K | kvf.KVF_OUT_V, self.rope_cos,
                                     self.rope_sin, q_out=self.q, k_out=self.fused_k, v_out=self.fused_v,
                                     kv_out_row=self.rows,
                                     M=self.M, workspace=self.gemm_ws)

    def _scatter(self):
        # deviation mode: K of the recomputed rows is the probe's
        if self.M == 0:
            return None
        if self.q8:
            k_src, k_row = (self.k_probe, self.rows) if self.probe else (self.k_new, None)
            return kvf.scatter_kv_q8(self.layer, k_src, k_row, self.v_new, None, self.rows, self.fused,
                                     M=self.M)
        return kvf.scatter_kv(self.layer, self.k_probe, self.rows, None, None, self.rows, self.fused_k,
                              self.fused_v, M=self.M)

    def _attention(self):
        if self.M == 0:
            return None
        if self.q8:
            return kvf.sparse_q_attention_q8(self.layer, self.kb, self.q, self.pos, self.cu_q, self.fused,
                                             self.sm_scale, self.out, self.lse, workspace=self.attn_ws)
        return kvf.sparse_q_attention(self.layer, self.kb, self.q, self.pos, self.cu_q, self.fused_k,
                                      self.fused_v, self.sm_scale, self.out, self.lse,
                                      workspace=self.attn_ws)

    def fn(self, name):
        """The library call `name` (rerotate, k_probe, u_probe, static_mask,
        score, select, recompute, scatter, attention) as a callable.  With
        use_prepared, its arguments are marshalled on first use and reused
        (device pointers, ctypes structs), so a pass costs the host little
        more than the launches; call invalidate_prepared() after replacing a
        buffer the calls read."""
        if not self.use_prepared:
            return getattr(self, "_" + name)
        p = self._prep.get(name)
        if p is None:
            with kvf.preparing():
                p = getattr(self, "_" + name)()
            if p is None:                        # nothing to run (no recomputed rows)
                p = _noop
            self._prep[name] = p
        return p

    def invalidate_prepared(self):
        self._prep = {}

    def calls(self):
        """The library calls of one pass, in order, as (name, stage, fn):
        stage is one of rerotate / score / select / recompute_fuse / attention."""
        f = self.fn
        fuse = [("recompute", "recompute_fuse", f("recompute"))]
        if self.probe or self.q8:
            fuse.append(("scatter", "recompute_fuse", f("scatter")))
        first = [("rerotate", "rerotate", f("rerotate"))]
        if self.fuse_dev:
            # the probe first: the re-positioning pass scores against it
            first.insert(0, ("k_probe", "rerotate", f("k_probe")))
            score = []
        elif self.fuse_mass:
            # the U-row probe first: the score's pass re-positions the keys
            first = [("u_probe", "rerotate", f("u_probe")), ("score", "rerotate", f("score"))]
            score = []
        elif self.probe:
            score = [("k_probe", "score", f("k_probe")), ("score", "score", f("score"))]
        elif self.mass:
            score = [("u_probe", "score", f("u_probe")), ("score", "score", f("score"))]
        elif self.selector == "anchor":
            score = [("score", "score", f("score"))]
        else:
            score = []
        select = [("select", "select", f("select"))]
        if self.static_mask is not None:
            select.insert(0, ("static_mask", "select", f("static_mask")))
        return (first + score + select + fuse +
                [("attention", "attention", f("attention"))])

    def _stage(self, stage):
        for _, st, fn in self.calls():
            if st == stage:
                fn()

    def stage_rerotate(self):
        self._stage("rerotate")

    def stage_score(self):
        self._stage("score")

    def stage_select(self):
        self._stage("select")

    def force_selection(self, sel: Sequence[np.ndarray]):
        """Replace the selection with given per-request positions (tests)."""
        rows, pos, flat = [], [], []
        b = self.batch
        for r in range(b.n_req):
            s = np.asarray(sel[r], dtype=np.int32)
            assert len(s) == self.k_per_req[r]
            p = np.concatenate([s, np.arange(b.n_ctx[r], b.cu_T[r + 1] - b.cu_T[r], dtype=np.int32)])
            pos.append(p)
            rows.append(p + b.cu_T[r])
            flat.append(s)
        self.rows.copy_(_i32(np.concatenate(rows), self.device))
        self.pos.copy_(_i32(np.concatenate(pos), self.device))
        if sum(self.k_per_req):
            self.sel.copy_(_i32(np.concatenate(flat), self.device))

    def stage_recompute_fuse(self):
        self._stage("recompute_fuse")

    def stage_attention(self):
        self._stage("attention")

    def step(self):
        """Enqueue one pass of the hot path (the calls() list) on the current
        stream; in keys-only mode the values must already be stitched
        (load()), and a pass leaves them stitched except at the rows it
        recomputes, which the next pass with the same selection rewrites."""
        for _, _, fn in self.calls():
            fn()

    def run(self, forced_sel: Optional[Sequence[np.ndarray]] = None):
        """Enqueue load() and one pass of the whole path on the current
        stream (optionally with a given selection instead of top-k)."""
        self.load()
        if forced_sel is None:
            self.step()
            return
        forced = False
        for _, st, fn in self.calls():
            if st != "select":
                fn()
            elif not forced:
                self.force_selection(forced_sel)
                forced = True

    # ------------------------------------------------------------------ readback
    def selection(self):
        s = self.sel.cpu().numpy()
        out, off = [], 0
        for k in self.k_per_req:
            out.append(s[off:off + k].copy())
            off += k
        return out
