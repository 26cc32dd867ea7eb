"""Several layers of the fused path: shared selection signals and a layer-wise
cache pipeline.

Each layer is a FusedLayerGPU (its own weights, hidden states, per-chunk
cache and fused cache); this module only orders their library calls and the
copies between host and device memory.  It computes nothing itself.

Selection across layers (QCFuse page, "QCFuse: Query-Aware Cache Fusion via
Compressed View for Efficient RAG Serving"):
  signal ""            every layer selects from its own score (one-layer path);
  signal "sum"         one P for every layer from the attention mass summed over
                       a layer set - all layers (section 3.2.1, Eq. 10) or a
                       critical set (section 3.4.2, Eq. 20): kvf_score with
                       KVF_SCORE_ACCUMULATE, then one kvf_select_topk;
  signal "progressive" CacheBlend's narrowing (section 2.2.1): layer l probes
                       only layer l-1's picks, scores them (kvf_score with the
                       previous selection mask as its eligible set) and keeps
                       its own, smaller budget.

Layer-wise pipeline (QCFuse section 3.5 and Fig. 2, loading the next
layer's cache while the current one is fused): with stream_pools, every
layer's per-chunk cache stays in pinned host memory; a second stream copies
it into one of two device slots while earlier layers compute, and the
compute stream waits for that copy (an event) before re-positioning the
layer.  A slot is refilled only after the layer that last read it has been
re-positioned (another event), also across passes, so back-to-back passes
load their first layers while the previous pass finishes.  The host buffers
must not change while a pass is in flight.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np
import torch

from . import kvfuse as kvf
from .layer import FusedLayerGPU


class MultiLayerGPU:
    def __init__(self, batches: Sequence, ratio_pct: int, device="cuda",
                 pics: Optional[Sequence[dict]] = None, stream_pools: Optional[bool] = None):
        wl = batches[0].wl
        self.wl = wl
        self.n_layers = len(batches)
        self.signal = wl.signal
        if self.signal not in ("", "sum", "progressive"):
            raise ValueError(f"unknown signal {self.signal!r}")
        if self.signal == "progressive":
            pcts = list(wl.progressive_pct)
            if len(pcts) != self.n_layers or wl.score != "deviation":
                raise ValueError("progressive filtering takes one budget per layer and the "
                                 "deviation score")
        else:
            pcts = [ratio_pct] * self.n_layers
        self.pcts = pcts
        self.device = torch.device(device)
        self.layers: List[FusedLayerGPU] = [
            # (the layers keep the re-positioning and the score apart: the
            # passes order them per layer, progressive filtering probes and
            # scores only the previous picks)
            FusedLayerGPU(b, p, device=device, pic=None if pics is None else pics[l], k_only=False,
                          fuse_score=False)
            for l, (b, p) in enumerate(zip(batches, pcts))]
        l0 = self.layers[0]
        self.kb = l0.kb
        self._prep = {}          # prepared calls of this driver's own closures

        if self.signal == "sum":
            if wl.score != "attn_mass":
                raise ValueError("the layer sum is taken over the attention mass")
            self.score_layers = list(wl.score_layers) or list(range(self.n_layers))
            # one selection for all layers
            for ly in self.layers[1:]:
                ly.scores, ly.sel, ly.rows, ly.pos = l0.scores, l0.sel, l0.rows, l0.pos
        if self.signal == "progressive":
            n = max(int(np.sum(batches[0].n_ctx)), 1)
            for l, ly in enumerate(self.layers):
                ly.sel_mask = torch.zeros(n, dtype=torch.uint8, device=self.device)
                if l > 0:
                    # the probe of the previous layer's picks may split K
                    need = kvf.recompute_workspace_size(ly.layer, self.layers[l - 1].M,
                                                        kvf.KVF_OUT_K)
                    if need > ly.gemm_ws.numel():
                        ly.gemm_ws = torch.zeros(need, dtype=torch.uint8, device=self.device)

        # layer-wise pipeline: per-chunk caches in pinned host memory
        self.stream_pools = wl.stream_pools if stream_pools is None else stream_pools
        if self.stream_pools:
            if any(ly.kivi is not None or ly.pool_k is None for ly in self.layers):
                raise ValueError("streamed caches are dense")
            shape = self.layers[0].pool_k.shape
            if any(ly.pool_k.shape != shape for ly in self.layers):
                raise ValueError("layers must share the cache layout")
            # K and V of a layer side by side, so one copy moves both
            self.host_pools = []
            for ly in self.layers:
                h = torch.empty((2,) + tuple(shape), dtype=ly.pool_k.dtype).pin_memory()
                h[0].copy_(ly.pool_k.cpu())
                h[1].copy_(ly.pool_v.cpu())
                self.host_pools.append(h)
            self.slots = [torch.empty((2,) + tuple(shape), dtype=self.layers[0].pool_k.dtype,
                                      device=self.device) for _ in range(2)]
            for ly in self.layers:
                ly.pool_k = ly.pool_v = None          # the device copies are freed
            torch.cuda.synchronize()
            # the last re-position that read each slot (kept across passes, so
            # the next pass's first copies start as soon as the slots are free)
            self._slot_reader = [None, None]
            # Events are made once and recorded again every pass; a stream's
            # wait takes the record current at the time of the wait.
            self._ev_read = [torch.cuda.Event(), torch.cuda.Event()]
            self._ev_copy = [torch.cuda.Event() for _ in range(self.n_layers)]
            self.copy_stream = torch.cuda.Stream(device=self.device)
        # Streamed passes keep at most two passes in flight: the host waits for
        # pass p - 2 before enqueuing pass p.  With an unbounded lead the
        # runtime's queues fill with cross-stream waits and a 4-layer pass
        # took 2.6 ms instead of 1.6 ms (the copies alone take 1.5 ms).
        self.max_passes_in_flight = 2
        self._pass_end = [torch.cuda.Event() for _ in range(self.max_passes_in_flight + 1)]
        self._n_pass = 0

    # ------------------------------------------------------------------ order
    def rerotate_order(self) -> List[int]:
        """Layers in the order their caches are re-positioned (and loaded)."""
        if self.signal == "sum":
            rest = [l for l in range(self.n_layers) if l not in self.score_layers]
            return list(self.score_layers) + rest
        return list(range(self.n_layers))

    def calls(self):
        """(name, layer, fn) for every library call of one pass, in order; the
        rerotate calls of a streamed pipeline include the wait for their copy."""
        L = self.layers
        out = []
        if self.signal == "sum":
            l0 = L[0]
            for j, l in enumerate(self.score_layers):
                ly = L[l]
                out.append(("rerotate", l, self._rerotate_fn(l)))
                out.append(("u_probe", l, ly.fn("u_probe")))
                out.append(("score", l, self._sum_score_fn(l, accumulate=j > 0)))
            out.append(("select", 0, l0.fn("select")))
            for l in range(self.n_layers):
                if l not in self.score_layers:
                    out.append(("rerotate", l, self._rerotate_fn(l)))
                out.append(("recompute", l, L[l].fn("recompute")))
                out.append(("attention", l, L[l].fn("attention")))
        elif self.signal == "progressive":
            for l, ly in enumerate(L):
                out.append(("rerotate", l, self._rerotate_fn(l)))
                out.append(("k_probe", l, self._probe_fn(l)))
                out.append(("score", l, self._prog_score_fn(l)))
                out.append(("select", l, self._prog_select_fn(l)))
                out.append(("recompute", l, ly.fn("recompute")))
                out.append(("scatter", l, ly.fn("scatter")))
                out.append(("attention", l, ly.fn("attention")))
        else:
            for l, ly in enumerate(L):
                for name, _, fn in ly.calls():
                    out.append((name, l, self._rerotate_fn(l) if name == "rerotate" else fn))
        return out

    # ------------------------------------------------------------------ calls
    def _prepared(self, key, make):
        """A prepared library call of this driver, made once by make()."""
        p = self._prep.get(key)
        if p is None:
            with kvf.preparing():
                p = make()
            self._prep[key] = p
        return p

    def _rerotate_fn(self, l):
        ly = self.layers[l]
        if not self.stream_pools:
            return ly.fn("rerotate")

        def rot_from(s):
            def make():
                ly.pool_k, ly.pool_v = self.slots[s][0], self.slots[s][1]
                try:
                    return ly._rerotate()
                finally:
                    ly.pool_k = ly.pool_v = None
            return self._prepared(("rerotate", l, s), make)

        def run():
            j = self._order_index[l]
            cur = torch.cuda.current_stream(self.device)
            cur.wait_event(self._copied[j])
            rot_from(j % 2)()
            done = self._ev_read[j % 2]
            done.record(cur)
            self._slot_reader[j % 2] = done
            self._issue_copy(j + 2)
        return run

    def _issue_copy(self, j):
        """Copy the cache of the j-th layer in re-position order into slot j % 2,
        after the re-position that last read that slot."""
        order = self._order
        if j >= len(order):
            return
        s = j % 2
        with torch.cuda.stream(self.copy_stream):
            if self._slot_reader[s] is not None:
                self.copy_stream.wait_event(self._slot_reader[s])
            self.slots[s].copy_(self.host_pools[order[j]], non_blocking=True)
            ev = self._ev_copy[j]
            ev.record(self.copy_stream)
        self._copied[j] = ev

    def _begin_pass(self):
        if not self.stream_pools:
            return
        self._order = self.rerotate_order()
        self._order_index = {l: j for j, l in enumerate(self._order)}
        self._copied = [None] * len(self._order)
        # no wait for the previous pass as a whole: a slot is refilled as soon
        # as its last reader is done, so the first layers of this pass load
        # while the previous pass is still fusing its last layers
        self._issue_copy(0)
        self._issue_copy(1)

    def _sum_score_fn(self, l, accumulate):
        ly, l0 = self.layers[l], self.layers[0]
        return self._prepared(("score", l), lambda: kvf.score(
            kvf.KVF_SCORE_ATTN_MASS, ly.layer, ly.kb, ly.fused_k, None, ly.q_u, l0.scores, ly.ws,
            n_last_q=ly.n_last_q, accumulate=accumulate))

    def _probe_fn(self, l):
        ly = self.layers[l]
        if l == 0:
            return ly.fn("k_probe")
        prev = self.layers[l - 1]
        # the probe keys of the previous layer's picks (and query rows) only
        return self._prepared(("k_probe", l), lambda: kvf.recompute_qkv(
            ly.layer, ly.x, prev.rows, prev.pos, ly.w, kvf.KVF_OUT_K, ly.rope_cos, ly.rope_sin,
            k_out=ly.k_probe, kv_out_row=prev.rows, M=prev.M, workspace=ly.gemm_ws))

    def _prog_score_fn(self, l):
        ly = self.layers[l]
        elig = None if l == 0 else self.layers[l - 1].sel_mask
        return self._prepared(("score", l), lambda: kvf.score(
            kvf.KVF_SCORE_DEVIATION, ly.layer, ly.kb, ly.fused_k, ly.k_probe, None, ly.scores,
            eligible=elig))

    def _prog_select_fn(self, l):
        ly = self.layers[l]
        return self._prepared(("select", l), lambda: kvf.select_topk(
            ly.scores, ly.kb, ly.k_per_req, ly.sel, ly.rows, ly.pos, out_mask=ly.sel_mask))

    # ------------------------------------------------------------------ passes
    def run(self, forced_sel: Optional[Sequence] = None):
        """Enqueue one pass over every layer on the current stream.

        forced_sel replaces the selection: one list of per-request positions
        (signal "sum") or one per layer ("progressive", ""), used to run the
        rest of the layers on another selection."""
        k = self.max_passes_in_flight
        if self.stream_pools and self._n_pass >= k:
            self._pass_end[(self._n_pass - k) % (k + 1)].synchronize()
        self._begin_pass()
        for name, l, fn in self.calls():
            if forced_sel is not None and name == "select":
                self._force(l, forced_sel)
            else:
                fn()
        self._pass_end[self._n_pass % (k + 1)].record(torch.cuda.current_stream(self.device))
        self._n_pass += 1

    def _force(self, l, forced_sel):
        if self.signal == "sum":
            self.layers[0].force_selection(forced_sel)
            return
        ly = self.layers[l]
        ly.force_selection(forced_sel[l])
        if self.signal == "progressive":
            b = ly.batch
            m = np.zeros(max(int(np.sum(b.n_ctx)), 1), dtype=np.uint8)
            off = 0
            for r in range(b.n_req):
                m[off + np.asarray(forced_sel[l][r], dtype=np.int64)] = 1
                off += int(b.n_ctx[r])
            ly.sel_mask.copy_(torch.from_numpy(m).to(self.device))

    def set_streaming(self, on: bool):
        """Switch between streamed caches (pinned host memory, copied in every
        pass) and resident ones (device copies made once), same layers."""
        if not hasattr(self, "host_pools"):
            raise ValueError("the layers were built with resident caches")
        torch.cuda.synchronize()
        for l, ly in enumerate(self.layers):
            if on:
                ly.pool_k = ly.pool_v = None
            else:
                h = self.host_pools[l].to(self.device)
                ly.pool_k, ly.pool_v = h[0], h[1]
        torch.cuda.synchronize()
        self.stream_pools = on
        self._slot_reader = [None, None]
        self._prep = {}
        for ly in self.layers:
            ly.invalidate_prepared()

    def cache_bytes(self) -> int:
        """Bytes of per-chunk cache a streamed pass copies in."""
        if not hasattr(self, "host_pools"):
            return 0
        return sum(h.numel() * h.element_size() for h in self.host_pools)

    def run_copies_only(self):
        """The pass's host-to-device cache copies alone (timing reference)."""
        if not hasattr(self, "host_pools"):
            return
        for l in self.rerotate_order():
            self.slots[0].copy_(self.host_pools[l], non_blocking=True)
