"""Benchmark of one fused RAG KV-cache layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--ratio PCT] [--no-cpu-baseline] [--no-extra] [--graph]
    python bench.py --copy-calibration      # plain 1 GiB device copy (counter scale)

A step is one pass of the whole hot path over one batch of synthetic input:
re-position -> score -> top-k -> Q/K/V recompute -> scatter -> sparse-query
attention (the attention-mass path for the default workload).  Inputs,
weights and the per-chunk caches are resident in HBM before timing starts
(the caches are built by the library's own projection at chunk-local
positions, ahead of the timed region; for per-request dense caches the
loader's stitch of the values also happens before timing, and the step
re-positions the keys only).  The metric is fused context tokens per second
per layer: (sum over requests of N) / step time.

Timing, after W warm-up steps:
  1. K steps, each after an untimed read of a 1 GiB buffer (which evicts
     the working set from the L2 caches and the Infinity Cache and leaves
     clean lines), each timed by HIP events on the launch stream: `value`
     and `ms_per_step` use the median, `timing` also gives p10 and p90, and
     the median after a read-modify-write flush instead (dirty lines);
  2. K steps back to back (warm caches), for comparison;
  3. K flushed steps with every library call bracketed by HIP events: each
     call's average duration and its roofline fraction (algorithmic bytes or
     flops / duration); `ms_warm` is the same without the flushes.
The roofline object describes the call that takes longest; its `traffic` is
the HBM bytes per launch from the committed counter summary of that kernel
and workload under profiles/, or null when the kernel source has changed
since the counters were taken.  The default run adds the 8-request pool
workload at 30% and 15%, and the Qwen2.5-3B-shaped int8 KIVI layer with a
bf16 and with an int8-resident fused cache, as sub-objects.  The CPU baseline runs the float64
oracle on the same batch on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "qwen3_8b_mass"
# the second workload the @r=30% metric is quoted on, measured in the same
# run at both of its ratios (sub-objects of the JSON line)
EXTRA_WORKLOAD = "qwen3_8b_dev_pool"
METRIC = "fused context tokens/s per layer @r=30% on 1 MI355X; % MFMA/HBM roofline"
UNIT = "fused context tokens/s per layer"
# MI355X published peaks: HBM3E bandwidth, dense MFMA bf16, fp32 vector, and
# the host link
PEAK = {"hbm": 8000.0, "bf16": 2500.0, "f32": 157.3,
        "pcie": 64.0}    # host link: PCIe 5.0 x16, one direction, GB/s
KDIR = os.path.join(ROOT, "rag_kv_cache_kvf_amd", "csrc")
# library call -> (kernel that dominates it, its source file)
CALL_KERNEL = {
    "rerotate": ("rerotate_kernel", "kernels/rope_rerotate.hip"),
    "k_probe": ("gemm_qkv_bf16_kernel", "kernels/gemm_qkv.hip"),
    "u_probe": ("gemm_qkv_bf16_kernel", "kernels/gemm_qkv.hip"),
    "score": ("mass_colsum_bf16_kernel", "kernels/attention.hip"),
    "static_mask": ("static_mask_kernel", "kernels/static_mask.hip"),
    "select": ("topk_kernel", "kernels/topk.hip"),
    "recompute": ("gemm_qkv_bf16_kernel", "kernels/gemm_qkv.hip"),
    "scatter": ("scatter_kernel", "kernels/scatter_deviation.hip"),
    "attention": ("attn_mfma_kernel", "kernels/attention.hip"),
}
# the int8-resident forms of the calls that touch the fused cache
CALL_KERNEL_Q8 = {
    "rerotate": ("rerotate_q8_kernel", "kernels/rope_rerotate.hip"),
    "scatter": ("scatter_q8_kernel", "kernels/scatter_deviation.hip"),
}
# the int8 KIVI workload with a bf16 fused cache and with an int8-resident
# one, measured in the default run as sub-objects
Q8_WORKLOADS = ("qwen25_3b_kivi8", "qwen25_3b_kivi8_resident")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--ratio", type=int, default=None, help="recompute ratio in percent")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the pool workload's sub-objects in the default run")
    ap.add_argument("--graph", action="store_true", help="replay the step as one HIP graph")
    ap.add_argument("--unfused", action="store_true",
                    help="deviation workloads: re-positioning and score as separate calls "
                         "(kvf_rerotate + kvf_score instead of kvf_rerotate_deviation)")
    ap.add_argument("--fuse-mass", action="store_true",
                    help="attention-mass workloads: re-position the keys inside the score's "
                         "first pass (kvf_rerotate_score_attn_mass)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of 1 GiB, 3 times")
    return ap.parse_args()


def call_work(g):
    """Algorithmic work of every library call of one step:
    name -> ("hbm", bytes) or ("mfma", flops)."""
    wl = g.wl
    b = g.batch
    hq, hkv, d, hid = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.hidden
    esz = 2 if wl.dtype == "bf16" else 4
    krow = hkv * d * esz                           # bytes of one token's K (or V)
    n_ctx = int(sum(b.n_ctx))
    total = b.total_rows
    nU = total - n_ctx
    M = g.M
    pos = g.pos.cpu().numpy()[:M].astype("int64")
    work = {}
    q8row = hkv * (d + 8)                          # int8-resident row: codes + (min, scale)
    n_chunks = b.chunk_table.shape[0]
    if g.q8:
        # pool K codes (or bf16 K) and per-chunk K stats in; V codes and
        # per-token stats copied (or bf16 V encoded); K and V codes + stats out
        src = (2 * hkv * d + 8 * hkv) if wl.kivi_bits == 8 else 2 * krow
        work["rerotate"] = ("hbm", n_ctx * (src + 2 * q8row)
                            + (n_chunks * 8 * hkv * d if wl.kivi_bits else 0))
    elif wl.kivi_bits:
        # read K/V codes (bits / 8 B each) + V per-token stats (min, scale) +
        # K per-channel stats once per chunk; write bf16 K and V
        work["rerotate"] = ("hbm", n_ctx * (2 * hkv * d * wl.kivi_bits // 8 + 8 * hkv + 2 * krow)
                            + n_chunks * 8 * hkv * d)
    elif g.k_only:
        work["rerotate"] = ("hbm", n_ctx * 2 * krow)      # keys only: read K, write K
    else:
        work["rerotate"] = ("hbm", n_ctx * 4 * krow)      # gather: read pool K,V; write fused K,V
    if g.selector == "static":
        work["recompute"] = ("mfma", 2.0 * hid * d * (hq + 2 * hkv) * M)
    elif g.selector == "anchor":
        work["score"] = ("hbm", n_ctx * ((q8row if g.q8 else krow) + 4))   # fused K -> one fp32 norm
        work["recompute"] = ("mfma", 2.0 * hid * d * (hq + 2 * hkv) * M)
    elif g.mode == "deviation":
        work["k_probe"] = ("mfma", 2.0 * hid * hkv * d * total)
        if g.fuse_dev:
            # the re-positioning pass also reads the probe K and writes the score
            kind, nbytes = work["rerotate"]
            work["rerotate"] = (kind, nbytes + n_ctx * (krow + 4))
        else:
            work["score"] = ("hbm", n_ctx * ((q8row if g.q8 else krow) + krow + 4))   # fused K, probe K -> fp32
        work["recompute"] = ("mfma", 2.0 * hid * d * (hq + hkv) * M)
    else:
        work["u_probe"] = ("mfma", 2.0 * hid * d * (hq + hkv) * nU)    # Q and K of the query rows
        # (with g.fuse_mass the score call also re-positions the keys: its
        # bound stays the two MFMA passes)
        flops = 0.0
        for r in range(b.n_req):
            U = b.n_query(r)
            N = int(b.n_ctx[r])
            keys = sum(N + i + 1 for i in range(U))        # row statistics over the causal row
            flops += 2.0 * d * hq * keys + 2.0 * d * hq * U * N   # then Q K^T over the context
        work["score"] = ("mfma", flops)
        work["recompute"] = ("mfma", 2.0 * hid * d * (hq + 2 * hkv) * M)
    # scores in (none for static selection), forced mask in; picks, row ids
    # and positions out
    k_sum = int(sum(g.k_per_req))
    work["select"] = ("hbm", (0 if g.selector == "static" else n_ctx * 4)
                      + (n_ctx if g.static_mask is not None else 0) + k_sum * 4 + M * 8)
    if g.static_mask is not None:
        work["static_mask"] = ("hbm", n_ctx + b.chunk_table.shape[0] * 32)   # mask out, table in
    if g.q8:
        work["scatter"] = ("hbm", M * 2 * (krow + q8row))   # bf16 K, V rows in; codes + stats out
    elif g.probe:
        work["scatter"] = ("hbm", M * 2 * krow)       # probe K in; fused K rows out
    work["attention"] = ("mfma", 4.0 * d * hq * float((pos + 1).sum()))   # QK^T + PV, causal
    return work


FLUSH_BYTES = 1 << 30


def _flusher(write=False):
    """A 1 GiB buffer swept before every timed step, which evicts the step's
    working set from the L2 caches and the 256 MB Infinity Cache.  The sweep
    reads the buffer (a sum), so the lines it leaves behind are clean; with
    write=True it is a read-modify-write instead, which leaves hundreds of MB
    of dirty lines whose write-back then competes with the step's own reads
    (a 50 MB weight read takes about twice as long after it)."""
    import torch
    # float32: its sum is a single reduction over the buffer (an int32 sum
    # would first widen the whole buffer to int64, writing 2 GiB)
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    def flush():
        if write:
            buf.add_(1.0)
        else:
            buf.sum()
    return flush


def _pct(vals, q):
    import numpy as np
    return float(np.percentile(np.asarray(vals), q))


def _timed_steps(step, steps, flush=None):
    """Time `steps` passes one by one with HIP events on the launch stream,
    each after an untimed flush; returns per-step ms and the wall clock of
    the whole loop (synchronised on both sides)."""
    import torch
    pairs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if flush is not None:
            flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in pairs], wall


def _timed_back_to_back(step, steps):
    """Wall clock per step of `steps` passes back to back (warm caches)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def _graph_step(g):
    """The pass captured once as a HIP graph; returns its replay."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            g.step()
    torch.cuda.synchronize()
    return graph.replay


def _timed_per_call(g, steps, flush=None):
    """Average duration (ms) of every library call, HIP events on the
    current stream (the one the library launches on), each pass after an
    untimed flush."""
    import torch
    calls = g.calls()
    ev = {name: [] for name, _, _ in calls}
    torch.cuda.synchronize()
    for _ in range(steps):
        if flush is not None:
            flush()
        for name, _, fn in calls:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ev[name].append((e0, e1))
    torch.cuda.synchronize()
    return {n: sum(a.elapsed_time(b) for a, b in v) / len(v) for n, v in ev.items()}


def _source_hash(rel):
    h = hashlib.sha256()
    for f in (rel, "kvf_common.h"):
        with open(os.path.join(KDIR, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _traffic(kernel, src, workload):
    """HBM bytes per launch from profiles/<kernel>.<workload>.md, if its
    recorded source hash matches the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"^traffic_bytes_per_launch:\s*([0-9.eE+]+)\s*$", text, re.M)
    m_h = re.search(r"^source_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    if not (m_b and m_h) or m_h.group(1) != _source_hash(src):
        return None
    return float(m_b.group(1))


def _oracle_selection(batch, lo, pk, pv, fusion, selectors):
    """The oracle's selection for the static and anchor selectors."""
    import numpy as np
    wl = batch.wl
    sels = []
    if wl.selector == "static":
        for r in range(batch.n_req):
            spans = batch.chunk_spans(r)
            m = selectors.static_mask(int(batch.n_ctx[r]), [p for p, _ in spans], *wl.static_rules)
            sels.append(np.flatnonzero(m).astype(np.int32))
        return sels
    fk, _ = fusion.rerotate_stitch(pk, pv, batch.chunk_table, batch.total_rows, lo)
    for r in range(batch.n_req):
        spans = batch.chunk_spans(r)
        a = int(batch.cu_T[r])
        s = selectors.key_norm(fk[a:a + int(batch.n_ctx[r])])
        sels.append(selectors.select_topk_segmented(
            s, [p for p, _ in spans], [n for _, n in spans],
            [selectors.anchor_budget(n, wl.anchor_pct, 100) for _, n in spans]))
    return sels


def cpu_baseline(batch, ratio, min_seconds=10.0):
    """The float64 oracle on the same batch (one full pass of every stage of
    the layer), repeated until at least `min_seconds` of host time."""
    import numpy as np
    from oracle import fusion, selectors, storage
    wl = batch.wl
    lo = fusion.Layer(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.rope_base)
    x = storage.decode(batch.x, wl.dtype)
    w = storage.decode(batch.w_qkv, wl.dtype)
    # per-chunk caches, ahead of serving (not timed)
    pk, pv = fusion.pic_encode(storage.decode(batch.pool_hidden, wl.dtype), batch.pool_pos, w, lo)
    ks = [fusion.budget(int(n), ratio) for n in batch.n_ctx]
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    runs, t0 = 0, time.perf_counter()
    while True:
        if wl.selector == "score":
            fusion.fused_layer(x, w, pk, pv, batch.chunk_table, batch.cu_T, batch.n_ctx, lo,
                               wl.score, ks)
        else:
            sel = _oracle_selection(batch, lo, pk, pv, fusion, selectors)
            fusion.fused_layer(x, w, pk, pv, batch.chunk_table, batch.cu_T, batch.n_ctx, lo,
                               "none", [len(s) for s in sel], forced_sel=sel)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    n_ctx = int(np.sum(batch.n_ctx))
    return {"value": round(n_ctx * runs / dt, 1), "unit": UNIT, "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{runs} full pass(es) of the layer over the whole {wl.name} batch "
                      f"({batch.n_req} request(s), {n_ctx} context tokens), float64 numpy"}


def cpu_baseline_multilayer(batches, pcts, min_seconds=10.0):
    """The float64 oracle over every layer of a multi-layer pass (selection
    signal included), repeated until at least `min_seconds` of host time."""
    import numpy as np
    from oracle import fusion, multilayer, storage
    wl = batches[0].wl
    lo = fusion.Layer(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.rope_base)
    prep = []
    for b in batches:
        x = storage.decode(b.x, wl.dtype)
        w = storage.decode(b.w_qkv, wl.dtype)
        pk, pv = fusion.pic_encode(storage.decode(b.pool_hidden, wl.dtype), b.pool_pos, w, lo)
        prep.append((b, x, w, pk, pv))
    L = len(batches)

    def one_pass():
        def layer(l, mode, ks, sel=None):
            b, x, w, pk, pv = prep[l]
            return fusion.fused_layer(x, w, pk, pv, b.chunk_table, b.cu_T, b.n_ctx, lo, mode, ks,
                                      forced_sel=sel)
        n = [int(v) for v in batches[0].n_ctx]
        if wl.signal == "sum":
            ks = [fusion.budget(v, pcts[0]) for v in n]
            layers = list(wl.score_layers) or list(range(L))
            per = [layer(l, "attn_mass", ks)["scores"] for l in layers]
            sel = [fusion.select_topk(multilayer.layer_sum([p[r] for p in per]).astype(np.float32),
                                      ks[r]) for r in range(len(n))]
            for l in range(L):
                layer(l, "none", ks, sel)
        elif wl.signal == "progressive":
            cand = [None] * len(n)
            for l in range(L):
                ks = [fusion.budget(v, pcts[l]) for v in n]
                dev = layer(l, "deviation", ks)["scores"]
                sel = []
                for r in range(len(n)):
                    s = dev[r] if cand[r] is None else multilayer.restrict(dev[r], cand[r])
                    sel.append(fusion.select_topk(np.asarray(s, dtype=np.float32), ks[r]))
                    cand[r] = np.isin(np.arange(n[r]), sel[-1])
                layer(l, "deviation", ks, sel)
        else:
            for l in range(L):
                layer(l, wl.score, [fusion.budget(v, pcts[l]) for v in n])

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    runs, t0 = 0, time.perf_counter()
    while True:
        one_pass()
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    n_ctx = int(np.sum(batches[0].n_ctx))
    return {"value": round(n_ctx * L * runs / dt, 1), "unit": UNIT, "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{runs} full pass(es) over all {L} layers of the {wl.name} batch "
                      f"({len(batches[0].n_ctx)} request(s), {n_ctx} context tokens), float64 numpy"}


def multilayer_work(m):
    """(name, layer) -> algorithmic work of every call of one multi-layer pass."""
    out = {}
    for name, l, _ in m.calls():
        ly = m.layers[l]
        w = call_work(ly)
        if name == "k_probe" and l > 0:            # probe of the previous picks only
            wl = ly.wl
            w[name] = ("mfma", 2.0 * wl.hidden * wl.n_kv_heads * wl.head_dim * m.layers[l - 1].M)
        out[(name, l)] = w[name]
    return out


def _timed_calls_ml(m, steps):
    """Average duration (ms) of every (call, layer) of a multi-layer pass."""
    import torch
    torch.cuda.synchronize()
    acc = {}
    for _ in range(steps):
        m._begin_pass()
        evs = []
        for name, l, fn in m.calls():
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            evs.append(((name, l), e0, e1))
        torch.cuda.synchronize()
        for key, e0, e1 in evs:
            acc[key] = acc.get(key, 0.0) + e0.elapsed_time(e1)
    return {k: v / steps for k, v in acc.items()}


def _time_passes(fn, steps):
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def main_multilayer(args, wl, ratio):
    """Several layers per step: `value` is (sum N) x layers / step time."""
    import numpy as np
    import torch
    from rag_kv_cache_kvf_amd import synth
    from rag_kv_cache_kvf_amd.multilayer import MultiLayerGPU
    batches = synth.make_layer_batches(wl)
    m = MultiLayerGPU(batches, ratio)
    # a streamed pipeline's first passes run slower (about 5 ms instead of
    # 1.6 ms for 4 layers over the first eight passes): it gets 12 warm-up
    # passes at least
    warmup = max(args.warmup, 12 if m.stream_pools else 1)
    for _ in range(warmup):
        m.run()
    torch.cuda.synchronize()
    sec = _time_passes(m.run, args.steps)
    pipeline = None
    if m.stream_pools:
        # the same layers with the caches resident, and the copies alone; the
        # per-call kernel times below are taken resident, so that a
        # re-position call does not include its wait for the copy
        copy_s = _time_passes(m.run_copies_only, args.steps)
        m.set_streaming(False)
        for _ in range(3):
            m.run()
        resident = _time_passes(m.run, args.steps)
        nbytes = m.cache_bytes()
        pipeline = {
            "streamed_ms": round(sec * 1e3, 4), "resident_ms": round(resident * 1e3, 4),
            "copies_ms": round(copy_s * 1e3, 4), "cache_bytes_per_pass": nbytes,
            "bound": "host link", "achieved_GBps": round(nbytes / sec / 1e9, 2),
            "copy_only_GBps": round(nbytes / copy_s / 1e9, 2),
            "peak_GBps": PEAK["pcie"],
            "frac": round(nbytes / sec / 1e9 / PEAK["pcie"], 4),
            "hidden_fraction": round(max(0.0, resident + copy_s - sec) / min(resident, copy_s), 4)}
    per = _timed_calls_ml(m, args.steps)
    work = multilayer_work(m)
    n_ctx = int(np.sum(batches[0].n_ctx))
    L = m.n_layers
    peak_mfma = PEAK["bf16"] if wl.dtype == "bf16" else PEAK["f32"]
    # per call name: summed over layers
    by_name = {}
    for (name, l), ms in per.items():
        kind, amount = work[(name, l)]
        t = by_name.setdefault(name, {"ms": 0.0, "kind": kind, "amount": 0.0, "layers": 0})
        t["ms"] += ms
        t["amount"] += amount
        t["layers"] += 1
    calls = {}
    for name, t in by_name.items():
        ms = t["ms"]
        if t["kind"] == "hbm":
            ach, peak, unit = t["amount"] / (ms * 1e-3) / 1e9, PEAK["hbm"], "GB/s"
        else:
            ach, peak, unit = t["amount"] / (ms * 1e-3) / 1e12, peak_mfma, "TFLOP/s"
        calls[name] = {"ms_all_layers": round(ms, 5), "launches": t["layers"], "bound": t["kind"],
                       "achieved": round(ach, 2), "unit": unit, "frac": round(ach / peak, 4)}
    dom = max(by_name, key=lambda n: by_name[n]["ms"])
    kname, ksrc = CALL_KERNEL[dom]
    if dom == "score" and wl.score == "deviation":
        kname, ksrc = "deviation_kernel", "kernels/scatter_deviation.hip"
    c = calls[dom]
    t = by_name[dom]
    roofline = {"kernel": kname, "call": dom, "bound": t["kind"], "achieved": c["achieved"],
                "peak": PEAK["hbm"] if t["kind"] == "hbm" else peak_mfma, "unit": c["unit"],
                "frac": c["frac"], "avg_ms": round(t["ms"] / t["layers"], 5),
                "algorithmic_per_launch": t["amount"] / t["layers"],
                "traffic": _traffic(kname, ksrc, wl.name)}
    out = {
        "metric": METRIC,
        "value": round(n_ctx * L / sec, 1),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description,
                   "requests": batches[0].n_req, "context_tokens": n_ctx, "layers": L,
                   "query_tokens": batches[0].total_rows - n_ctx, "signal": wl.signal or "per-layer",
                   "score": wl.score, "recompute_ratio_pct": m.pcts,
                   "score_layers": getattr(m, "score_layers", None),
                   "streamed_caches": bool(wl.stream_pools)},
        "roofline": roofline,
        "calls": calls,
    }
    if pipeline is not None:
        out["pipeline"] = pipeline
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_multilayer(batches, m.pcts)
    print(json.dumps(out), flush=True)


def copy_calibration():
    """A plain 1 GiB device-to-device copy, three times: the HBM byte
    counters read for it scale the counters of the kernels."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 3
    print(json.dumps({"copy_bytes": n, "copies": 3, "read_bytes": n, "write_bytes": n,
                      "GBps_read_plus_write": round(2 * n / dt / 1e9, 1)}), flush=True)


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the fused layer is "
              "built and measured for a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    from rag_kv_cache_kvf_amd import synth

    wl = synth.get_workload(args.workload)
    ratio = args.ratio if args.ratio is not None else wl.ratio_pct[-1]
    if wl.n_layers > 1:
        main_multilayer(args, wl, ratio)
        return
    flush = _flusher()
    head, batch, g = measure(wl, ratio, args.steps, args.warmup, flush, graph=args.graph,
                             fuse=not args.unfused, fuse_mass=args.fuse_mass)
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": head["config"],
        "timing": head["timing"],
        "roofline": head["roofline"],
        "calls": head["calls"],
    }
    if not args.no_extra and wl.name == DEFAULT_WORKLOAD:
        # the 8-request pool workload at both of its ratios (same layer shape)
        del g
        import torch
        torch.cuda.empty_cache()
        extra = synth.get_workload(EXTRA_WORKLOAD)
        for pct in extra.ratio_pct[::-1]:
            sub, _, gx = measure(extra, pct, args.steps, args.warmup, flush, fuse=not args.unfused)
            out[f"{EXTRA_WORKLOAD}@{pct}"] = {k: sub[k] for k in
                                               ("value", "unit", "ms_per_step", "config", "timing",
                                                "roofline", "calls")}
            del gx
            torch.cuda.empty_cache()
        # the int8 KIVI layer with a bf16 fused cache and with an int8-resident one
        for name in Q8_WORKLOADS:
            qwl = synth.get_workload(name)
            sub, _, gx = measure(qwl, qwl.ratio_pct[-1], args.steps, args.warmup, flush,
                                 fuse=not args.unfused)
            out[name] = {k: sub[k] for k in ("value", "unit", "ms_per_step", "config", "timing",
                                             "roofline", "calls")}
            del gx
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(batch, ratio)
    print(json.dumps(out), flush=True)


def measure(wl, ratio, steps, warmup, flush, graph=False, fuse=True, fuse_mass=False):
    """One single-layer workload: flushed per-step times, back-to-back time,
    per-call durations and the roofline of the longest call."""
    import numpy as np
    import torch
    from rag_kv_cache_kvf_amd import synth
    from rag_kv_cache_kvf_amd.layer import FusedLayerGPU

    batch = synth.make_batch(wl)
    g = FusedLayerGPU(batch, ratio, fuse_score=fuse, fuse_mass=fuse_mass)
    g.load()                              # the loader's stitch, ahead of the passes
    step = _graph_step(g) if graph else g.step
    for _ in range(max(warmup, 1)):
        step()
    torch.cuda.synchronize()

    times, wall = _timed_steps(step, steps, flush)
    times_dirty, _ = _timed_steps(step, steps, _flusher(write=True))
    warm = _timed_back_to_back(step, steps)
    per_call = _timed_per_call(g, steps, flush)
    per_call_warm = _timed_per_call(g, steps, None)
    work = call_work(g)
    n_ctx = int(np.sum(batch.n_ctx))
    med = _pct(times, 50)

    peak_mfma = PEAK["bf16"] if wl.dtype == "bf16" else PEAK["f32"]
    calls = {}
    for name, ms in per_call.items():
        kind, amount = work[name]
        if kind == "hbm":
            ach, peak, unit = amount / (ms * 1e-3) / 1e9, PEAK["hbm"], "GB/s"
        else:
            ach, peak, unit = amount / (ms * 1e-3) / 1e12, peak_mfma, "TFLOP/s"
        calls[name] = {"ms": round(ms, 5), "bound": kind, "achieved": round(ach, 2),
                       "unit": unit, "frac": round(ach / peak, 4),
                       "algorithmic": float(amount), "ms_warm": round(per_call_warm[name], 5)}
    dom = max(per_call, key=per_call.get)
    kname, ksrc = (CALL_KERNEL_Q8 if g.q8 and dom in CALL_KERNEL_Q8 else CALL_KERNEL)[dom]
    if dom == "score" and g.selector == "anchor":
        kname, ksrc = "key_norm_kernel", "kernels/scatter_deviation.hip"
    elif dom == "score" and g.mode == "deviation":
        kname, ksrc = "deviation_kernel", "kernels/scatter_deviation.hip"
    if dom == "select" and g.selector == "anchor":
        kname = "topk_segmented_kernel"
    kind, amount = work[dom]
    c = calls[dom]
    roofline = {"kernel": kname, "call": dom, "bound": kind, "achieved": c["achieved"],
                "peak": PEAK["hbm"] if kind == "hbm" else peak_mfma, "unit": c["unit"],
                "frac": c["frac"], "avg_ms": c["ms"], "algorithmic_per_launch": float(amount),
                "traffic": _traffic(kname, ksrc, wl.name)}
    timing = {"protocol": f"{steps} steps timed one by one with HIP events on the launch stream, "
                          f"each after an untimed read of {FLUSH_BYTES >> 30} GiB "
                          "(evicts L2 and the Infinity Cache, leaves clean lines); "
                          "value = context tokens / median",
              "ms_median": round(med, 5), "ms_p10": round(_pct(times, 10), 5),
              "ms_p90": round(_pct(times, 90), 5), "flush_bytes": FLUSH_BYTES,
              "ms_median_after_write_flush": round(_pct(times_dirty, 50), 5),
              "loop_wall_s": round(wall, 4),
              "ms_per_step_back_to_back": round(warm * 1e3, 5),
              "graph": bool(graph)}
    config = {"workload": wl.name, "description": wl.description, "requests": batch.n_req,
              "context_tokens": n_ctx, "query_tokens": batch.total_rows - n_ctx,
              "recompute_ratio_pct": ratio if wl.selector == "score" else None,
              "selector": wl.selector,
              "score": g.mode if wl.selector == "score" else
              ("key_norm" if wl.selector == "anchor" else None),
              "recomputed_context_tokens": int(sum(g.k_per_req)),
              "rerotate": "keys only (values stitched by the loader)" if g.k_only else
              ("KIVI decode" if wl.kivi_bits else "gather keys and values") +
              (", int8-resident fused cache (8-bit codes + per-row min/scale)" if g.q8 else
               ", bf16 fused cache") +
              (", deviation score in the same pass" if g.fuse_dev else "") +
              (", keys re-positioned inside the attention-mass score's first pass" if g.fuse_mass else "")}
    res = {"value": round(n_ctx / (med * 1e-3), 1), "unit": UNIT, "ms_per_step": round(med, 5),
           "ms_median": round(med, 5), "config": config, "timing": timing, "roofline": roofline,
           "calls": calls}
    return res, batch, g


if __name__ == "__main__":
    main()
