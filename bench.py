"""Benchmark of one fused RAG KV-cache layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--graph]

A step is one pass of the whole hot path over one batch of synthetic input:
re-position/stitch -> score -> top-k -> Q/K/V recompute -> scatter ->
sparse-query attention (the attention-mass path for the default workload).
Inputs, weights and the per-chunk caches are resident in HBM before timing
starts (the caches are built by the library's own projection at chunk-local
positions, ahead of the timed region).  The metric is fused context tokens per
second per layer: (sum over requests of N) / step time.

Prints one JSON line.  Each library call of a step is bracketed with HIP
events on the stream it is launched on; the dominant kernel's average
duration over the timed steps gives the roofline fraction.  The CPU baseline
runs the float64 oracle on the same workload (one full pass) on the host.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "qwen3_8b_mass"
PEAK = {"hbm_gbs": 8000.0, "bf16_tflops": 2500.0, "fp32_tflops": 157.3}


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--ratio", type=int, default=None, help="recompute ratio in percent")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay the step as one HIP graph")
    return ap.parse_args()


def stage_work(g):
    """Algorithmic work of every stage of one step (flops or bytes)."""
    wl = g.wl
    b = g.batch
    hq, hkv, d, hid = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.hidden
    esz = 2 if wl.dtype == "bf16" else 4
    krow = hkv * d * esz
    n_ctx = int(sum(b.n_ctx))
    total = b.total_rows
    nU = total - n_ctx
    M = g.M
    pos = g.pos.cpu().numpy()[:M].astype("int64")
    work = {}
    if wl.kivi8:
        # codes K + V, V stats (8 B per head per token), K stats amortised per chunk
        n_chunks = b.chunk_table.shape[0]
        s1 = n_ctx * (2 * hkv * d + 8 * hkv + 2 * krow) + n_chunks * 8 * hkv * d
    else:
        s1 = n_ctx * 4 * krow                       # read K,V from the pool, write K,V
    work["rerotate"] = ("hbm", s1)
    if g.mode == "deviation":
        work["k_probe"] = ("mfma", 2.0 * hid * hkv * d * total)
        work["score"] = ("hbm", n_ctx * (2 * krow + 4))
        work["recompute"] = ("mfma", 2.0 * hid * d * (hq + hkv) * M)
    else:
        G = hq // hkv
        work["u_probe"] = ("mfma", 2.0 * hid * d * (hq + 2 * hkv) * nU)
        work["u_scatter"] = ("hbm", nU * 4 * krow)
        flops = 0.0
        for r in range(b.n_req):
            U = b.n_query(r)
            N = int(b.n_ctx[r])
            keys = sum(N + i + 1 for i in range(U))        # pass 1 (statistics)
            flops += 2.0 * d * hq * keys + 2.0 * d * hq * U * N   # pass 2 (context keys)
        work["score"] = ("mfma", flops)
        work["recompute"] = ("mfma", 2.0 * hid * d * (hq + 2 * hkv) * M)
    work["select"] = ("hbm", n_ctx * 4 + M * 8)
    work["scatter"] = ("hbm", M * 4 * krow)
    work["attention"] = ("mfma", 4.0 * d * hq * float((pos + 1).sum()))
    return work


def run_steps(g, steps, use_graph):
    """Run `steps` steps; with events around every library call."""
    import torch
    names = ["rerotate", "score_all", "select", "recompute_fuse", "attention"]
    ev = {n: [] for n in names}

    def one_step(record):
        def bracket(name, fn):
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                ev[name].append((e0, e1))
            else:
                fn()
        bracket("rerotate", g.stage_rerotate)
        bracket("score_all", g.stage_score)
        bracket("select", g.stage_select)
        bracket("recompute_fuse", g.stage_recompute_fuse)
        bracket("attention", g.stage_attention)

    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            one_step(False)
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=s):
                one_step(False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) / steps, None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = {n: sum(a.elapsed_time(b) for a, b in v) / max(1, len(v)) for n, v in ev.items()}
    return (t1 - t0) / steps, per


def kernel_times(g, steps):
    """Per-kernel average durations (ms) of the dominant-kernel candidates,
    with HIP events on the launch stream, over `steps` steps."""
    import torch
    from rag_kv_cache_kvf_amd import kvfuse as kvf
    L = g.layer
    res = {"recompute": [], "attention": []}
    for _ in range(steps):
        g.stage_rerotate()
        g.stage_score()
        g.stage_select()
        e0, e1, e2, e3 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
        if g.mode == "deviation":
            e0.record()
            kvf.recompute_qkv(L, g.x, g.rows, g.pos, g.w, kvf.KVF_OUT_Q | kvf.KVF_OUT_V, g.rope_cos,
                              g.rope_sin, q_out=g.q, v_out=g.v_new, M=g.M)
            e1.record()
            kvf.scatter_kv(L, g.k_probe, g.rows, g.v_new, None, g.rows, g.fused_k, g.fused_v, M=g.M)
        else:
            e0.record()
            kvf.recompute_qkv(L, g.x, g.rows, g.pos, g.w, kvf.KVF_OUT_Q | kvf.KVF_OUT_K | kvf.KVF_OUT_V,
                              g.rope_cos, g.rope_sin, q_out=g.q, k_out=g.k_new, v_out=g.v_new, M=g.M)
            e1.record()
            kvf.scatter_kv(L, g.k_new, None, g.v_new, None, g.rows, g.fused_k, g.fused_v, M=g.M)
        e2.record()
        g.stage_attention()
        e3.record()
        res["recompute"].append((e0, e1))
        res["attention"].append((e2, e3))
    torch.cuda.synchronize()
    return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in res.items()}


def cpu_baseline(batch, ratio):
    """The float64 oracle on the same workload: one full pass (every stage of
    the layer), timed on the host cores."""
    import numpy as np
    from oracle import fusion, storage
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
    t0 = time.perf_counter()
    fusion.fused_layer(x, w, pk, pv, batch.chunk_table, batch.cu_T, batch.n_ctx, lo, wl.score, ks)
    dt = time.perf_counter() - t0
    n_ctx = int(np.sum(batch.n_ctx))
    return {"value": n_ctx / dt, "unit": "fused context tokens/s per layer", "cores": int(threads),
            "kind": "oracle", "seconds": dt,
            "sample": f"one full pass of the layer over the whole {wl.name} batch "
                      f"({batch.n_req} request(s), {n_ctx} context tokens), float64 numpy"}


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the fused layer is "
              "built and measured for a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from rag_kv_cache_kvf_amd import synth
    from rag_kv_cache_kvf_amd.layer import FusedLayerGPU

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = synth.get_workload(args.workload)
    ratio = args.ratio if args.ratio is not None else wl.ratio_pct[-1]
    batch = synth.make_batch(wl)
    g = FusedLayerGPU(batch, ratio)
    for _ in range(max(args.warmup, 1)):
        g.run()
    torch.cuda.synchronize()

    sec, per_stage = run_steps(g, args.steps, args.graph)
    kt = kernel_times(g, max(5, min(args.steps, 20)))
    work = stage_work(g)
    n_ctx = int(np.sum(batch.n_ctx))
    value = n_ctx / sec

    # dominant kernel: the larger of the projection and attention kernels
    dom = max(kt, key=kt.get)
    kind, amount = work[dom]
    achieved = amount / (kt[dom] * 1e-3) / 1e12
    roofline = {"kernel": "gemm_qkv_bf16_kernel" if dom == "recompute" else "attn_bf16_kernel",
                "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK["bf16_tflops"] if wl.dtype == "bf16" else PEAK["fp32_tflops"],
                "unit": "TFLOP/s", "avg_ms": round(kt[dom], 5), "traffic": None}
    roofline["frac"] = round(roofline["achieved"] / roofline["peak"], 4)

    stages = {}
    if per_stage:
        for k, v in per_stage.items():
            stages[k] = {"ms": round(v, 5)}
    for k, v in kt.items():
        stages.setdefault(f"{k}_kernel", {})["ms"] = round(v, 5)
        kk, amt = work[k]
        stages[f"{k}_kernel"]["tflops"] = round(amt / (v * 1e-3) / 1e12, 2)

    out = {
        "metric": "fused context tokens/s per layer @r=30% on 1 MI355X; % MFMA/HBM roofline",
        "value": round(value, 1),
        "unit": "fused context tokens/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "requests": batch.n_req,
                   "context_tokens": n_ctx, "query_tokens": batch.total_rows - n_ctx,
                   "recompute_ratio_pct": ratio, "score": g.mode, "graph": bool(args.graph)},
        "roofline": roofline,
        "stages": stages,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(batch, ratio)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
