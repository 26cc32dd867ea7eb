"""End-to-end parity at the full workload sizes (GPU): the whole call chain
of one fused layer on each workload's own seeded data, against the float64
oracle at the serving precision.

Per workload:
  * scores: every context position, max|d| / rms within the bf16 tolerance;
  * selection: bit-exact against the oracle's TopK of the GPU's own fp32
    scores, and every position where it differs from the oracle's selection
    lies within 2 max|d| of the oracle's k-th score (the most a top-k can
    move when no score moves by more than max|d|);
  * with the oracle's selection forced into the GPU path: the recomputed row
    list bit-exact, the fused cache and the queries (against the exact
    float64 layer), and the attention output and LSE of the recomputed rows - every row for the 8B-shaped mass workload and
    the int8 workload, sampled rows (the oracle computes their queries and
    attention one by one) for the 8-request pool workload and the 70B-shaped
    layer.
The per-chunk caches are the oracle's, stored in the workload's format.
"""
import functools

import numpy as np
import pytest

from oracle import fusion
from rag_kv_cache_kvf_amd import synth
from tests.gpu_util import assert_close, assert_close_vectors, check_selection, from_gpu, raw
from tests.test_gpu_layer import _oracle_inputs

pytestmark = pytest.mark.gpu

# (workload, recompute ratio in percent, rows compared after the forced selection)
FULL = [("qwen3_8b_mass", 30, "all"), ("qwen25_3b_kivi8", 15, "all"),
        ("qwen3_8b_dev_pool", 30, "sampled"), ("qwen3_8b_dev_pool", 15, "sampled"),
        ("llama3_70b_mass", 20, "sampled")]


@pytest.fixture(scope="module")
def layer_mod():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from rag_kv_cache_kvf_amd import layer
    return layer


@functools.lru_cache(maxsize=1)
def _inputs(name):
    # one workload's batch and oracle-built per-chunk caches (both ratios of
    # the pool workload share them)
    return _oracle_inputs(name)


def _sample(m, n, seed):
    """n of m row indices, always the first and the last."""
    if m <= n:
        return np.arange(m)
    return np.unique(np.concatenate([synth.random_rows(m, n, seed), [0, m - 1]]))


@pytest.mark.parametrize("name,pct,rows", FULL, ids=[f"{n}@{p}" for n, p, _ in FULL])
def test_full_size_layer(layer_mod, name, pct, rows):
    import torch
    print(f"[case] full-size layer {name} at {pct}%", flush=True)
    b, wl, lo, x, w, pic, opk, opv, _, _ = _inputs(name)
    ks = [fusion.budget(int(n), pct) for n in b.n_ctx]
    g = layer_mod.FusedLayerGPU(b, pct, pic=pic)
    g.run()
    torch.cuda.synchronize()
    gs = from_gpu(g.scores)[: int(np.sum(b.n_ctx))]
    sel_gpu = g.selection()

    U = [b.n_query(r) for r in range(b.n_req)]
    attend = None
    if rows == "sampled":
        attend = [_sample(ks[r] + U[r], 24, 40 + r) for r in range(b.n_req)]
    ref = fusion.fused_layer(x, w, opk, opv, b.chunk_table, b.cu_T, b.n_ctx, lo, wl.score, ks,
                             store=wl.dtype, attend=attend)
    rs = np.concatenate(ref["scores"])
    assert_close(gs, rs, wl.dtype, f"{name}@{pct} scores ({len(rs)} positions)")
    check_selection(f"{name}@{pct}", sel_gpu, gs, rs, ks, b.n_ctx)

    # the rest of the layer on the oracle's selection
    g.run(forced_sel=ref["sel"])
    torch.cuda.synchronize()
    assert np.array_equal(raw(g.rows)[: g.M], ref["rows"])
    assert np.array_equal(raw(g.pos)[: g.M], ref["pos"])
    if rows == "all":
        crow = np.arange(b.total_rows)
    else:
        # every recomputed row plus a sample of the re-positioned ones
        crow = np.unique(np.concatenate([ref["rows"], synth.random_rows(b.total_rows, 8192, 41)]))
    # cache entries and queries: the exact float64 layer on the same
    # selection (the GPU's are one bf16 rounding of an fp32 sum from it)
    exact = fusion.fused_layer(x, w, opk, opv, b.chunk_table, b.cu_T, b.n_ctx, lo, wl.score, ks,
                               forced_sel=ref["sel"], attend=attend)
    gk = from_gpu(g.fused_k[torch.from_numpy(crow).cuda()])
    gv = from_gpu(g.fused_v[torch.from_numpy(crow).cuda()])
    assert_close(gk, exact["fused_k"][crow], wl.dtype, f"{name}@{pct} fused K ({len(crow)} rows)")
    assert_close(gv, exact["fused_v"][crow], wl.dtype, f"{name}@{pct} fused V ({len(crow)} rows)")
    flat = ref["attend_flat"]
    sel_t = torch.from_numpy(flat).cuda()
    assert_close(from_gpu(g.q[sel_t]), exact["q"], wl.dtype, f"{name}@{pct} recomputed Q ({len(flat)} rows)")
    assert_close_vectors(from_gpu(g.out[sel_t]), ref["out"], wl.dtype,
                         f"{name}@{pct} attention output ({len(flat)} rows)")
    assert_close(from_gpu(g.lse[sel_t]), ref["lse"], wl.dtype, f"{name}@{pct} lse", tol=1e-3)
