"""End-to-end parity of the fused layer (all six calls in order) against the
oracle, plus determinism and HIP-graph replay (GPU).

Inputs: the seeded synthetic batch; the per-chunk caches are built by the
oracle in float64 and stored in the workload's format (bf16 / fp32 / int8
KIVI), then fed to both sides.  Checks:
  * scores: max|d| / rms within the dtype tolerance;
  * the GPU's selection is bit for bit the TopK of its own fp32 scores, and
    it differs from the oracle's only where the score error can reorder;
  * with the oracle's selection forced into the GPU path, the fused cache,
    the attention output and its LSE match the oracle.
"""
import numpy as np
import pytest

from oracle import fusion, kivi, selectors
from rag_kv_cache_kvf_amd import synth
from tests.gpu_util import (TOL, assert_close, assert_close_vectors, check_selection, decode, encode,
                             from_gpu, raw, rel_err_vectors)

pytestmark = pytest.mark.gpu

E2E = ["tiny_fp32_dev", "mini_bf16_mass", "mini_bf16_dev_pool", "mini_bf16_kivi8", "mini_bf16_kivi4",
       "mini_bf16_d64_mass", "mini_f32_mass"]


@pytest.fixture(scope="module")
def layer_mod():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from rag_kv_cache_kvf_amd import layer
    return layer


def _oracle_inputs(name, pct=None):
    b = synth.make_batch(name)
    wl = b.wl
    lo = fusion.Layer(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.rope_base)
    x = decode(b.x, wl.dtype)
    w = decode(b.w_qkv, wl.dtype)
    pk, pv = fusion.pic_encode(decode(b.pool_hidden, wl.dtype), b.pool_pos, w, lo)
    if wl.kivi_bits:
        bits = wl.kivi_bits
        pk32 = decode(encode(pk, "bf16"), "bf16").astype(np.float32)
        pv32 = decode(encode(pv, "bf16"), "bf16").astype(np.float32)
        kc, kmin, ksc = kivi.encode_keys(pk32, b.pool_cu, bits=bits)
        vc, vmin, vsc = kivi.encode_values(pv32, bits=bits)
        store = kivi.pack4 if bits == 4 else (lambda c: c)
        pic = {"k_codes": store(kc), "v_codes": store(vc), "k_min": kmin, "k_scale": ksc,
               "v_min": vmin, "v_scale": vsc}
        opk = kivi.decode_keys(kc, kmin, ksc, b.pool_cu)
        opv = kivi.decode_values(vc, vmin, vsc)
    else:
        pic = {"k": encode(pk, wl.dtype), "v": encode(pv, wl.dtype)}
        opk, opv = decode(pic["k"], wl.dtype), decode(pic["v"], wl.dtype)
    pct = pct if pct is not None else wl.ratio_pct[0]
    ks = [fusion.budget(int(n), pct) for n in b.n_ctx]
    return b, wl, lo, x, w, pic, opk, opv, pct, ks


def _check_selection_valid(sel_gpu, scores_ref, tol_abs, what):
    """Every selected score is at least every unselected one, up to tol_abs."""
    n = len(scores_ref)
    mask = np.zeros(n, dtype=bool)
    mask[sel_gpu] = True
    if mask.all() or not mask.any():
        return
    lo_sel = scores_ref[mask].min()
    hi_uns = scores_ref[~mask].max()
    print(f"[parity] {what}: min selected {lo_sel:.6g}, max unselected {hi_uns:.6g}", flush=True)
    assert lo_sel >= hi_uns - tol_abs, f"{what}: selection is not a top-k of the oracle scores"


@pytest.mark.parametrize("name", E2E)
def test_fused_layer_end_to_end(layer_mod, name):
    import torch
    b, wl, lo, x, w, pic, opk, opv, pct, ks = _oracle_inputs(name)
    print(f"[case] {name}", flush=True)
    g = layer_mod.FusedLayerGPU(b, pct, pic=pic)
    g.run()
    torch.cuda.synchronize()
    # scores and attention outputs: the oracle at the serving precision of the
    # workload (bf16 / fp32 tensors rounded where they are materialised)
    ref = fusion.fused_layer(x, w, opk, opv, b.chunk_table, b.cu_T, b.n_ctx, lo, wl.score, ks,
                             store=wl.dtype)
    # cache entries: the exact float64 layer, same selection
    exact = fusion.fused_layer(x, w, opk, opv, b.chunk_table, b.cu_T, b.n_ctx, lo, wl.score, ks,
                               forced_sel=ref["sel"])
    gs = from_gpu(g.scores)[: int(np.sum(b.n_ctx))]
    rs = np.concatenate(ref["scores"])
    assert_close(gs, rs, wl.dtype, f"{name} scores")
    sel = g.selection()
    for r in range(b.n_req):
        assert len(sel[r]) == ks[r] and np.all(np.diff(sel[r]) > 0)
    check_selection(name, sel, gs, rs, ks, b.n_ctx)

    # downstream with the oracle's selection
    g.run(forced_sel=ref["sel"])
    torch.cuda.synchronize()
    assert np.array_equal(raw(g.rows)[: g.M], ref["rows"])
    assert_close(from_gpu(g.fused_k), exact["fused_k"], wl.dtype, f"{name} fused K")
    assert_close(from_gpu(g.fused_v), exact["fused_v"], wl.dtype, f"{name} fused V")
    assert_close(from_gpu(g.q)[: g.M], exact["q"], wl.dtype, f"{name} recomputed Q")
    go = from_gpu(g.out)[: g.M]
    row_err = np.abs(go - ref["out"]).max(axis=(1, 2))
    worst = np.argsort(row_err)[::-1][:5]
    print(f"[diag] {name}: worst rows {worst.tolist()} pos {ref['pos'][worst].tolist()} "
          f"err {row_err[worst].tolist()}", flush=True)
    assert_close_vectors(go, ref["out"], wl.dtype, f"{name} attention output")
    assert_close(from_gpu(g.lse)[: g.M], ref["lse"], wl.dtype, f"{name} lse",
                 tol=1e-3 if wl.dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("name,pct", [("mini_bf16_mass", 0), ("mini_bf16_mass", 100),
                                      ("mini_bf16_dev_pool", 0), ("mini_bf16_dev_pool", 100)])
def test_ratio_endpoints(layer_mod, name, pct):
    """rho = 0 (direct reuse) and rho = 100% (every context token recomputed)."""
    import torch
    b, wl, lo, x, w, pic, opk, opv, pct, ks = _oracle_inputs(name, pct)
    g = layer_mod.FusedLayerGPU(b, pct, pic=pic)
    g.run()
    torch.cuda.synchronize()
    ref = fusion.fused_layer(x, w, opk, opv, b.chunk_table, b.cu_T, b.n_ctx, lo, wl.score, ks,
                             store=wl.dtype)
    exact = fusion.fused_layer(x, w, opk, opv, b.chunk_table, b.cu_T, b.n_ctx, lo, wl.score, ks)
    assert np.array_equal(raw(g.rows)[: g.M], ref["rows"])
    assert_close(from_gpu(g.fused_k), exact["fused_k"], wl.dtype, f"{name}@{pct} fused K")
    assert_close_vectors(from_gpu(g.out)[: g.M], ref["out"], wl.dtype, f"{name}@{pct} output")
    if pct == 100:
        # rho = 100% is full prefill ([QCF] 4.1: the full-recompute endpoint).
        # The GPU output is held to the exact float64 prefill by the triangle
        # inequality: its distance to the serving-precision oracle (within TOL
        # per vector, asserted above) plus the oracle's own serving-vs-exact
        # distance, both relative to the exact vector's RMS.
        full = fusion.full_prefill(x, w, b.cu_T, lo)
        assert_close(from_gpu(g.fused_k), full["k"], wl.dtype, f"{name} rho=1 vs full prefill K")
        assert_close(from_gpu(g.fused_v), full["v"], wl.dtype, f"{name} rho=1 vs full prefill V")
        go = from_gpu(g.out)[: g.M]
        assert np.array_equal(ref["pos"], np.concatenate(
            [np.arange(b.cu_T[r + 1] - b.cu_T[r]) for r in range(b.n_req)]))
        xs = full["out"].reshape(-1, full["out"].shape[-1])
        ss = ref["out"].reshape(-1, xs.shape[-1])
        ratio = float(np.max(np.sqrt(np.mean(ss * ss, axis=1)) /
                             np.maximum(np.sqrt(np.mean(xs * xs, axis=1)), 1e-30)))
        e_serving = rel_err_vectors(ref["out"], full["out"])
        bound = TOL[wl.dtype] * ratio + e_serving
        e = rel_err_vectors(go, full["out"])
        print(f"[parity] {name} rho=1 output vs exact full prefill: {e:.3e} (bound {bound:.3e} = "
              f"{TOL[wl.dtype]:.0e} x {ratio:.4f} + serving-vs-exact {e_serving:.3e})", flush=True)
        assert e <= bound, f"rho=1 output differs from full prefill by {e:.3e} > {bound:.3e}"


def test_deterministic_and_graph_replay(layer_mod):
    import torch
    b, wl, lo, x, w, pic, opk, opv, pct, ks = _oracle_inputs("mini_bf16_mass")
    g = layer_mod.FusedLayerGPU(b, pct, pic=pic)
    g.run()
    torch.cuda.synchronize()
    first = {k: raw(getattr(g, k)).copy() for k in ("scores", "sel", "fused_k", "fused_v", "out", "lse")}
    g.run()
    torch.cuda.synchronize()
    for k, v in first.items():
        assert np.array_equal(raw(getattr(g, k)), v), f"{k} differs between runs"
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.run()                       # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            g.run()
    torch.cuda.synchronize()
    for rep in range(3):
        g.out.zero_()
        g.fused_k.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in first.items():
            assert np.array_equal(raw(getattr(g, k)), v), f"replay {rep}: {k} differs"


@pytest.mark.parametrize("name", ["mini_bf16_mass", "mini_bf16_dev_pool", "mini_bf16_kivi8"])
def test_fused_score_passes_match_separate_calls(layer_mod, name):
    """The re-positioning pass that also scores (deviation: kvf_rerotate_
    deviation; attention mass: kvf_rerotate_score_attn_mass) against the two
    separate calls through the whole layer: attention mass bit for bit
    everywhere (the same keys and arithmetic); deviation with the same
    fused caches, scores within fp32 summation order, and everything after
    the selection bit for bit when both take the same selection."""
    import torch
    b, wl, lo, x, w, pic, opk, opv, pct, ks = _oracle_inputs(name)
    fields = ("scores", "sel", "fused_k", "fused_v", "out", "lse")
    res = []
    for fused in (True, False):
        g = layer_mod.FusedLayerGPU(b, pct, pic=pic, fuse_score=fused, fuse_mass=fused)
        assert (g.fuse_mass if g.mass else g.fuse_dev) == fused
        g.run()
        torch.cuda.synchronize()
        res.append({k: raw(getattr(g, k)).copy() for k in fields})
    a, c = res
    if wl.score != "deviation":
        for k in fields:
            assert np.array_equal(a[k], c[k]), f"{k} differs"
        return
    assert np.max(np.abs(a["scores"].astype(np.float64) - c["scores"])) < 2e-6
    if np.array_equal(a["sel"], c["sel"]):
        for k in ("fused_k", "fused_v", "out", "lse"):
            assert np.array_equal(a[k], c[k]), f"{k} differs"


# ----------------------------------------------------------------------------
# other selectors feeding the same path
# ----------------------------------------------------------------------------
SEL_E2E = ["mini_bf16_seam", "mini_bf16_anchor", "mini_bf16_dev_sink"]


def _static_masks(b, wl):
    return [selectors.static_mask(int(b.n_ctx[r]), [p for p, _ in b.chunk_spans(r)],
                                  *wl.static_rules) for r in range(b.n_req)]


@pytest.mark.parametrize("name", SEL_E2E)
def test_selector_end_to_end(layer_mod, name):
    """Static selection (KVBoost sections 4.1 and 4.6.1, EPIC's boundary
    tokens), per-chunk key-norm anchors (QCFuse section 3.3.1, Eq. 14) and a
    deviation score with a forced static set, each through the whole layer:
    the selection against the oracle's (bit-exact where no floating point
    decides it), then the fused cache and attention with the oracle's
    selection forced in."""
    import torch
    b, wl, lo, x, w, pic, opk, opv, pct, ks = _oracle_inputs(name)
    print(f"[case] {name}", flush=True)
    g = layer_mod.FusedLayerGPU(b, pct, pic=pic)
    g.run()
    torch.cuda.synchronize()
    sel_gpu = g.selection()
    nsum = int(np.sum(b.n_ctx))
    offs = np.concatenate([[0], np.cumsum(b.n_ctx)]).astype(int)
    masks = None
    if wl.selector == "static" or any(wl.static_rules):
        masks = _static_masks(b, wl)
        assert np.array_equal(raw(g.static_mask)[:nsum], np.concatenate(masks))
    if wl.selector == "static":
        sel = [np.flatnonzero(m).astype(np.int32) for m in masks]
        for r in range(b.n_req):
            assert np.array_equal(sel_gpu[r], sel[r]), f"request {r}"
        mode = "none"
    elif wl.selector == "anchor":
        fk, _ = fusion.rerotate_stitch(opk, opv, b.chunk_table, b.total_rows, lo)
        fk = decode(encode(fk, wl.dtype), wl.dtype)
        gs = from_gpu(g.scores)[:nsum]
        sel = []
        for r in range(b.n_req):
            a, n = int(b.cu_T[r]), int(b.n_ctx[r])
            s = selectors.key_norm(fk[a:a + n])
            rel = np.abs(gs[offs[r]:offs[r] + n] - s) / s
            print(f"[parity] {name} req {r} key norm: max rel {float(rel.max()):.3e}", flush=True)
            assert rel.max() <= 4e-3
            spans = b.chunk_spans(r)
            kk = [selectors.anchor_budget(ln, wl.anchor_pct, 100) for _, ln in spans]
            sel.append(selectors.select_topk_segmented(s, [p for p, _ in spans],
                                                       [ln for _, ln in spans], kk))
            for (p0, ln), kc in zip(spans, kk):
                mine = sel_gpu[r][(sel_gpu[r] >= p0) & (sel_gpu[r] < p0 + ln)] - p0
                assert len(mine) == kc
                _check_selection_valid(mine, s[p0:p0 + ln], 4e-3 * float(s.max()),
                                       f"{name} req {r} chunk at {p0}")
        mode = "none"
    else:
        ref0 = fusion.fused_layer(x, w, opk, opv, b.chunk_table, b.cu_T, b.n_ctx, lo, wl.score,
                                  ks, store=wl.dtype)
        rs = np.concatenate(ref0["scores"])
        assert_close(from_gpu(g.scores)[:nsum], rs, wl.dtype, f"{name} scores")
        rms = float(np.sqrt(np.mean(rs * rs)))
        sel = []
        for r in range(b.n_req):
            s = ref0["scores"][r]
            sel.append(selectors.select_topk_forced(s.astype(np.float32), ks[r], masks[r]))
            f = np.flatnonzero(masks[r])
            assert len(f) <= ks[r] and np.isin(f, sel_gpu[r]).all(), f"request {r}: forced set"
            ranked = s.astype(np.float64).copy()
            ranked[f] = np.inf
            _check_selection_valid(sel_gpu[r], ranked, 2 * TOL[wl.dtype] * rms, f"{name} req {r}")
        mode = wl.score
    for r in range(b.n_req):
        assert len(sel_gpu[r]) == g.k_per_req[r] and np.all(np.diff(sel_gpu[r]) > 0)

    kk = [len(s) for s in sel]
    ref = fusion.fused_layer(x, w, opk, opv, b.chunk_table, b.cu_T, b.n_ctx, lo, mode, kk,
                             forced_sel=sel, store=wl.dtype)
    exact = fusion.fused_layer(x, w, opk, opv, b.chunk_table, b.cu_T, b.n_ctx, lo, mode, kk,
                               forced_sel=sel)
    g.run(forced_sel=sel)
    torch.cuda.synchronize()
    assert np.array_equal(raw(g.rows)[: g.M], ref["rows"])
    assert_close(from_gpu(g.fused_k), exact["fused_k"], wl.dtype, f"{name} fused K")
    assert_close(from_gpu(g.fused_v), exact["fused_v"], wl.dtype, f"{name} fused V")
    assert_close(from_gpu(g.q)[: g.M], exact["q"], wl.dtype, f"{name} recomputed Q")
    assert_close_vectors(from_gpu(g.out)[: g.M], ref["out"], wl.dtype, f"{name} attention output")
    assert_close(from_gpu(g.lse)[: g.M], ref["lse"], wl.dtype, f"{name} lse", tol=1e-3)
