"""Parity of the static and segmented selectors and the key-norm score (GPU).

Static mask, forced top-k and segmented top-k are integer work: bit-exact
against the oracle (oracle/selectors.py) on the same inputs; the segmented
and forced selections take their decisions on the same fp32 scores on both
sides.  Key norm is fp32 arithmetic over stored keys: relative error per
token within 1e-5 of the float64 norm.  Sources: KVBoost page, sections 4.1
and 4.6.1 (Algorithm 1); QCFuse page, sections 2.2.1 and 3.3.1 (Eq. 14).
"""
import numpy as np
import pytest

from oracle import fusion, selectors
from rag_kv_cache_kvf_amd import synth
from tests.gpu_util import decode, encode, from_gpu, raw, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvf():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from rag_kv_cache_kvf_amd import kvfuse
    return kvfuse


def _cu(n_ctx, n_query):
    cu = [0]
    for n, u in zip(n_ctx, n_query):
        cu.append(cu[-1] + n + u)
    return cu


# ----------------------------------------------------------------------------
# key norm
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,hkv,d", [("bf16", 8, 128), ("bf16", 2, 128), ("f32", 4, 64),
                                         ("bf16", 1, 64), ("bf16", 3, 64)])
def test_key_norm(kvf, dtype, hkv, d):
    import torch
    n_ctx, n_query = [260, 0, 777, 5], [40, 1, 23, 0]
    cu = _cu(n_ctx, n_query)
    k = synth.random_normal((cu[-1], hkv, d), 11, "knorm").astype(np.float64)
    k[3] = 0.0                                         # a zero key -> norm 0
    k[cu[2] + 7] *= 1e3
    ks = encode(k, dtype)
    sc = torch.full((sum(n_ctx),), -7.0, dtype=torch.float32, device="cuda")
    kvf.score(kvf.KVF_SCORE_KEY_NORM, kvf.Layer(256, hkv, hkv, d, dtype), kvf.Batch(cu, n_ctx),
              to_gpu(ks, dtype), None, None, sc)
    dk = decode(ks, dtype)
    ref = np.concatenate([selectors.key_norm(dk[cu[r]:cu[r] + n_ctx[r]]) for r in range(4)])
    got = from_gpu(sc)
    err = np.abs(got - ref) / np.maximum(ref, 1e-30)
    print(f"[parity] key norm {dtype} hkv={hkv} d={d}: max rel {float(err[ref > 0].max()):.3e}",
          flush=True)
    assert got[3] == 0.0
    assert np.all(err[ref > 0] <= 1e-5)


def test_key_norm_full_size(kvf):
    """qwen3-8b pool workload rows: 8 requests x 10240 context tokens."""
    import torch
    wl = synth.get_workload("qwen3_8b_dev_pool")
    n_ctx = [10240] * 8
    cu = _cu(n_ctx, [128] * 8)
    k = synth.random_normal((cu[-1], wl.n_kv_heads, wl.head_dim), 12, "knorm_full")
    ks = encode(k, "bf16")
    sc = torch.empty((sum(n_ctx),), dtype=torch.float32, device="cuda")
    kvf.score(kvf.KVF_SCORE_KEY_NORM, kvf.Layer(4096, 32, 8, 128, "bf16"), kvf.Batch(cu, n_ctx),
              to_gpu(ks, "bf16"), None, None, sc)
    dk = decode(ks, "bf16")
    ref = np.concatenate([selectors.key_norm(dk[cu[r]:cu[r] + n_ctx[r]]) for r in range(8)])
    err = np.abs(from_gpu(sc) - ref) / ref
    print(f"[parity] key norm full size: max rel {float(err.max()):.3e}", flush=True)
    assert np.all(err <= 1e-5)


# ----------------------------------------------------------------------------
# static mask
# ----------------------------------------------------------------------------
def _static_case(kvf, n_ctx, n_query, starts, rules, seed, extra_rows=()):
    """starts[r]: chunk start positions of request r.  The chunk table is
    shuffled and may hold rows outside every context (ignored)."""
    import torch
    cu = _cu(n_ctx, n_query)
    rows = [[0, cu[r] + p, p, 1, 0, 0, 0, 0] for r in range(len(n_ctx)) for p in starts[r]]
    rows += [[0, e, 0, 1, 0, 0, 0, 0] for e in extra_rows]
    table = np.asarray(rows, dtype=np.int32).reshape(-1, 8)
    np.random.default_rng(seed).shuffle(table)
    kb = kvf.Batch(cu, n_ctx)
    mask = torch.full((max(sum(n_ctx), 1),), 7, dtype=torch.uint8, device="cuda")
    kvf.select_static(kb, to_gpu(table), rules, mask)
    got = raw(mask)
    counts = kvf.static_counts(kb, table, rules)
    off = 0
    for r, n in enumerate(n_ctx):
        want = selectors.static_mask(n, sorted(starts[r]), *rules)
        assert np.array_equal(got[off:off + n], want), f"request {r}"
        assert counts[r] == int(want.sum())
        off += n
    return got


@pytest.mark.parametrize("seed", range(6))
def test_static_mask_random(kvf, seed):
    g = np.random.default_rng(700 + seed)
    R = int(g.integers(1, 7))
    n_ctx = [int(g.integers(0, 3000)) for _ in range(R)]
    n_query = [int(g.integers(0, 50)) for _ in range(R)]
    starts = []
    for n in n_ctx:
        st = set([0] + g.integers(0, max(n, 1), size=int(g.integers(0, 12))).tolist())
        starts.append(sorted(p for p in st if p < n) if n else [])
    rules = tuple(int(v) for v in g.integers(0, 40, size=3))
    cu = _cu(n_ctx, n_query)
    extra = [cu[0] + n_ctx[0]] if n_query[0] else []      # a chunk starting at a query row
    _static_case(kvf, n_ctx, n_query, starts, rules, seed, extra)


def test_static_mask_windows_and_edges(kvf):
    # longer than one LDS window (16384 positions); llama3-70b chunk layout
    starts = [list(range(0, 32768, 1024))]
    m = _static_case(kvf, [32768], [256], starts, (4, 2, 16), 1)
    assert int(m.sum()) == 4 + 32 * 2 + 31 * 16 - 2    # sink overlaps chunk 0's boundary
    # a window that straddles the LDS window edge
    _static_case(kvf, [40000], [0], [[0, 16380, 16384, 16390, 39999]], (0, 9, 9), 2)
    # rules longer than the context, empty requests, no rules at all
    _static_case(kvf, [5, 0, 12], [3, 4, 0], [[0, 2], [], [0, 6]], (100, 100, 100), 3)
    _static_case(kvf, [300, 10], [1, 1], [[0, 100, 200], [0]], (0, 0, 0), 4)


# ----------------------------------------------------------------------------
# forced top-k
# ----------------------------------------------------------------------------
def _forced_case(kvf, scores, forced, ks, n_query, use_scores=True):
    import torch
    n_ctx = [len(s) for s in scores]
    cu = _cu(n_ctx, n_query)
    kb = kvf.Batch(cu, n_ctx)
    flat = np.concatenate(scores).astype(np.float32) if sum(n_ctx) else np.zeros(1, np.float32)
    fm = np.concatenate(forced).astype(np.uint8) if sum(n_ctx) else np.zeros(1, np.uint8)
    out = torch.full((max(sum(ks), 1),), -1, dtype=torch.int32, device="cuda")
    M = sum(ks) + sum(n_query)
    rows = torch.full((max(M, 1),), -1, dtype=torch.int32, device="cuda")
    pos = torch.full((max(M, 1),), -1, dtype=torch.int32, device="cuda")
    kvf.select_topk(to_gpu(flat) if use_scores else None, kb, ks, out, rows, pos,
                    forced=to_gpu(fm))
    got, grows, gpos = raw(out), raw(rows), raw(pos)
    off = moff = 0
    for r in range(len(scores)):
        s = scores[r].astype(np.float32) if use_scores else np.zeros(n_ctx[r], np.float32)
        ref = selectors.select_topk_forced(s, ks[r], forced[r])
        assert np.array_equal(got[off:off + ks[r]], ref), f"request {r}"
        want = np.concatenate([ref, np.arange(n_ctx[r], n_ctx[r] + n_query[r])])
        m = ks[r] + n_query[r]
        assert np.array_equal(gpos[moff:moff + m], want)
        assert np.array_equal(grows[moff:moff + m], want + cu[r])
        off += ks[r]
        moff += m


@pytest.mark.parametrize("seed", range(5))
def test_forced_topk_random(kvf, seed):
    g = np.random.default_rng(800 + seed)
    scores, forced, ks, nq = [], [], [], []
    for r in range(int(g.integers(1, 8))):
        n = int(g.integers(1, 6000))
        s = synth.random_scores(n, seed * 10 + r, distinct_levels=5 if r % 2 else None)
        f = (g.random(n) < [0.0, 0.01, 0.2, 0.9][r % 4]).astype(np.uint8)
        f[f > 0] = g.integers(1, 256, size=int(f.sum()))       # any nonzero byte forces
        scores.append(s)
        forced.append(f)
        ks.append(int(g.integers(0, n + 1)))
        nq.append(int(g.integers(0, 70)))
    _forced_case(kvf, scores, forced, ks, nq)


def test_forced_topk_edges(kvf):
    nan = np.array([np.nan, 3.0, np.inf, -np.inf, -0.0, 0.0, 2.0], dtype=np.float32)
    f = np.array([0, 0, 0, 1, 0, 0, 1], dtype=np.uint8)
    # forced below NaN, -inf and every score; k smaller than the forced set
    _forced_case(kvf, [nan, nan, nan, nan], [f, f, f, np.ones(7, np.uint8)], [2, 1, 7, 3],
                 [2, 0, 1, 3])
    # no scores: exactly the forced set when k = |forced|
    g = np.random.default_rng(5)
    fs = [(g.random(n) < 0.1).astype(np.uint8) for n in (1000, 37000, 12)]
    _forced_case(kvf, [np.zeros(len(x), np.float32) for x in fs], fs,
                 [int(x.sum()) for x in fs], [4, 64, 0], use_scores=False)


def test_forced_topk_full_size(kvf):
    """qwen3-8b pool layout (8 x 10240 context, r = 30%) with sink + seam
    windows forced; the llama3-70b request (32 x 1024, r = 20%)."""
    for n, R, pct, step in ((10240, 8, 30, 512), (32768, 1, 20, 1024)):
        scores = [synth.random_scores(n, 900 + r) for r in range(R)]
        forced = [selectors.static_mask(n, list(range(0, n, step)), 4, 1, 16) for _ in range(R)]
        _forced_case(kvf, scores, forced, [fusion.budget(n, pct)] * R, [64] * R)


# ----------------------------------------------------------------------------
# segmented top-k
# ----------------------------------------------------------------------------
def _segmented_case(kvf, scores, n_query, segs_per_req, forced=None, bad_segs=()):
    """segs_per_req[r]: list of (pos0, len, k) ascending and disjoint; the
    picks take consecutive slots.  bad_segs: extra rows that break the
    contract (they must write nothing)."""
    import torch
    n_ctx = [len(s) for s in scores]
    cu = _cu(n_ctx, n_query)
    kb = kvf.Batch(cu, n_ctx)
    table, ks = [], []
    for r, segs in enumerate(segs_per_req):
        kr = 0
        for p0, ln, k in segs:
            table.append([r, p0, ln, k, kr, 0, 0, 0])
            kr += k
        ks.append(kr)
    table += [list(b) + [0] * (8 - len(b)) for b in bad_segs]
    t = np.asarray(table, dtype=np.int32).reshape(-1, 8)
    np.random.default_rng(len(table)).shuffle(t)          # any table order
    flat = np.concatenate(scores).astype(np.float32)
    fm = None if forced is None else to_gpu(np.concatenate(forced).astype(np.uint8))
    out = torch.full((max(sum(ks), 1),), -1, dtype=torch.int32, device="cuda")
    M = sum(ks) + sum(n_query)
    rows = torch.full((max(M, 1),), -1, dtype=torch.int32, device="cuda")
    pos = torch.full((max(M, 1),), -1, dtype=torch.int32, device="cuda")
    kvf.select_topk_segmented(to_gpu(flat), kb, to_gpu(t), ks, out, rows, pos, forced=fm)
    got, grows, gpos = raw(out), raw(rows), raw(pos)
    off = moff = 0
    for r, segs in enumerate(segs_per_req):
        s = scores[r].astype(np.float32)
        if forced is None:
            ref = selectors.select_topk_segmented(s, [a for a, _, _ in segs],
                                                  [b for _, b, _ in segs], [c for _, _, c in segs])
        else:
            ref = np.concatenate([p0 + selectors.select_topk_forced(s[p0:p0 + ln], k,
                                                                    forced[r][p0:p0 + ln])
                                  for p0, ln, k in segs] or [np.zeros(0, np.int32)])
        assert np.array_equal(got[off:off + ks[r]], ref), f"request {r}"
        want = np.concatenate([ref, np.arange(n_ctx[r], n_ctx[r] + n_query[r])])
        m = ks[r] + n_query[r]
        assert np.array_equal(gpos[moff:moff + m], want)
        assert np.array_equal(grows[moff:moff + m], want + cu[r])
        off += ks[r]
        moff += m


def _random_segments(g, n):
    cuts = sorted(set([0, n] + g.integers(0, n, size=int(g.integers(0, 9))).tolist()))
    segs = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        if g.random() < 0.15:                               # gaps are allowed
            continue
        segs.append((a, b - a, int(g.integers(0, b - a + 1))))
    return segs


@pytest.mark.parametrize("seed", range(5))
def test_segmented_random(kvf, seed):
    g = np.random.default_rng(900 + seed)
    scores, nq, segs = [], [], []
    for r in range(int(g.integers(1, 6))):
        n = int(g.integers(1, 4000))
        scores.append(synth.random_scores(n, seed * 10 + r, distinct_levels=4 if r % 2 else None))
        nq.append(int(g.integers(0, 40)))
        segs.append(_random_segments(g, n))
    forced = None
    if seed % 2:
        forced = [(g.random(len(s)) < 0.05).astype(np.uint8) for s in scores]
    _segmented_case(kvf, scores, nq, segs, forced)


def test_segmented_edges(kvf):
    s = [synth.random_scores(20000, 1), synth.random_scores(50, 2)]
    # a segment longer than the LDS key cache (8192), k = len, k = 0, a
    # single-position segment, a request without segments
    segs = [[(0, 9000, 900), (9000, 10000, 37), (19000, 999, 999), (19999, 1, 1)], []]
    bad = [(1, 40, 20, 3, 0), (0, 0, 5, 6, 0), (2, 0, 1, 1, 0), (0, 19990, 20, 1, 0),
           (0, 0, 5, 1, 10**6), (-1, 0, 1, 1, 0)]
    _segmented_case(kvf, s, [3, 5], segs, bad_segs=bad)
    # bad rows aimed at the slots of a good segment leave them alone
    _segmented_case(kvf, [synth.random_scores(10, 3)], [2], [[(0, 4, 2)]],
                    bad_segs=[(0, 0, 10, 11, 0), (0, 5, 6, 2, 0), (0, 0, 3, 3, 0)])


@pytest.mark.parametrize("wl_name", ["llama3_70b_mass", "qwen3_8b_dev_pool", "qwen3_8b_anchor"])
def test_segmented_full_size(kvf, wl_name):
    """Per-chunk anchors (ceil(r_a |c_i|), r_a = 10%) over the chunks of the
    benchmark workloads."""
    wl = synth.get_workload(wl_name)
    lens = list(wl.chunk_lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).tolist()
    n = sum(lens)
    scores = [synth.random_scores(n, 950 + r, ties=n // 8) for r in range(wl.n_req)]
    segs = [[(p, ln, selectors.anchor_budget(ln, 10, 100)) for p, ln in zip(starts, lens)]
            for _ in range(wl.n_req)]
    _segmented_case(kvf, scores, [wl.query_len(r) for r in range(wl.n_req)], segs)
