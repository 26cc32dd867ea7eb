"""Stage parity of the int8-resident fused cache (GPU): KVBoost page, section
4.5, Eq. 7 with b = 8 kept by the fused cache, decoded by its readers.

Against the oracle (oracle/q8cache.py) on the same stored inputs:
  * re-positioning: values copied from an 8-bit KIVI cache, and values
    encoded from a dense bf16 cache, bit-exact; keys are rotated in fp32 on
    the GPU and in float64 by the oracle before the float32 encoder, so a code
    may differ by one where the exact value lies within rounding of a level
    midpoint - each key must decode within half a step of the exact
    re-positioned key, the statistics must agree to float32 rounding, and
    codes may differ by at most one;
  * fusion (scatter): the encoding of bf16 rows, bit-exact;
  * scores: deviation and key norm of the decoded keys within 1e-5;
  * attention: per output vector within the bf16 tolerance, LSE within 1e-3.
"""
import math

import numpy as np
import pytest

from oracle import fusion, kivi, q8cache, selectors
from rag_kv_cache_kvf_amd import synth
from tests.gpu_util import assert_close, assert_close_vectors, decode, encode, from_gpu, raw, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvf():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from rag_kv_cache_kvf_amd import kvfuse
    return kvfuse


def _bf(x):
    return decode(encode(x, "bf16"), "bf16")


def _rope(kvf, base, d, n):
    import torch
    c = torch.empty((n, d // 2), dtype=torch.float32, device="cuda")
    s = torch.empty_like(c)
    kvf.rope_table(base, d, n, c, s)
    return c, s


def _upload(c: q8cache.Cache) -> dict:
    return {"k_codes": to_gpu(c.k_codes), "v_codes": to_gpu(c.v_codes),
            "k_stats": to_gpu(c.k_stats), "v_stats": to_gpu(c.v_stats)}


def _download(g: dict) -> q8cache.Cache:
    return q8cache.Cache(raw(g["k_codes"]), raw(g["k_stats"]), raw(g["v_codes"]), raw(g["v_stats"]))


def check_keys(name, got: q8cache.Cache, ref: q8cache.Cache, exact_k: np.ndarray, rows):
    """Re-positioned keys: decode within half a step of the exact key, stats
    equal to float32 rounding, codes within one of the oracle's."""
    gk = q8cache.decode(got.k_codes[rows], got.k_stats[rows])
    half = got.k_stats[rows][..., 1:2].astype(np.float64) / 2
    ex = exact_k[rows]
    slack = 1e-6 * np.abs(ex).max()
    err = np.abs(gk - ex) - half * (1 + 1e-5)
    assert np.all(err <= slack), f"{name}: a key decodes {err.max():.3g} beyond half a step"
    gs, rs = got.k_stats[rows].astype(np.float64), ref.k_stats[rows].astype(np.float64)
    span = np.abs(rs[..., 0]) + 255 * rs[..., 1] + 1e-30
    assert np.max(np.abs(gs[..., 0] - rs[..., 0]) / span) < 1e-6, f"{name}: key minima differ"
    assert np.max(np.abs(gs[..., 1] - rs[..., 1]) / (rs[..., 1] + 1e-30)) < 1e-5, f"{name}: key scales differ"
    dc = np.abs(got.k_codes[rows].astype(int) - ref.k_codes[rows].astype(int))
    frac = float(np.mean(dc != 0))
    print(f"[parity] {name}: keys within half a step; {frac:.2e} of codes differ by one "
          f"from the oracle's (rounding of the rotation)", flush=True)
    assert dc.max() <= 1 and frac < 1e-2


@pytest.mark.parametrize("name", ["mini_bf16_kivi8", "qwen25_3b_kivi8", "mini_bf16_dev_pool",
                                  "mini_bf16_d64_mass"])
def test_rerotate_q8(kvf, name):
    """S1 into the int8-resident cache from an 8-bit KIVI or a dense bf16
    per-chunk cache (all rows of the small workloads, sampled rows at the
    Qwen2.5-3B-shaped 16 x (24 x 128 + 64) size)."""
    b = synth.make_batch(name)
    wl = b.wl
    print(f"[case] rerotate_q8 {name}", flush=True)
    lo = fusion.Layer(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.rope_base)
    full = name.startswith("qwen25")
    if full:
        pk = synth.random_normal((b.pool_rows, wl.n_kv_heads, wl.head_dim), 3, "pool_k").astype(np.float64)
        pv = synth.random_normal((b.pool_rows, wl.n_kv_heads, wl.head_dim), 3, "pool_v").astype(np.float64)
    else:
        w = decode(b.w_qkv, wl.dtype)
        pk, pv = fusion.pic_encode(decode(b.pool_hidden, wl.dtype), b.pool_pos, w, lo)
    pk, pv = _bf(pk), _bf(pv)
    L = kvf.Layer(wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, "bf16")
    c, s = _rope(kvf, wl.rope_base, wl.head_dim, int(np.diff(b.cu_T).max()))
    g = kvf.q8_cache(b.total_rows, wl.n_kv_heads, wl.head_dim)
    if wl.kivi_bits == 8:
        kc, kmin, ksc = kivi.encode_keys(pk.astype(np.float32), b.pool_cu)
        vc, vmin, vsc = kivi.encode_values(pv.astype(np.float32))
        pq = {"k_codes": kc, "k_min": kmin, "k_scale": ksc, "v_codes": vc, "v_min": vmin, "v_scale": vsc}
        kvf.rerotate_q8(L, to_gpu(b.chunk_table), int(b.chunk_table[:, 3].max()), None, None, c, s, g,
                        kivi={k: to_gpu(v) for k, v in pq.items()})
        ref = q8cache.stitch(b.chunk_table, b.total_rows, lo, pool_q8=pq, pool_cu=b.pool_cu)
        src_k = kivi.decode_keys(kc, kmin, ksc, b.pool_cu)
    else:
        kvf.rerotate_q8(L, to_gpu(b.chunk_table), int(b.chunk_table[:, 3].max()), to_gpu(encode(pk, "bf16")),
                        to_gpu(encode(pv, "bf16")), c, s, g)
        ref = q8cache.stitch(b.chunk_table, b.total_rows, lo, pool_k=pk, pool_v=pv)
        src_k = pk
    exact_k, _ = fusion.rerotate_stitch(src_k, np.zeros_like(src_k), b.chunk_table, b.total_rows, lo)
    got = _download(g)
    ctx = b.context_rows()
    rows = ctx[synth.random_rows(len(ctx), 2048, 7)] if full else ctx
    check_keys(f"{name} re-positioned keys", got, ref, exact_k, rows)
    assert np.array_equal(got.v_codes[rows], ref.v_codes[rows]), f"{name}: value codes"
    assert np.array_equal(got.v_stats[rows], ref.v_stats[rows]), f"{name}: value statistics"
    # query rows are covered by no chunk: left as they were (zero)
    q = b.query_rows()
    assert not got.k_codes[q].any() and not got.k_stats[q].any() and not got.v_stats[q].any()


@pytest.mark.parametrize("name,variant", [("mini_bf16_kivi8", "plain"), ("mini_bf16_dev_pool", "eligible_acc"),
                                          ("qwen25_3b_kivi8", "plain")])
def test_rerotate_q8_deviation(kvf, name, variant):
    """S1 into the int8-resident cache with the deviation score in the same
    pass (kvf_rerotate_q8_deviation): the cache bit for bit as
    kvf_rerotate_q8 writes it, the scores as kvf_score_q8 computes them from
    that cache (to fp32 summation order; NaN where ineligible, added to the
    previous scores when accumulating), and against the oracle: the
    deviation of the oracle's int8-resident cache keys from the probe keys,
    within the bf16 layer's tolerance."""
    import torch
    b = synth.make_batch(name)
    wl = b.wl
    hkv, d = wl.n_kv_heads, wl.head_dim
    print(f"[case] rerotate_q8_deviation {name} {variant}", flush=True)
    lo = fusion.Layer(wl.hidden, wl.n_q_heads, hkv, d, wl.rope_base)
    pk = _bf(synth.random_normal((b.pool_rows, hkv, d), 15, "q8dev_k").astype(np.float64))
    pv = _bf(synth.random_normal((b.pool_rows, hkv, d), 15, "q8dev_v").astype(np.float64))
    L = kvf.Layer(wl.hidden, wl.n_q_heads, hkv, d, "bf16")
    c, s = _rope(kvf, wl.rope_base, d, int(np.diff(b.cu_T).max()))
    ch = to_gpu(b.chunk_table)
    max_len = int(b.chunk_table[:, 3].max())
    if wl.kivi_bits == 8:
        kc, kmin, ksc = kivi.encode_keys(pk.astype(np.float32), b.pool_cu)
        vc, vmin, vsc = kivi.encode_values(pv.astype(np.float32))
        pq = {"k_codes": kc, "k_min": kmin, "k_scale": ksc, "v_codes": vc, "v_min": vmin, "v_scale": vsc}
        kq = {k: to_gpu(v) for k, v in pq.items()}
        pool = (None, None)
        ref = q8cache.stitch(b.chunk_table, b.total_rows, lo, pool_q8=pq, pool_cu=b.pool_cu)
        src_k = kivi.decode_keys(kc, kmin, ksc, b.pool_cu)
    else:
        kq = None
        pool = (to_gpu(encode(pk, "bf16")), to_gpu(encode(pv, "bf16")))
        ref = q8cache.stitch(b.chunk_table, b.total_rows, lo, pool_k=pk, pool_v=pv)
        src_k = pk
    exact_k, _ = fusion.rerotate_stitch(src_k, np.zeros_like(src_k), b.chunk_table, b.total_rows, lo)
    kf = exact_k + 0.3 * synth.random_normal(exact_k.shape, 16, "q8dev_fresh").astype(np.float64)
    ctx = b.context_rows()
    kf[ctx[5], hkv - 1] = 0.0                     # a zero-norm head: cos := 0
    kf_s = encode(kf, "bf16")
    n_sum = int(np.sum(b.n_ctx))
    elig, prefill = None, np.zeros(n_sum, dtype=np.float32)
    if variant == "eligible_acc":
        elig = (synth.random_rows(n_sum, n_sum, 17) % 5 != 0).astype(np.uint8)
        prefill = (0.5 + 0.003 * np.arange(n_sum) % 1.0).astype(np.float32)
    el_g = None if elig is None else to_gpu(elig)
    acc = variant == "eligible_acc"
    kb = kvf.Batch(b.cu_T, b.n_ctx)
    kf_g = to_gpu(kf_s)
    g1 = kvf.q8_cache(b.total_rows, hkv, d)
    g2 = kvf.q8_cache(b.total_rows, hkv, d)
    sc1, sc2 = to_gpu(prefill.copy()), to_gpu(prefill.copy())
    kvf.rerotate_q8_deviation(L, kb, ch, max_len, pool[0], pool[1], c, s, g1, kf_g, sc1, kivi=kq,
                              eligible=el_g, accumulate=acc)
    kvf.rerotate_q8(L, ch, max_len, pool[0], pool[1], c, s, g2, kivi=kq)
    kvf.score_q8(kvf.KVF_SCORE_DEVIATION, L, kb, g2, kf_g, sc2, eligible=el_g, accumulate=acc)
    torch.cuda.synchronize()
    got1, got2 = _download(g1), _download(g2)
    for f in ("k_codes", "k_stats", "v_codes", "v_stats"):
        assert np.array_equal(getattr(got1, f), getattr(got2, f)), f"{name}: {f} differ from kvf_rerotate_q8's"
    s1, s2 = raw(sc1).astype(np.float64), raw(sc2).astype(np.float64)
    nan1 = np.isnan(s1)
    assert np.array_equal(nan1, np.isnan(s2))
    assert np.array_equal(nan1, elig == 0) if elig is not None else not nan1.any()
    keep = ~nan1
    assert np.max(np.abs(s1[keep] - s2[keep])) < 2e-6, np.max(np.abs(s1[keep] - s2[keep]))
    refk = q8cache.decode_k(ref)
    want = np.concatenate([fusion.deviation(refk[b.cu_T[r]:b.cu_T[r] + b.n_ctx[r]],
                                            decode(kf_s, "bf16")[b.cu_T[r]:b.cu_T[r] + b.n_ctx[r]])
                           for r in range(b.n_req)]) + prefill.astype(np.float64)
    assert_close(s1[keep], want[keep], "bf16", f"{name} {variant} int8-resident fused deviation score")


@pytest.mark.parametrize("hkv,d,M", [(2, 128, 300), (8, 128, 77), (3, 64, 129), (1, 64, 40)])
def test_scatter_q8_bit_exact(kvf, hkv, d, M):
    """S5 into the int8-resident cache: every destination row is the oracle's
    encoding of its bf16 source row, bit for bit; other rows keep their
    contents; rows with an out-of-range destination or source are skipped."""
    rows_total = 3 * M + 11
    g0 = np.random.default_rng(hkv * 1000 + d + M)
    k0 = g0.standard_normal((rows_total, hkv, d)) * 2
    v0 = g0.standard_normal((rows_total, hkv, d))
    start = q8cache.Cache(*q8cache.encode(k0), *q8cache.encode(v0))
    ks = encode(g0.standard_normal((M + 5, hkv, d)) * 3 + 1, "bf16")
    vs = encode(g0.standard_normal((M, hkv, d)), "bf16")
    ks_row = g0.permutation(M + 5)[:M].astype(np.int32)
    dst = g0.permutation(rows_total)[:M].astype(np.int32)
    dst[3] = rows_total + 4                       # skipped row
    ks_row[5] = M + 9                             # K source out of range: K of that row skipped
    L = kvf.Layer(256, hkv, hkv, d, "bf16")
    g = _upload(start)
    kvf.scatter_kv_q8(L, to_gpu(ks, "bf16"), to_gpu(ks_row), to_gpu(vs, "bf16"), None, to_gpu(dst), g)
    got = _download(g)
    want = start.copy()
    kd, vd = decode(ks, "bf16"), decode(vs, "bf16")
    for m in range(M):
        t = int(dst[m])
        if not 0 <= t < rows_total:
            continue
        if 0 <= ks_row[m] < M + 5:
            c, st = q8cache.encode(kd[ks_row[m]][None])
            want.k_codes[t], want.k_stats[t] = c[0], st[0]
        c, st = q8cache.encode(vd[m][None])
        want.v_codes[t], want.v_stats[t] = c[0], st[0]
    for key in ("k_codes", "k_stats", "v_codes", "v_stats"):
        a, w = getattr(got, key), getattr(want, key)
        assert np.array_equal(a, w), f"{key}: {int(np.sum(a != w))} mismatches"


def _q8_random(T, hkv, d, seed):
    K = synth.random_normal((T, hkv, d), seed, "q8_k").astype(np.float64)
    V = synth.random_normal((T, hkv, d), seed, "q8_v").astype(np.float64)
    # per-row offsets and spreads, and an outlier channel, as real caches have
    g = np.random.default_rng(seed)
    K = K * g.uniform(0.5, 3, (T, hkv, 1)) + g.uniform(-1, 1, (T, hkv, 1))
    K[:, :, 3] *= 6
    return q8cache.Cache(*q8cache.encode(K), *q8cache.encode(V))


@pytest.mark.parametrize("hkv,d", [(2, 128), (8, 128), (3, 64)])
def test_score_q8(kvf, hkv, d):
    import torch
    cu_T = [0, 300, 301, 1100]
    n_ctx = [260, 0, 777]
    T = cu_T[-1]
    cache = _q8_random(T, hkv, d, 31 + hkv)
    dk = q8cache.decode_k(cache)
    fresh = encode(dk + 0.3 * synth.random_normal((T, hkv, d), 32, "q8_fresh"), "bf16")
    fresh[5, 0] = 0                                # zero-norm fresh head: cos 0
    L = kvf.Layer(256, hkv, hkv, d, "bf16")
    kb = kvf.Batch(cu_T, n_ctx)
    g = _upload(cache)
    sc = torch.full((sum(n_ctx),), -7.0, dtype=torch.float32, device="cuda")
    kvf.score_q8(kvf.KVF_SCORE_DEVIATION, L, kb, g, to_gpu(fresh, "bf16"), sc)
    df = decode(fresh, "bf16")
    ref = np.concatenate([fusion.deviation(dk[cu_T[r]:cu_T[r] + n_ctx[r]], df[cu_T[r]:cu_T[r] + n_ctx[r]])
                          for r in range(3)])
    gd = from_gpu(sc)
    assert np.max(np.abs(gd - ref)) < 1e-5, np.max(np.abs(gd - ref))
    kvf.score_q8(kvf.KVF_SCORE_KEY_NORM, L, kb, g, None, sc)
    refn = np.concatenate([selectors.key_norm(dk[cu_T[r]:cu_T[r] + n_ctx[r]]) for r in range(3)])
    gn = from_gpu(sc)
    assert np.max(np.abs(gn - refn) / np.maximum(refn, 1e-30)) < 1e-5
    # accumulate adds to what is there
    kvf.score_q8(kvf.KVF_SCORE_KEY_NORM, L, kb, g, None, sc, accumulate=True)
    assert np.max(np.abs(from_gpu(sc) - 2 * refn) / np.maximum(refn, 1e-30)) < 1e-5


Q8_ATTN_CASES = [
    # hq, hkv, d, T per request, recomputed rows per request
    (16, 2, 128, [400, 1000], [130, 301]),
    (4, 4, 128, [90], [90]),
    (16, 2, 128, [700, 33], [199, 33]),
    (4, 2, 64, [500], [150]),
    (64, 8, 128, [300], [40]),
    # long rows in a small grid: key splitting with the workspace
    (32, 8, 128, [3000, 2000], [400, 700]),
    (8, 2, 64, [2500], [300]),
    (32, 8, 128, [5184], [212]),
    (8, 2, 64, [6000, 300], [40, 3]),
]


@pytest.mark.parametrize("case", Q8_ATTN_CASES, ids=lambda c: "-".join(map(str, c[:3])) + f"-{c[3]}")
def test_attention_q8(kvf, case):
    import torch
    hq, hkv, d, Ts, Ms = case
    print(f"[case] attention_q8 {case}", flush=True)
    cu_T = np.concatenate([[0], np.cumsum(Ts)]).astype(int).tolist()
    cu_q = np.concatenate([[0], np.cumsum(Ms)]).astype(int).tolist()
    T = cu_T[-1]
    cache = _q8_random(T, hkv, d, 14)
    q_s = encode(synth.random_normal((cu_q[-1], hq, d), 14, "att_q", 2.0), "bf16")
    pos = np.concatenate([synth.random_rows(Ts[r], Ms[r], 15 + r) for r in range(len(Ts))])
    L = kvf.Layer(256, hq, hkv, d, "bf16")
    kb = kvf.Batch(cu_T, list(Ts))
    g = _upload(cache)
    need = kvf.attention_workspace_size(L, kb, cu_q)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda") if need > 0 else None
    runs = []
    for w in [None] + ([ws, ws] if ws is not None else []):
        out = torch.zeros((cu_q[-1], hq, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.zeros((cu_q[-1], hq), dtype=torch.float32, device="cuda")
        kvf.sparse_q_attention_q8(L, kb, to_gpu(q_s, "bf16"), to_gpu(pos), cu_q, g, 1 / math.sqrt(d),
                                  out, lse, workspace=w)
        runs.append((from_gpu(out), from_gpu(lse)))
    if ws is not None:
        assert not bool(ws[:4096].any()), "arrival counters not reset"
    lo = fusion.Layer(256, hq, hkv, d, 1e4)
    dk, dv, dq = q8cache.decode_k(cache), q8cache.decode_v(cache), decode(q_s, "bf16")
    refs, lses = [], []
    for r in range(len(Ts)):
        o, l = fusion.causal_attention(dq[cu_q[r]:cu_q[r + 1]], pos[cu_q[r]:cu_q[r + 1]],
                                       dk[cu_T[r]:cu_T[r + 1]], dv[cu_T[r]:cu_T[r + 1]], lo)
        refs.append(o)
        lses.append(l)
    for i, (go, gl) in enumerate(runs):
        tag = f"attention_q8 {case[:3]} run {i} ({'split' if i else 'unsplit'})"
        assert_close_vectors(go, np.concatenate(refs), "bf16", tag)
        assert_close(gl, np.concatenate(lses), "bf16", tag + " lse", tol=1e-3)


def test_attention_q8_degenerate(kvf):
    """Degenerate rows of an int8-resident cache: constant key and value rows
    (scale 0: every code 0, the row is its minimum), all-zero rows (the
    format of rows no chunk covers: statistics (0, 0)), a key row whose
    affine map is 0 * q + min * sum(q), and queries at positions 0 and 1
    (one or two visible keys).  The kernel's exact-key path must match the
    oracle over the decoded cache; unsplit and split runs alike."""
    import torch
    hq, hkv, d = 8, 2, 128
    Ts, Ms = [700, 64], [150, 64]
    cu_T = np.concatenate([[0], np.cumsum(Ts)]).astype(int).tolist()
    cu_q = np.concatenate([[0], np.cumsum(Ms)]).astype(int).tolist()
    T = cu_T[-1]
    K = synth.random_normal((T, hkv, d), 51, "q8d_k").astype(np.float64)
    V = synth.random_normal((T, hkv, d), 51, "q8d_v").astype(np.float64)
    K[0:100] = np.linspace(-2, 2, 100)[:, None, None]          # constant rows
    V[50:150] = np.linspace(3, -1, 100)[:, None, None]
    K[200:210] = 0.0
    V[200:210] = 0.0
    K[700:710] = 0.0                                             # start of request 1
    cache = q8cache.Cache(*q8cache.encode(K), *q8cache.encode(V))
    assert np.all(cache.k_stats[0:100, :, 1] == 0) and np.all(cache.k_codes[0:100] == 0)
    cache.k_stats[200:210] = 0.0                                 # uncovered-row format
    cache.v_stats[200:210] = 0.0
    forced = [0, 1, 2, 99, 100, 205, 699]
    rest = np.setdiff1d(synth.random_rows(700, 400, 52), forced)
    pos0 = np.sort(np.concatenate([forced, rest[:Ms[0] - len(forced)]]))
    assert len(pos0) == Ms[0] and len(np.unique(pos0)) == Ms[0]
    pos = np.concatenate([pos0, np.arange(64)]).astype(np.int32)
    q_s = encode(synth.random_normal((cu_q[-1], hq, d), 53, "q8d_q", 4.0), "bf16")
    L = kvf.Layer(256, hq, hkv, d, "bf16")
    kb = kvf.Batch(cu_T, list(Ts))
    g = _upload(cache)
    need = kvf.attention_workspace_size(L, kb, cu_q)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda") if need > 0 else None
    lo = fusion.Layer(256, hq, hkv, d, 1e4)
    dk, dv, dq = q8cache.decode_k(cache), q8cache.decode_v(cache), decode(q_s, "bf16")
    refs, lses = [], []
    for r in range(len(Ts)):
        o, l = fusion.causal_attention(dq[cu_q[r]:cu_q[r + 1]], pos[cu_q[r]:cu_q[r + 1]],
                                       dk[cu_T[r]:cu_T[r + 1]], dv[cu_T[r]:cu_T[r + 1]], lo)
        refs.append(o)
        lses.append(l)
    for i, w in enumerate([None] + ([ws] if ws is not None else [])):
        out = torch.zeros((cu_q[-1], hq, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.zeros((cu_q[-1], hq), dtype=torch.float32, device="cuda")
        kvf.sparse_q_attention_q8(L, kb, to_gpu(q_s, "bf16"), to_gpu(pos), cu_q, g, 1 / math.sqrt(d),
                                  out, lse, workspace=w)
        tag = f"attention_q8 degenerate run {i}"
        assert_close_vectors(from_gpu(out), np.concatenate(refs), "bf16", tag)
        assert_close(from_gpu(lse), np.concatenate(lses), "bf16", tag + " lse", tol=1e-3)


def test_attention_q8_full_size_sampled(kvf):
    """The Qwen2.5-3B-shaped workload (16 requests of 24 x 128 context + 64
    query tokens, 15% recomputed) with its workspace, sampled rows."""
    import torch
    wl = synth.get_workload("qwen25_3b_kivi8")
    N = sum(wl.chunk_lens)
    U = wl.n_query[0]
    T = N + U
    k = fusion.budget(N, wl.ratio_pct[0])
    n_req = wl.n_req
    hq, hkv, d = wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    cu_T = [r * T for r in range(n_req + 1)]
    cu_q = [r * (k + U) for r in range(n_req + 1)]
    pos = np.concatenate([np.concatenate([synth.random_rows(N, k, 20 + r), np.arange(N, T, dtype=np.int32)])
                          for r in range(n_req)])
    cache = _q8_random(T * n_req, hkv, d, 21)
    q_s = encode(synth.random_normal((cu_q[-1], hq, d), 21, "q_full", std=2.0), "bf16")
    L = kvf.Layer(wl.hidden, hq, hkv, d, "bf16")
    kb = kvf.Batch(cu_T, [N] * n_req)
    out = torch.zeros((cu_q[-1], hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((cu_q[-1], hq), dtype=torch.float32, device="cuda")
    need = kvf.attention_workspace_size(L, kb, cu_q)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda") if need > 0 else None
    kvf.sparse_q_attention_q8(L, kb, to_gpu(q_s, "bf16"), to_gpu(pos), cu_q, _upload(cache),
                              1 / math.sqrt(d), out, lse, workspace=ws)
    go, gl = from_gpu(out), from_gpu(lse)
    lo = fusion.Layer(wl.hidden, hq, hkv, d, wl.rope_base)
    dk, dv = q8cache.decode_k(cache), q8cache.decode_v(cache)
    samp = np.unique(np.concatenate([synth.random_rows(cu_q[-1], 32, 22), [0, cu_q[-1] - 1]]))
    ref_o, ref_l = [], []
    for m in samp:
        r = int(m // (k + U))
        o, l = fusion.causal_attention(decode(q_s[m:m + 1], "bf16"), pos[m:m + 1],
                                       dk[cu_T[r]:cu_T[r + 1]], dv[cu_T[r]:cu_T[r + 1]], lo)
        ref_o.append(o[0])
        ref_l.append(l[0])
    assert_close_vectors(go[samp], np.array(ref_o), "bf16", "qwen25_3b attention_q8 (sampled rows)")
    assert_close(gl[samp], np.array(ref_l), "bf16", "qwen25_3b attention_q8 lse (sampled rows)", tol=1e-3)


# ----------------------------------------------------------------------------
# the whole layer over the int8-resident cache
# ----------------------------------------------------------------------------
# (workload, rows whose attention is compared after the forced selection)
LAYER_Q8 = [("mini_bf16_kivi8_resident", "all"), ("mini_bf16_dense_resident", "all"),
            ("qwen25_3b_kivi8_resident", "all")]


@pytest.mark.parametrize("name,rows", LAYER_Q8, ids=[n for n, _ in LAYER_Q8])
def test_fused_layer_q8(kvf, name, rows):
    """Scores, selection (bit-exact TopK of the GPU's own scores), then on the
    oracle's selection: row list, cache (values copied or encoded bit-exact;
    keys and recomputed rows within half a step of the exact value plus the
    bf16 rounding of a recomputed source row), queries, attention and LSE."""
    import torch
    from rag_kv_cache_kvf_amd import layer as layer_mod
    from tests.gpu_util import check_selection
    from tests.test_gpu_layer import _oracle_inputs
    print(f"[case] fused layer (int8-resident) {name}", flush=True)
    b, wl, lo, x, w, pic, opk, opv, pct, ks = _oracle_inputs(name)
    g = layer_mod.FusedLayerGPU(b, pct, pic=pic)
    assert g.q8
    g.run()
    torch.cuda.synchronize()
    gs = from_gpu(g.scores)[: int(np.sum(b.n_ctx))]
    kw = {}
    if wl.kivi_bits:
        pq = {k: pic[k] for k in ("k_codes", "k_min", "k_scale", "v_codes", "v_min", "v_scale")}
        kw = dict(pool_q8=pq, pool_cu=b.pool_cu)
    else:
        kw = dict(pool_k=opk, pool_v=opv)
    ref = q8cache.fused_layer(x, w, b.chunk_table, b.cu_T, b.n_ctx, lo, ks, store="bf16", **kw)
    rs = np.concatenate(ref["scores"])
    assert_close(gs, rs, "bf16", f"{name} scores ({len(rs)} positions)")
    check_selection(name, g.selection(), gs, rs, ks, b.n_ctx)

    g.run(forced_sel=ref["sel"])
    torch.cuda.synchronize()
    assert np.array_equal(raw(g.rows)[: g.M], ref["rows"])
    assert np.array_equal(raw(g.pos)[: g.M], ref["pos"])
    got = _download(g.fused)
    want = ref["cache"]
    keep = np.setdiff1d(b.context_rows(), ref["rows"])
    # re-positioned rows: values exact, keys within half a step of the exact key
    assert np.array_equal(got.v_codes[keep], want.v_codes[keep])
    assert np.array_equal(got.v_stats[keep], want.v_stats[keep])
    src_k = kivi.decode_keys(pic["k_codes"], pic["k_min"], pic["k_scale"], b.pool_cu) if wl.kivi_bits else opk
    exact_k, _ = fusion.rerotate_stitch(src_k, np.zeros_like(src_k), b.chunk_table, b.total_rows, lo)
    check_keys(f"{name} re-positioned keys", got, ref["cache_pic"], exact_k, keep)
    # recomputed rows: the encoding of the GPU's own bf16 rows, so within half
    # a step plus one bf16 rounding of the exact (float64) recomputed values
    exact = q8cache.fused_layer(x, w, b.chunk_table, b.cu_T, b.n_ctx, lo, ks, store=None,
                                forced_sel=ref["sel"], **kw)
    rr = ref["rows"]
    for what, codes, st, ex in (("K", got.k_codes, got.k_stats, exact["k_new"]),
                                ("V", got.v_codes, got.v_stats, exact["v_new"])):
        dec = q8cache.decode(codes[rr], st[rr])
        bound = st[rr][..., 1:2].astype(np.float64) / 2 * (1 + 1e-5) + 2 ** -8 * np.abs(ex) + 1e-6
        err = np.abs(dec - ex) - bound
        print(f"[parity] {name} recomputed {what} ({len(rr)} rows): max excess {err.max():.3g}", flush=True)
        assert np.all(err <= 0), f"{name}: recomputed {what} beyond half a step + bf16 rounding"
    flat = ref["attend_flat"]
    sel_t = torch.from_numpy(flat).cuda()
    assert_close(from_gpu(g.q[sel_t]), exact["q"], "bf16", f"{name} recomputed Q")
    assert_close_vectors(from_gpu(g.out[sel_t]), ref["out"], "bf16", f"{name} attention output ({len(flat)} rows)")
    assert_close(from_gpu(g.lse[sel_t]), ref["lse"], "bf16", f"{name} lse", tol=1e-3)
