"""The C-ABI library: it loads, exports every declared entry point, and its
host-side validation rejects malformed arguments before anything reaches the
GPU (CPU only: no call here launches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import fusion, selectors

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvfuse.h")
LIB = os.path.join(ROOT, "rag_kv_cache_kvf_amd", "libkvfuse.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libkvfuse.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvf_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    lib = ctypes.CDLL(LIB)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.kvf_recompute_qkv.argtypes = [P, P, I64, P, P, I32, P, ctypes.c_uint32, P, P, I32,
                                      P, P, P, P, I64, P, ctypes.c_size_t, P]
    lib.kvf_recompute_workspace_size.argtypes = [P, I32, ctypes.c_uint32]
    lib.kvf_recompute_workspace_size.restype = ctypes.c_size_t
    return lib


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in ["kvf_rerotate", "kvf_score", "kvf_select_topk", "kvf_recompute_qkv",
              "kvf_scatter_kv", "kvf_sparse_q_attention"]:
        assert n in names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    lib.kvf_status_string.restype = ctypes.c_char_p
    assert lib.kvf_status_string(0) == b"KVF_OK"
    assert lib.kvf_status_string(2) == b"KVF_ERR_UNSUPPORTED"
    assert lib.kvf_abi_version() == 11


def test_budget_matches_oracle(lib):
    for n in (0, 1, 7, 9, 256, 3072, 5120, 10240, 32768):
        for pct in (0, 15, 20, 30, 33, 100):
            assert lib.kvf_recompute_budget(n, pct) == fusion.budget(n, pct)
    assert lib.kvf_recompute_budget(-1, 30) == -1
    assert lib.kvf_recompute_budget(10, 101) == -1


class Layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Batch(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("cu_T", ctypes.POINTER(ctypes.c_int32)),
                ("n_ctx", ctypes.POINTER(ctypes.c_int32))]


def _batch(cu, nc):
    a = (ctypes.c_int32 * len(cu))(*cu)
    b = (ctypes.c_int32 * len(nc))(*nc)
    return Batch(len(nc), ctypes.cast(a, ctypes.POINTER(ctypes.c_int32)),
                 ctypes.cast(b, ctypes.POINTER(ctypes.c_int32))), (a, b)


class StaticRules(ctypes.Structure):
    _fields_ = [("sink", ctypes.c_int32), ("boundary", ctypes.c_int32), ("seam", ctypes.c_int32)]


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def test_validation_errors(lib):
    lib.kvf_last_error.restype = ctypes.c_char_p
    ok = Layer(256, 4, 4, 64, 0)
    # head_dim and GQA shape
    assert lib.kvf_recompute_qkv(ctypes.byref(Layer(256, 4, 4, 96, 0)), FAKE, 10, None, FAKE, 1,
                                 FAKE, 7, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None, 0, None, 0, None) == 2
    assert lib.kvf_recompute_qkv(ctypes.byref(Layer(256, 6, 4, 64, 0)), FAKE, 10, None, FAKE, 1,
                                 FAKE, 7, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None, 0, None, 0, None) == 2
    assert b"multiple" in lib.kvf_last_error()
    # bad dtype, NULL layer, bad mask
    assert lib.kvf_recompute_qkv(ctypes.byref(Layer(256, 4, 4, 64, 7)), FAKE, 10, None, FAKE, 1,
                                 FAKE, 7, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None, 0, None, 0, None) == 1
    assert lib.kvf_recompute_qkv(None, FAKE, 10, None, FAKE, 1, FAKE, 7, FAKE, FAKE, 4, FAKE, FAKE,
                                 FAKE, None, 0, None, 0, None) == 1
    assert lib.kvf_recompute_qkv(ctypes.byref(ok), FAKE, 10, None, FAKE, 1, FAKE, 8, FAKE, FAKE, 4,
                                 FAKE, FAKE, FAKE, None, 0, None, 0, None) == 1
    # identity row map larger than x
    assert lib.kvf_recompute_qkv(ctypes.byref(ok), FAKE, 10, None, FAKE, 11, FAKE, 1, FAKE, FAKE, 4,
                                 FAKE, FAKE, FAKE, None, 0, None, 0, None) == 1
    # bf16 projection with Hkv * d not a multiple of 128
    assert lib.kvf_recompute_qkv(ctypes.byref(Layer(256, 3, 1, 64, 1)), FAKE, 10, None, FAKE, 1,
                                 FAKE, 7, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None, 0, None, 0, None) == 2
    # bf16 projection of few rows splits K and needs its workspace
    bf = Layer(4096, 32, 8, 128, 1)
    need = lib.kvf_recompute_workspace_size(ctypes.byref(bf), 64, 7)
    # 48 column tiles of 128 x 4 slices = 192 workgroups in one round (8
    # slices would take two): 4096 bytes of arrival counters, then the
    # slices' partial sums
    assert need == 4096 + 4 * 64 * (32 + 16) * 128 * 4
    assert lib.kvf_recompute_qkv(ctypes.byref(bf), FAKE, 64, None, FAKE, 64, FAKE, 7, FAKE, FAKE, 4,
                                 FAKE, FAKE, FAKE, None, 0, None, 0, None) == 3
    assert lib.kvf_recompute_qkv(ctypes.byref(bf), FAKE, 64, None, FAKE, 64, FAKE, 7, FAKE, FAKE, 4,
                                 FAKE, FAKE, FAKE, None, 0, FAKE, need - 1, None) == 3
    # destination rows need their count
    assert lib.kvf_recompute_qkv(ctypes.byref(ok), FAKE, 10, None, FAKE, 1, FAKE, 7, FAKE, FAKE, 4,
                                 FAKE, FAKE, FAKE, FAKE, 0, None, 0, None) == 1
    # many rows or fp32: no workspace
    assert lib.kvf_recompute_workspace_size(ctypes.byref(bf), 5000, 7) == 0
    assert lib.kvf_recompute_workspace_size(ctypes.byref(Layer(4096, 32, 8, 128, 0)), 64, 7) == 0
    assert lib.kvf_recompute_workspace_size(None, 64, 7) == 0
    # batch checks
    b, keep = _batch([0, 10, 5], [4, 2])
    assert lib.kvf_score(0, ctypes.byref(ok), ctypes.byref(b), FAKE, FAKE, None, 0, None, FAKE, None, 0,
                         None) == 1
    b, keep = _batch([0, 10], [11])
    assert lib.kvf_score(0, ctypes.byref(ok), ctypes.byref(b), FAKE, FAKE, None, 0, None, FAKE, None, 0,
                         None) == 1
    # unknown score modes and flag bits
    b, keep = _batch([0, 10], [6])
    for mode in (3, 0x200, 0x101 | 0x1000):
        assert lib.kvf_score(mode, ctypes.byref(ok), ctypes.byref(b), FAKE, FAKE, FAKE, 0, None,
                             FAKE, None, 0, None) == 1
    lib.kvf_score_workspace_size.restype = ctypes.c_size_t
    assert lib.kvf_score_workspace_size(1 | 0x100, ctypes.byref(ok), ctypes.byref(b), 0) == \
        lib.kvf_score_workspace_size(1, ctypes.byref(ok), ctypes.byref(b), 0) > 0
    assert lib.kvf_score_workspace_size(0 | 0x100, ctypes.byref(ok), ctypes.byref(b), 0) == 0
    # attention mass needs a workspace (also when accumulating)
    assert lib.kvf_score(1 | 0x100, ctypes.byref(ok), ctypes.byref(b), FAKE, None, FAKE, 0, None,
                         FAKE, None, 0, None) == 3
    assert lib.kvf_score(1, ctypes.byref(ok), ctypes.byref(b), FAKE, None, FAKE, 0, None, FAKE, None, 0,
                         None) == 3
    # attention: the key-split workspace exists only for small bf16 grids and
    # a non-NULL workspace must be large enough
    lib.kvf_attention_workspace_size.restype = ctypes.c_size_t
    lib.kvf_sparse_q_attention.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_float] + \
        [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]
    bq = Layer(4096, 32, 8, 128, 1)
    ba, keep_a = _batch([0, 5184], [5120])
    cq = (ctypes.c_int32 * 2)(0, 1600)
    need = lib.kvf_attention_workspace_size(ctypes.byref(bq), ctypes.byref(ba), cq)
    # 4096 bytes of arrival counters, then 400 (row tile, kv head) items x 2
    # parts x (16 + 1) 16-byte chunks per thread of 256
    assert need == 4096 + 50 * 8 * 2 * (4 * 4 + 1) * 256 * 16
    assert lib.kvf_sparse_q_attention(ctypes.byref(bq), ctypes.byref(ba), FAKE, FAKE, cq, FAKE, FAKE,
                                      0.088, FAKE, None, FAKE, need - 1, None) == 3
    big = (ctypes.c_int32 * 2)(0, 5184)
    assert lib.kvf_attention_workspace_size(ctypes.byref(bq), ctypes.byref(ba), big) == 0
    assert lib.kvf_attention_workspace_size(ctypes.byref(Layer(4096, 32, 8, 128, 0)),
                                            ctypes.byref(ba), cq) == 0
    bad = (ctypes.c_int32 * 2)(1, 1600)
    assert lib.kvf_sparse_q_attention(ctypes.byref(bq), ctypes.byref(ba), FAKE, FAKE, bad, FAKE,
                                      FAKE, 0.088, FAKE, None, None, 0, None) == 1
    # top-k: k > N
    k = (ctypes.c_int32 * 1)(7)
    assert lib.kvf_select_topk(FAKE, None, ctypes.byref(b), k, FAKE, None, None, None, None, 0, None) == 1
    assert lib.kvf_select_topk(FAKE, FAKE, ctypes.byref(b), k, FAKE, None, None, None, None, 0, None) == 1
    assert lib.kvf_select_topk_segmented(FAKE, None, ctypes.byref(b), FAKE, 1, k, FAKE, None,
                                         None, None) == 1
    k = (ctypes.c_int32 * 1)(3)
    assert lib.kvf_select_topk(FAKE, None, ctypes.byref(b), k, None, None, None, None, None, 0,
                               None) == 1                         # out_idx NULL
    assert lib.kvf_select_topk_segmented(FAKE, None, ctypes.byref(b), FAKE, 1, k, FAKE, FAKE,
                                         None, None) == 1         # rows without pos
    assert lib.kvf_select_topk_segmented(FAKE, None, ctypes.byref(b), None, 1, k, FAKE, None,
                                         None, None) == 1         # segs NULL
    assert lib.kvf_select_topk_segmented(FAKE, None, ctypes.byref(b), FAKE, -1, k, FAKE, None,
                                         None, None) == 1
    # static selection: negative rules, missing mask
    neg = StaticRules(-1, 0, 0)
    assert lib.kvf_select_static(ctypes.byref(b), FAKE, 1, ctypes.byref(neg), FAKE, None) == 1
    good = StaticRules(1, 1, 1)
    assert lib.kvf_select_static(ctypes.byref(b), FAKE, 1, ctypes.byref(good), None, None) == 1
    assert lib.kvf_select_static(ctypes.byref(b), None, 1, ctypes.byref(good), FAKE, None) == 1
    assert lib.kvf_select_static(ctypes.byref(b), FAKE, 1, None, FAKE, None) == 1
    # too many requests
    cu = list(range(0, 66))
    b, keep = _batch(cu, [0] * 65)
    assert lib.kvf_score(0, ctypes.byref(ok), ctypes.byref(b), FAKE, FAKE, None, 0, None, FAKE, None, 0,
                         None) == 1
    # rerotate: int8 caches need bf16 output
    class Kivi(ctypes.Structure):
        _fields_ = [(n, ctypes.c_void_p) for n in ("kc", "vc", "km", "ks", "vm", "vs")] + [
            ("n", ctypes.c_int32), ("bits", ctypes.c_int32)]
    kv = Kivi(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8)
    assert lib.kvf_rerotate(ctypes.byref(ok), FAKE, 1, 4, None, None, ctypes.byref(kv), 4, FAKE,
                            FAKE, 4, FAKE, FAKE, 4, 0, None) == 2
    # KIVI codes are 8 or 4 bits
    bfl = Layer(256, 4, 4, 64, 1)
    for bits, want in ((3, 2), (16, 2), (0, 2)):
        kv = Kivi(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, bits)
        assert lib.kvf_rerotate(ctypes.byref(bfl), FAKE, 1, 4, None, None, ctypes.byref(kv), 4,
                                FAKE, FAKE, 4, FAKE, FAKE, 4, 0, None) == want
        assert lib.kvf_kivi_encode(ctypes.byref(bfl), FAKE, FAKE, FAKE, 1, 4, 4,
                                   ctypes.byref(kv), None) == want
    # keys-only re-positioning: dense caches only, a pool_k, k_only 0 or 1
    kv = Kivi(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8)
    assert lib.kvf_rerotate(ctypes.byref(bfl), FAKE, 1, 4, None, None, ctypes.byref(kv), 4,
                            FAKE, FAKE, 4, FAKE, None, 4, 1, None) == 2
    assert lib.kvf_rerotate(ctypes.byref(bfl), FAKE, 1, 4, None, None, None, 4,
                            FAKE, FAKE, 4, FAKE, None, 4, 1, None) == 1
    assert lib.kvf_rerotate(ctypes.byref(bfl), FAKE, 1, 4, FAKE, FAKE, None, 4,
                            FAKE, FAKE, 4, FAKE, FAKE, 4, 2, None) == 1
    # gather mode needs fused_v
    assert lib.kvf_rerotate(ctypes.byref(bfl), FAKE, 1, 4, FAKE, FAKE, None, 4,
                            FAKE, FAKE, 4, FAKE, None, 4, 0, None) == 1
    # re-positioning with the deviation score: a row's rotation units
    # (Hkv d / 16) must be a power of two of at most 64, accumulate 0 or 1,
    # k_fresh and scores given, plus kvf_rerotate's own checks
    rd = lib.kvf_rerotate_deviation
    rd.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int32] * 2 + [ctypes.c_void_p] * 3 + [
        ctypes.c_int64] + [ctypes.c_void_p] * 2 + [ctypes.c_int32] + [ctypes.c_void_p] * 2 + [
        ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 2 + [ctypes.c_int32] + [ctypes.c_void_p] * 2
    b1, keep1 = _batch([0, 8], [6])

    def dev_call(layer, k_fresh=FAKE, scores=FAKE, acc=0, kivi=None, pool=(FAKE, FAKE), fv=FAKE, k_only=0):
        return rd(ctypes.byref(layer), ctypes.byref(b1), FAKE, 1, 4, pool[0], pool[1],
                  kivi, 8, FAKE, FAKE, 8, FAKE, fv, 8, k_only, k_fresh, None, acc, scores, None)
    assert dev_call(Layer(256, 4, 3, 64, 1)) == 2           # 12 units per row
    assert dev_call(Layer(4096, 32, 16, 128, 1)) == 2       # 128 units per row
    assert dev_call(Layer(256, 4, 4, 40, 1)) == 2           # head_dim 40
    assert dev_call(bfl, acc=2) == 1
    assert dev_call(bfl, k_fresh=None) == 1
    assert dev_call(bfl, scores=None) == 1
    assert dev_call(bfl, fv=None) == 1                      # gather mode needs fused_v
    assert dev_call(ok, kivi=ctypes.byref(kv), pool=(None, None)) == 2   # KIVI decodes to bf16 only
    assert dev_call(bfl, kivi=ctypes.byref(kv), pool=(None, None), fv=None, k_only=1) == 2
    bad_batch, keep2 = _batch([0, 8, 4], [6, 2])            # cu_T decreasing
    assert rd(ctypes.byref(bfl), ctypes.byref(bad_batch), FAKE, 1, 4, FAKE, FAKE, None, 8, FAKE, FAKE,
              8, FAKE, FAKE, 8, 0, FAKE, None, 0, FAKE, None) == 1


def test_rerotate_score_attn_mass_validation(lib):
    """Keys-only re-positioning inside the attention-mass pass: kvf_score's
    and kvf_rerotate's checks on the host, plus the fused cache holding the
    batch."""
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    f = lib.kvf_rerotate_score_attn_mass
    f.argtypes = [P, P, P, I32, I32, P, I64, P, P, I32, P, I64, P, I32, P, I32, P, P, ctypes.c_size_t, P]
    bf = Layer(2048, 16, 2, 128, 1)
    b, keep = _batch([0, 100, 200], [90, 90])

    def call(layer=bf, pool=FAKE, fused_rows=200, acc=0, ws_bytes=1 << 30, q=FAKE, scores=FAKE, nch=1):
        return f(ctypes.byref(layer), ctypes.byref(b), FAKE, nch, 8, pool, 100, FAKE, FAKE, 8, FAKE,
                 fused_rows, q, 0, None, acc, scores, FAKE, ws_bytes, None)
    assert call(fused_rows=199) == 1          # the fused cache must hold the batch
    assert call(pool=None) == 1               # chunks need the per-chunk keys
    assert call(acc=2) == 1
    assert call(q=None) == 1
    assert call(scores=None) == 1
    assert call(ws_bytes=0) == 3
    assert call(nch=-1) == 1


def test_empty_calls_are_noops(lib):
    ok = Layer(256, 4, 4, 64, 0)
    assert lib.kvf_rope_table(ctypes.c_double(1e4), 64, 0, None, None, None) == 0
    assert lib.kvf_recompute_qkv(ctypes.byref(ok), None, 0, None, None, 0, None, 7, None, None, 0,
                                 None, None, None, None, 0, None, 0, None) == 0
    assert lib.kvf_scatter_kv(ctypes.byref(ok), None, None, 0, None, None, 0, None, 0, None, None, 0,
                              None) == 0


def test_anchor_budget_matches_oracle(lib):
    for n in (0, 1, 5, 37, 64, 128, 512, 1000, 1024):
        for num, den in ((1, 10), (15, 100), (1, 3), (0, 7), (7, 7), (333, 1000)):
            assert lib.kvf_anchor_budget(n, num, den) == selectors.anchor_budget(n, num, den)
    for args in ((-1, 1, 4), (5, 1, 0), (5, -1, 4), (5, 5, 4)):
        assert lib.kvf_anchor_budget(*args) == -1


def _chunk_rows(cu_T, starts_per_req, pos_shift=0):
    rows = []
    for r, starts in enumerate(starts_per_req):
        for p in starts:
            rows.append([0, cu_T[r] + p, p + pos_shift, 1, 0, 0, 0, 0])
    return np.array(rows, dtype=np.int32).reshape(-1, 8)


@pytest.mark.parametrize("seed", range(8))
def test_static_counts_match_oracle(lib, seed):
    """The host count the library sizes static selections with equals the
    number of positions in the oracle's static mask (host code only)."""
    g = np.random.default_rng(500 + seed)
    n_req = int(g.integers(1, 5))
    ns = [int(g.integers(0, 300)) for _ in range(n_req)]
    us = [int(g.integers(0, 20)) for _ in range(n_req)]
    cu = [0]
    for n, u in zip(ns, us):
        cu.append(cu[-1] + n + u)
    starts = []
    for n in ns:
        st = sorted(set([0] + g.integers(0, max(n, 1), size=int(g.integers(0, 6))).tolist()))
        starts.append([p for p in st if p < n] if n else [])
    ch = _chunk_rows(cu, starts)
    # chunks of other requests and a chunk starting in the query rows are ignored
    if n_req and us[0]:
        ch = np.concatenate([ch, np.array([[0, cu[0] + ns[0], 0, 1, 0, 0, 0, 0]], np.int32)])
    g.shuffle(ch)
    sink, boundary, seam = (int(v) for v in g.integers(0, 20, size=3))
    b, keep = _batch(cu, ns)
    out = (ctypes.c_int32 * n_req)()
    rules = StaticRules(sink, boundary, seam)
    assert lib.kvf_static_counts(ctypes.byref(b), ch.ctypes.data_as(ctypes.c_void_p),
                                 ch.shape[0], ctypes.byref(rules), out) == 0
    for r in range(n_req):
        want = int(selectors.static_mask(ns[r], starts[r] or [0], sink, boundary, seam).sum()) \
            if ns[r] else 0
        assert out[r] == want


def test_noalloc_rejects_oversized_calls(lib):
    """The allocation-free attention-mass call refuses, on the host, a call
    whose workspace would exceed its fixed scratch array (48 MiB), and
    validates like kvf_score otherwise."""
    P = ctypes.c_void_p
    lib.kvf_score_attn_mass_noalloc.argtypes = [P, P, P, P, ctypes.c_int32, P, P, ctypes.c_int32, P]
    lib.kvf_score_workspace_size.restype = ctypes.c_size_t
    lib.kvf_score_workspace_size.argtypes = [ctypes.c_int32, P, P, ctypes.c_int32]
    L = Layer(8192, 64, 8, 128, 1)
    T, N = 66048, 65536
    b, keep = _batch([0, T], [N])
    need = lib.kvf_score_workspace_size(1, ctypes.byref(L), ctypes.byref(b), 0)
    assert need > 48 << 20
    assert lib.kvf_score_attn_mass_noalloc(ctypes.byref(L), ctypes.byref(b), FAKE, FAKE, 0, None, FAKE,
                                           0, None) == 2
    assert lib.kvf_score_attn_mass_noalloc(ctypes.byref(L), ctypes.byref(b), FAKE, None, 0, None, FAKE,
                                           0, None) == 1
    assert lib.kvf_score_attn_mass_noalloc(ctypes.byref(L), ctypes.byref(b), FAKE, FAKE, 0, None, FAKE,
                                           2, None) == 1
    # within the limit the same call size passes validation (not launched here)
    b2, keep2 = _batch([0, 5184], [5120])
    assert lib.kvf_score_workspace_size(1, ctypes.byref(Layer(4096, 32, 8, 128, 1)), ctypes.byref(b2),
                                        0) < 48 << 20


class Q8(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("kc", "vc", "ks", "vs")] + [("rows", ctypes.c_int64)]


def test_q8_validation(lib):
    """The int8-resident calls check the cache descriptor, its row count
    against the batch, the layer precision and the supported sources and
    modes on the host."""
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.kvf_rerotate_q8.argtypes = [P, P, I32, I32, P, P, P, I64, P, P, I32, P, P]
    lib.kvf_score_q8.argtypes = [I32, P, P, P, P, P, P, P]
    lib.kvf_scatter_kv_q8.argtypes = [P, P, P, I64, P, P, I64, P, I32, P, P]
    lib.kvf_sparse_q_attention_q8.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, P,
                                              ctypes.c_size_t, P]
    bf = Layer(2048, 16, 2, 128, 1)
    f32 = Layer(2048, 16, 2, 128, 0)
    c = Q8(FAKE, FAKE, FAKE, FAKE, 100)
    short = Q8(FAKE, FAKE, FAKE, FAKE, 99)
    partial = Q8(FAKE, None, FAKE, FAKE, 100)

    class Kivi(ctypes.Structure):
        _fields_ = [(n, ctypes.c_void_p) for n in ("kc", "vc", "km", "ks", "vm", "vs")] + [
            ("n", ctypes.c_int32), ("bits", ctypes.c_int32)]
    k8 = Kivi(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8)
    k4 = Kivi(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4)
    rr = lib.kvf_rerotate_q8
    assert rr(ctypes.byref(f32), FAKE, 1, 4, None, None, ctypes.byref(k8), 4, FAKE, FAKE, 4,
              ctypes.byref(c), None) == 2                      # bf16 layers only
    assert rr(ctypes.byref(bf), FAKE, 1, 4, None, None, ctypes.byref(k4), 4, FAKE, FAKE, 4,
              ctypes.byref(c), None) == 2                      # 4-bit sources unsupported
    assert rr(ctypes.byref(bf), FAKE, 1, 4, FAKE, FAKE, ctypes.byref(k8), 4, FAKE, FAKE, 4,
              ctypes.byref(c), None) == 1                      # dense and KIVI at once
    assert rr(ctypes.byref(bf), FAKE, 1, 4, FAKE, None, None, 4, FAKE, FAKE, 4,
              ctypes.byref(c), None) == 1                      # dense needs both tensors
    assert rr(ctypes.byref(bf), FAKE, 1, 4, FAKE, FAKE, None, 4, FAKE, FAKE, 4,
              None, None) == 1                                 # no cache
    assert rr(ctypes.byref(bf), FAKE, 1, 4, FAKE, FAKE, None, 4, FAKE, FAKE, 4,
              ctypes.byref(partial), None) == 1
    assert rr(ctypes.byref(bf), FAKE, 0, 4, FAKE, FAKE, None, 4, FAKE, FAKE, 4,
              ctypes.byref(c), None) == 0                      # no chunks: nothing to do
    # with the deviation score in the same pass: a row's lanes (Hkv d / 8)
    # a power of two of at most 64, accumulate 0 or 1, k_fresh and scores,
    # then kvf_rerotate_q8's own checks
    rqd = lib.kvf_rerotate_q8_deviation
    rqd.argtypes = [P, P, P, I32, I32, P, P, P, I64, P, P, I32, P, P, P, I32, P, P]
    bq, keepq = _batch([0, 60, 100], [50, 30])

    def q8dev(layer, kv=None, pool=(FAKE, FAKE), cache=c, k_fresh=FAKE, scores=FAKE, acc=0):
        return rqd(ctypes.byref(layer), ctypes.byref(bq), FAKE, 1, 4, pool[0], pool[1], kv, 4, FAKE,
                   FAKE, 4, None if cache is None else ctypes.byref(cache), k_fresh, None, acc, scores,
                   None)
    assert q8dev(Layer(4096, 32, 8, 128, 1)) == 2              # 128 lanes per row
    assert q8dev(Layer(2048, 16, 2, 96, 1)) == 2               # head_dim 96
    assert q8dev(bf, acc=3) == 1
    assert q8dev(bf, k_fresh=None) == 1
    assert q8dev(bf, scores=None) == 1
    assert q8dev(f32) == 2                                     # bf16 layers only
    assert q8dev(bf, kv=ctypes.byref(k4), pool=(None, None)) == 2
    assert q8dev(bf, cache=None) == 1
    assert q8dev(bf, cache=partial) == 1
    b, keep = _batch([0, 60, 100], [50, 30])
    sq = lib.kvf_score_q8
    assert sq(1, ctypes.byref(bf), ctypes.byref(b), ctypes.byref(c), FAKE, None, FAKE, None) == 2
    assert sq(0, ctypes.byref(bf), ctypes.byref(b), ctypes.byref(c), None, None, FAKE, None) == 1
    assert sq(0, ctypes.byref(bf), ctypes.byref(b), ctypes.byref(short), FAKE, None, FAKE, None) == 1
    assert sq(3, ctypes.byref(bf), ctypes.byref(b), ctypes.byref(c), FAKE, None, FAKE, None) == 1
    assert sq(0, ctypes.byref(f32), ctypes.byref(b), ctypes.byref(c), FAKE, None, FAKE, None) == 2
    sc = lib.kvf_scatter_kv_q8
    assert sc(ctypes.byref(bf), FAKE, None, 4, None, None, 0, FAKE, 5, ctypes.byref(c), None) == 1
    assert sc(ctypes.byref(bf), FAKE, None, 4, None, None, 0, None, 4, ctypes.byref(c), None) == 1
    assert sc(ctypes.byref(bf), None, None, 0, None, None, 0, None, 4, ctypes.byref(c), None) == 0
    at = lib.kvf_sparse_q_attention_q8
    cq = (ctypes.c_int32 * 3)(0, 20, 30)
    assert at(ctypes.byref(bf), ctypes.byref(b), FAKE, FAKE, cq, ctypes.byref(short), 0.088, FAKE,
              None, None, 0, None) == 1
    assert at(ctypes.byref(f32), ctypes.byref(b), FAKE, FAKE, cq, ctypes.byref(c), 0.088, FAKE,
              None, None, 0, None) == 2
    lib.kvf_attention_workspace_size.restype = ctypes.c_size_t
    need = lib.kvf_attention_workspace_size(ctypes.byref(bf), ctypes.byref(b), cq)
    assert need > 0
    assert at(ctypes.byref(bf), ctypes.byref(b), FAKE, FAKE, cq, ctypes.byref(c), 0.088, FAKE,
              None, FAKE, need - 1, None) == 3

