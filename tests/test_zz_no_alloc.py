"""The allocation-free attention-mass entry point (GPU): through the C ABI,
kvf_score_attn_mass_noalloc gives bit for bit what kvf_score gives with a
caller workspace, on calls in a row whose inputs shrink (the scratch array
keeps the previous call's contents)."""
import numpy as np
import pytest

from rag_kv_cache_kvf_amd import synth
from tests.gpu_util import raw, to_gpu, encode

pytestmark = pytest.mark.gpu

CASES = [
    # (hq, hkv, d, cu_T, n_ctx, n_last_q)
    (32, 8, 128, [0, 5184], [5120], 0),           # the 8B-shaped request
    (16, 2, 128, [0, 3136, 6272], [3072, 3072], 0),
    (4, 2, 64, [0, 233], [188], 5),               # smaller again, last 5 query rows
]


def _run_case(kvf, torch, case, seed, accumulate=False, eligible=False):
    hq, hkv, d, cu_T, n_ctx, nlq = case
    T = cu_T[-1]
    nU = T - sum(n_ctx)
    k = to_gpu(encode(synth.random_normal((T, hkv, d), seed, "noalloc_k").astype(np.float64), "bf16"), "bf16")
    q = to_gpu(encode(synth.random_normal((nU, hq, d), seed, "noalloc_q", 1.5).astype(np.float64), "bf16"),
               "bf16")
    L = kvf.Layer(256, hq, hkv, d, "bf16")
    kb = kvf.Batch(cu_T, n_ctx)
    n = sum(n_ctx)
    elig = None
    if eligible:
        m = (synth.random_scores(n, seed) > -0.3).astype(np.uint8)
        elig = torch.from_numpy(m).cuda()
    start = torch.from_numpy(synth.random_scores(n, seed + 1)).cuda()
    ws = torch.zeros(kvf.score_workspace_size(kvf.KVF_SCORE_ATTN_MASS, L, kb, nlq), dtype=torch.uint8,
                     device="cuda")
    a = start.clone()
    kvf.score(kvf.KVF_SCORE_ATTN_MASS, L, kb, k, None, q, a, ws, n_last_q=nlq, eligible=elig,
              accumulate=accumulate)
    b = start.clone()
    kvf.score_attn_mass_noalloc(L, kb, k, q, b, n_last_q=nlq, eligible=elig, accumulate=accumulate)
    torch.cuda.synchronize()
    return raw(a), raw(b)


def test_noalloc_matches_workspace_call():
    import torch
    assert torch.cuda.is_available()
    from rag_kv_cache_kvf_amd import kvfuse as kvf
    for i, case in enumerate(CASES):
        print(f"[case] no-alloc attention mass call {i}: {case}", flush=True)
        ref, got = _run_case(kvf, torch, case, 50 + i)
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), f"call {i} differs"
    # again, smaller than the first, with an eligibility mask and accumulation
    print("[case] no-alloc attention mass: accumulate + eligible", flush=True)
    ref, got = _run_case(kvf, torch, CASES[1], 60, accumulate=True, eligible=True)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))
    assert np.isnan(got).any() and np.isfinite(got).any()
