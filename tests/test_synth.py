"""The seeded input generator: determinism and the request layout."""
import numpy as np
import pytest

from rag_kv_cache_kvf_amd import synth


@pytest.mark.parametrize("name", sorted(synth.MINI_WORKLOADS) + ["tiny_fp32_dev"])
def test_deterministic_and_consistent(name):
    a = synth.make_batch(name)
    b = synth.make_batch(name)
    for f in ("x", "pool_hidden", "w_qkv", "chunk_table", "cu_T", "n_ctx", "pool_pos"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = synth.make_batch(name, seed=1)
    assert not np.array_equal(a.x, c.x)
    wl = a.wl
    # every request's context rows are covered exactly once by its chunks
    cover = np.zeros(a.total_rows, dtype=int)
    for src, dst, pos0, n, pc in a.chunk_table[:, :5]:
        cover[dst:dst + n] += 1
        r = np.searchsorted(a.cu_T, dst, side="right") - 1
        assert dst - a.cu_T[r] == pos0
        assert a.pool_cu[pc] == src and a.pool_cu[pc + 1] - src == n
        assert np.array_equal(a.pool_pos[src:src + n], np.arange(n))
    assert np.array_equal(cover[a.context_rows()], np.ones(len(a.context_rows())))
    assert cover[a.query_rows()].sum() == 0
    # slot 0 caches the fresh hidden state itself
    for src, dst, pos0, n in a.chunk_table[a.chunk_table[:, 2] == 0][:, :4]:
        assert np.array_equal(a.x[dst:dst + n], a.pool_hidden[src:src + n])
    assert a.x.dtype == (np.float32 if wl.dtype == "f32" else np.uint16)


def test_pool_permutation_distinct_per_request():
    b = synth.make_batch("mini_bf16_dev_pool")
    ids = b.chunk_table[:, 4].reshape(b.n_req, -1)
    for r in range(b.n_req):
        assert len(set(ids[r].tolist())) == ids.shape[1]
    assert not all(np.array_equal(ids[0], ids[r]) for r in range(1, b.n_req))


def test_bf16_encoding_rounds_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0029296875, -2.5], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    assert back.tolist() == [1.0, 1.0, 1.0078125, 1.0, -2.5]


@pytest.mark.parametrize("name", ["mini_bf16_seam", "mini_bf16_dev_pool", "qwen3_8b_anchor"])
def test_chunk_spans_tile_the_context(name):
    b = synth.make_batch(name) if name.startswith("mini") else None
    if b is None:
        wl = synth.get_workload(name)
        # layout only: the spans follow the workload's chunk lengths
        import dataclasses
        b = synth.make_batch(dataclasses.replace(wl, hidden=64, n_q_heads=1, n_kv_heads=1,
                                                 head_dim=64))
    for r in range(b.n_req):
        spans = b.chunk_spans(r)
        assert [ln for _, ln in spans] == list(b.wl.chunk_lens)
        pos = 0
        for p, ln in spans:
            assert p == pos
            pos += ln
        assert pos == int(b.n_ctx[r])
