"""Seeded synthetic inputs for the fused-layer path.

This module draws random numbers and lays out index arrays; it holds none of
the fusion method's arithmetic (no projection, rotation, scoring, selection or
attention).  Both the HIP path and the CPU oracle consume what it returns.

Workload shapes follow the RAG cache-fusion setting of the QCFuse page
("QCFuse: Query-Aware Cache Fusion via Compressed View for Efficient RAG
Serving", section 2.1.1, Eq. 1): a request is a context C = [c_1; ...; c_m] of
retrieved chunks followed by the user query U.  Every chunk has a *cached*
hidden state (what the chunk looked like when its cache was built in
isolation) and a *fresh* hidden state (what the same tokens look like inside
the current request).  The first chunk of a request has no preceding context,
so its cached and fresh hidden states are identical.

Random tensors are keyed by (seed, tensor name, request, slot) through
numpy SeedSequence, so the order in which they are drawn does not matter.
Floating-point tensors are returned in their storage encoding: float32 arrays
for fp32 workloads, uint16 bf16 bit patterns (round-to-nearest-even from
float32) for bf16 workloads.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import List, Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16"
    n_req: int
    chunk_lens: tuple          # token count of every context chunk slot
    n_query: tuple             # query tokens per request (len n_req) or 1-tuple
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rope_base: float
    score: str                 # "deviation" or "attn_mass"
    ratio_pct: tuple           # recompute ratios in percent
    sigma: float               # cached-hidden perturbation of non-first chunks
    pool_chunks: int = 0       # >0: chunks drawn from a shared pool of this size
    kivi_bits: int = 0         # cached K/V stored as KIVI codes of 8 or 4 bits (0: dense)
    resident: str = ""         # fused cache format: "" bf16/f32 as dtype, "q8" int8-resident
    seed: int = 0
    description: str = ""
    # selector feeding the recompute path: "score" (top-k of `score`, with
    # static_rules as a forced set when any is nonzero), "static" (exactly the
    # static_rules positions) or "anchor" (per-chunk top-k of the key norm,
    # ceil(anchor_pct / 100 * chunk length) per chunk)
    selector: str = "score"
    static_rules: tuple = (0, 0, 0)     # (sink, boundary, seam)
    anchor_pct: int = 0
    # several layers, each with its own weights, hidden states and per-chunk
    # caches (drawn independently).  signal: "" (every layer selects on its
    # own score), "sum" (one selection for all layers from the score summed
    # over score_layers, all layers when empty) or "progressive" (layer l
    # keeps progressive_pct[l] % of N out of layer l-1's picks).
    # stream_pools: the per-chunk caches stay in pinned host memory and every
    # layer's cache is copied in on a second stream while earlier layers run.
    n_layers: int = 1
    signal: str = ""
    score_layers: tuple = ()
    progressive_pct: tuple = ()
    stream_pools: bool = False

    @property
    def n_chunks(self) -> int:
        return len(self.chunk_lens)

    def query_len(self, r: int) -> int:
        return self.n_query[r] if len(self.n_query) > 1 else self.n_query[0]


def _wl(**kw) -> Workload:
    return Workload(**kw)


WORKLOADS = {
    # 4 chunks x 64 + 32 query tokens, fp32, deviation score, r = 30%.
    "tiny_fp32_dev": _wl(
        name="tiny_fp32_dev", dtype="f32", n_req=1, chunk_lens=(64,) * 4,
        n_query=(32,), hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64,
        rope_base=1e4, score="deviation", ratio_pct=(30,), sigma=0.1,
        description="tiny fp32 layer, 4x64 context + 32 query tokens"),
    # Qwen3-8B-shaped layer, 10 x 512 + 64 query, attention-mass score, r = 30%.
    "qwen3_8b_mass": _wl(
        name="qwen3_8b_mass", dtype="bf16", n_req=1, chunk_lens=(512,) * 10,
        n_query=(64,), hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
        rope_base=1e6, score="attn_mass", ratio_pct=(30,), sigma=0.1,
        description="Qwen3-8B-shaped layer, bf16, 1 request of 10x512 + 64 query"),
    # Same layer, 8 requests of 20 x 512 + 128 drawn from a 64-chunk pool.
    "qwen3_8b_dev_pool": _wl(
        name="qwen3_8b_dev_pool", dtype="bf16", n_req=8, chunk_lens=(512,) * 20,
        n_query=(128,), hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
        rope_base=1e6, score="deviation", ratio_pct=(15, 30), sigma=0.1,
        pool_chunks=64,
        description="Qwen3-8B-shaped layer, bf16, 8 requests of 20x512 + 128 "
                    "query from a 64-chunk pool"),
    # Llama-3-70B-shaped layer, 32 x 1024 + 256 query, attention mass, r = 20%.
    "llama3_70b_mass": _wl(
        name="llama3_70b_mass", dtype="bf16", n_req=1, chunk_lens=(1024,) * 32,
        n_query=(256,), hidden=8192, n_q_heads=64, n_kv_heads=8, head_dim=128,
        rope_base=5e5, score="attn_mass", ratio_pct=(20,), sigma=0.05,
        description="Llama-3-70B-shaped layer, bf16, 1 request of 32x1024 + 256 query"),
    # The Qwen3-8B-shaped request with static selection: KVBoost's seam
    # windows (R = 16) plus 4 attention-sink tokens.
    "qwen3_8b_seam": _wl(
        name="qwen3_8b_seam", dtype="bf16", n_req=1, chunk_lens=(512,) * 10,
        n_query=(64,), hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
        rope_base=1e6, score="attn_mass", ratio_pct=(0,), sigma=0.1,
        selector="static", static_rules=(4, 0, 16),
        description="Qwen3-8B-shaped layer, bf16, 1 request of 10x512 + 64 query, "
                    "static selection (seam windows R=16, 4 sink tokens)"),
    # The same request with per-chunk key-norm anchors, r_a = 10%.
    "qwen3_8b_anchor": _wl(
        name="qwen3_8b_anchor", dtype="bf16", n_req=1, chunk_lens=(512,) * 10,
        n_query=(64,), hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
        rope_base=1e6, score="attn_mass", ratio_pct=(0,), sigma=0.1,
        selector="anchor", anchor_pct=10,
        description="Qwen3-8B-shaped layer, bf16, 1 request of 10x512 + 64 query, "
                    "per-chunk key-norm anchors (r_a = 10%) as the recompute set"),
    # Several Qwen3-8B-shaped layers over the headline request: the attention
    # mass summed over all 4 layers (ProphetKV's full view), over 3 of 8
    # layers (QCFuse's critical set), CacheBlend's filtering over 3 layers,
    # and 4 independent layers whose caches stream in from host memory.
    "qwen3_8b_prophet4": _wl(
        name="qwen3_8b_prophet4", dtype="bf16", n_req=1, chunk_lens=(512,) * 10,
        n_query=(64,), hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
        rope_base=1e6, score="attn_mass", ratio_pct=(30,), sigma=0.1,
        n_layers=4, signal="sum",
        description="4 Qwen3-8B-shaped layers, bf16, 1 request of 10x512 + 64 query, "
                    "one selection from the attention mass summed over all 4 layers"),
    "qwen3_8b_critical3": _wl(
        name="qwen3_8b_critical3", dtype="bf16", n_req=1, chunk_lens=(512,) * 10,
        n_query=(64,), hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
        rope_base=1e6, score="attn_mass", ratio_pct=(30,), sigma=0.1,
        n_layers=8, signal="sum", score_layers=(3, 4, 5),
        description="8 Qwen3-8B-shaped layers, bf16, 1 request of 10x512 + 64 query, "
                    "one selection from the attention mass summed over layers 3-5"),
    "qwen3_8b_dev_progressive": _wl(
        name="qwen3_8b_dev_progressive", dtype="bf16", n_req=1, chunk_lens=(512,) * 10,
        n_query=(64,), hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
        rope_base=1e6, score="deviation", ratio_pct=(30,), sigma=0.1,
        n_layers=3, signal="progressive", progressive_pct=(50, 40, 30),
        description="3 Qwen3-8B-shaped layers, bf16, 1 request of 10x512 + 64 query, "
                    "deviation candidates narrowed 50% -> 40% -> 30% layer by layer"),
    "qwen3_8b_mass_stream4": _wl(
        name="qwen3_8b_mass_stream4", dtype="bf16", n_req=1, chunk_lens=(512,) * 10,
        n_query=(64,), hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128,
        rope_base=1e6, score="attn_mass", ratio_pct=(30,), sigma=0.1,
        n_layers=4, stream_pools=True,
        description="4 Qwen3-8B-shaped layers, bf16, 1 request of 10x512 + 64 query, "
                    "per-chunk caches streamed from pinned host memory layer by layer"),
    # Qwen2.5-3B-shaped layer, int8 KIVI cache, 16 requests of 24 x 128 + 64.
    "qwen25_3b_kivi8": _wl(
        name="qwen25_3b_kivi8", dtype="bf16", n_req=16, chunk_lens=(128,) * 24,
        n_query=(64,), hidden=2048, n_q_heads=16, n_kv_heads=2, head_dim=128,
        rope_base=1e6, score="deviation", ratio_pct=(15,), sigma=0.1,
        kivi_bits=8,
        description="Qwen2.5-3B-shaped layer, bf16 + int8 KIVI cache, 16 requests "
                    "of 24x128 + 64 query"),
    # The same layer and data with the fused cache itself held as 8-bit codes
    # (int8-resident: the scores and the attention decode on load).
    "qwen25_3b_kivi8_resident": _wl(
        name="qwen25_3b_kivi8_resident", dtype="bf16", n_req=16, chunk_lens=(128,) * 24,
        n_query=(64,), hidden=2048, n_q_heads=16, n_kv_heads=2, head_dim=128,
        rope_base=1e6, score="deviation", ratio_pct=(15,), sigma=0.1,
        kivi_bits=8, resident="q8",
        description="Qwen2.5-3B-shaped layer, bf16 + int8 KIVI cache, int8-resident fused "
                    "cache, 16 requests of 24x128 + 64 query"),
    # The same with 4-bit KIVI codes (KVBoost's int4 setting).
    "qwen25_3b_kivi4": _wl(
        name="qwen25_3b_kivi4", dtype="bf16", n_req=16, chunk_lens=(128,) * 24,
        n_query=(64,), hidden=2048, n_q_heads=16, n_kv_heads=2, head_dim=128,
        rope_base=1e6, score="deviation", ratio_pct=(15,), sigma=0.1,
        kivi_bits=4,
        description="Qwen2.5-3B-shaped layer, bf16 + int4 KIVI cache, 16 requests "
                    "of 24x128 + 64 query"),
}

# Small workloads for parity tests: several tiles, ragged chunk and query
# lengths, every score mode and storage format.
MINI_WORKLOADS = {
    "mini_bf16_mass": _wl(
        name="mini_bf16_mass", dtype="bf16", n_req=2, chunk_lens=(97, 130, 64, 33),
        n_query=(19, 40), hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
        rope_base=1e6, score="attn_mass", ratio_pct=(30,), sigma=0.1),
    "mini_bf16_dev_pool": _wl(
        name="mini_bf16_dev_pool", dtype="bf16", n_req=3, chunk_lens=(70, 70, 70, 70),
        n_query=(21,), hidden=384, n_q_heads=4, n_kv_heads=4, head_dim=128,
        rope_base=1e6, score="deviation", ratio_pct=(30,), sigma=0.1,
        pool_chunks=6),
    "mini_bf16_kivi8": _wl(
        name="mini_bf16_kivi8", dtype="bf16", n_req=2, chunk_lens=(128, 45, 128),
        n_query=(33, 7), hidden=256, n_q_heads=8, n_kv_heads=1, head_dim=128,
        rope_base=1e6, score="deviation", ratio_pct=(15,), sigma=0.1, kivi_bits=8),
    "mini_bf16_kivi8_resident": _wl(
        name="mini_bf16_kivi8_resident", dtype="bf16", n_req=2, chunk_lens=(128, 45, 128),
        n_query=(33, 7), hidden=256, n_q_heads=8, n_kv_heads=1, head_dim=128,
        rope_base=1e6, score="deviation", ratio_pct=(15,), sigma=0.1, kivi_bits=8,
        resident="q8"),
    "mini_bf16_dense_resident": _wl(
        name="mini_bf16_dense_resident", dtype="bf16", n_req=3, chunk_lens=(70, 70, 70, 70),
        n_query=(21,), hidden=384, n_q_heads=4, n_kv_heads=2, head_dim=64,
        rope_base=1e6, score="deviation", ratio_pct=(30,), sigma=0.1, resident="q8"),
    "mini_bf16_kivi4": _wl(
        name="mini_bf16_kivi4", dtype="bf16", n_req=2, chunk_lens=(128, 45, 128),
        n_query=(33, 7), hidden=256, n_q_heads=8, n_kv_heads=1, head_dim=128,
        rope_base=1e6, score="deviation", ratio_pct=(15,), sigma=0.1, kivi_bits=4),
    "mini_bf16_d64_mass": _wl(
        name="mini_bf16_d64_mass", dtype="bf16", n_req=1, chunk_lens=(50, 77, 61),
        n_query=(45,), hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
        rope_base=1e4, score="attn_mass", ratio_pct=(20,), sigma=0.1),
    "mini_bf16_seam": _wl(
        name="mini_bf16_seam", dtype="bf16", n_req=2, chunk_lens=(97, 130, 64, 33),
        n_query=(19, 40), hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
        rope_base=1e6, score="attn_mass", ratio_pct=(0,), sigma=0.1,
        selector="static", static_rules=(3, 2, 16)),
    "mini_bf16_anchor": _wl(
        name="mini_bf16_anchor", dtype="bf16", n_req=2, chunk_lens=(97, 130, 64, 33),
        n_query=(19, 40), hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
        rope_base=1e6, score="attn_mass", ratio_pct=(0,), sigma=0.1,
        selector="anchor", anchor_pct=15),
    "mini_bf16_dev_sink": _wl(
        name="mini_bf16_dev_sink", dtype="bf16", n_req=3, chunk_lens=(70, 70, 70, 70),
        n_query=(21,), hidden=384, n_q_heads=4, n_kv_heads=4, head_dim=128,
        rope_base=1e6, score="deviation", ratio_pct=(30,), sigma=0.1,
        pool_chunks=6, static_rules=(4, 1, 0)),
    "mini_bf16_mass_sum3": _wl(
        name="mini_bf16_mass_sum3", dtype="bf16", n_req=2, chunk_lens=(97, 130, 64, 33),
        n_query=(19, 40), hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
        rope_base=1e6, score="attn_mass", ratio_pct=(30,), sigma=0.1,
        n_layers=4, signal="sum", score_layers=(1, 3)),
    "mini_bf16_dev_progressive": _wl(
        name="mini_bf16_dev_progressive", dtype="bf16", n_req=3, chunk_lens=(70, 70, 70, 70),
        n_query=(21,), hidden=384, n_q_heads=4, n_kv_heads=4, head_dim=128,
        rope_base=1e6, score="deviation", ratio_pct=(30,), sigma=0.1,
        pool_chunks=6, n_layers=3, signal="progressive", progressive_pct=(60, 45, 30)),
    "mini_bf16_mass_stream": _wl(
        name="mini_bf16_mass_stream", dtype="bf16", n_req=2, chunk_lens=(97, 130, 64, 33),
        n_query=(19, 40), hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
        rope_base=1e6, score="attn_mass", ratio_pct=(30,), sigma=0.1,
        n_layers=5, stream_pools=True),
    "mini_f32_mass": _wl(
        name="mini_f32_mass", dtype="f32", n_req=2, chunk_lens=(40, 23, 64),
        n_query=(9, 30), hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=64,
        rope_base=1e4, score="attn_mass", ratio_pct=(30,), sigma=0.1),
}


def get_workload(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name in MINI_WORKLOADS:
        return MINI_WORKLOADS[name]
    raise KeyError(f"unknown workload {name!r}")


# ----------------------------------------------------------------------------
# storage encodings
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even: add
    0x7FFF plus the lowest kept bit, then drop the low 16 bits.  Works in
    blocks of 2^20 values so large tensors stay cache-sized."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 20
    t = np.empty(min(step, max(u.size, 1)), dtype=np.uint32)
    for i in range(0, u.size, step):
        uc = u[i:i + step]
        tc = t[:uc.size]
        np.right_shift(uc, 16, out=tc)
        np.bitwise_and(tc, 1, out=tc)
        np.add(tc, uc, out=tc)
        np.add(tc, np.uint32(0x7FFF), out=tc)
        np.right_shift(tc, 16, out=tc)
        out[i:i + step] = tc
    return out.reshape(x.shape)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def _encode_rows(x: np.ndarray, dtype: str) -> np.ndarray:
    """encode() of a 2-D array, row blocks in parallel."""
    if dtype != "bf16" or x.ndim != 2 or x.shape[0] < 64:
        return encode(x, dtype)
    out = np.empty(x.shape, dtype=np.uint16)
    step = max(1, x.shape[0] // 32)

    def one(i):
        out[i:i + step] = f32_to_bf16_bits(x[i:i + step])
    list(_pool().map(one, range(0, x.shape[0], step)))
    return out


# ----------------------------------------------------------------------------
# random streams
# ----------------------------------------------------------------------------
def _rng(seed: int, name: str, *keys: int) -> np.random.Generator:
    tag = zlib.crc32(name.encode())
    return np.random.default_rng(np.random.SeedSequence([seed, tag, *keys]))


def _pool():
    """Thread pool for independent seeded draws (one per process)."""
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import os
        n = min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 8)
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=max(1, n))
    return _POOL


_POOL = None


def _normal(seed: int, name: str, shape, *keys: int, std: float = 1.0) -> np.ndarray:
    g = _rng(seed, name, *keys)
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


# ----------------------------------------------------------------------------
# generated request batch
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Batch:
    wl: Workload
    # layout
    cu_T: np.ndarray            # int32 [n_req+1] row offset of each request
    n_ctx: np.ndarray           # int32 [n_req]  context tokens N_r
    chunk_table: np.ndarray     # int32 [n_chunks_total, 8]: src_row, dst_row,
                                #   pos0, len, pool_chunk, 0, 0, 0
    pool_cu: np.ndarray         # int32 [n_pool+1] first row of every pool chunk
    pool_pos: np.ndarray        # int32 [pool_rows] chunk-local position of each
                                #   pool row (0..len-1)
    # tensors in storage encoding
    pool_hidden: np.ndarray     # [pool_rows, hidden] cached hidden states
    x: np.ndarray               # [sum T, hidden] fresh hidden states
    w_qkv: np.ndarray           # [(Hq + 2 Hkv) d, hidden]; rows = [Wq; Wk; Wv]

    @property
    def n_req(self) -> int:
        return self.wl.n_req

    @property
    def total_rows(self) -> int:
        return int(self.cu_T[-1])

    @property
    def pool_rows(self) -> int:
        return int(self.pool_cu[-1])

    def n_query(self, r: int) -> int:
        return int(self.cu_T[r + 1] - self.cu_T[r] - self.n_ctx[r])

    def query_rows(self) -> np.ndarray:
        """Flat rows (into x / the fused cache) of every query token."""
        return np.concatenate([
            np.arange(self.cu_T[r] + self.n_ctx[r], self.cu_T[r + 1], dtype=np.int32)
            for r in range(self.n_req)])

    def query_pos(self) -> np.ndarray:
        """Request positions of every query token (N_r .. T_r - 1)."""
        return np.concatenate([
            np.arange(self.n_ctx[r], self.cu_T[r + 1] - self.cu_T[r], dtype=np.int32)
            for r in range(self.n_req)])

    def context_rows(self) -> np.ndarray:
        return np.concatenate([
            np.arange(self.cu_T[r], self.cu_T[r] + self.n_ctx[r], dtype=np.int32)
            for r in range(self.n_req)])

    def context_pos(self) -> np.ndarray:
        return np.concatenate([np.arange(self.n_ctx[r], dtype=np.int32)
                               for r in range(self.n_req)])

    def all_pos(self) -> np.ndarray:
        return np.concatenate([np.arange(self.cu_T[r + 1] - self.cu_T[r], dtype=np.int32)
                               for r in range(self.n_req)])

    def chunk_spans(self, r: int):
        """(start position, length) of every stitched chunk of request r,
        ascending."""
        t = self.chunk_table
        mine = t[(t[:, 1] >= self.cu_T[r]) & (t[:, 1] < self.cu_T[r] + self.n_ctx[r])]
        mine = mine[np.argsort(mine[:, 1], kind="stable")]
        return [(int(row[1] - self.cu_T[r]), int(row[3])) for row in mine]


def _chunk_ids(wl: Workload, r: int) -> List[int]:
    """Pool chunk used by every slot of request r."""
    if wl.pool_chunks:
        perm = _rng(wl.seed, "pool_permutation", r).permutation(wl.pool_chunks)
        return [int(c) for c in perm[: wl.n_chunks]]
    return [r * wl.n_chunks + s for s in range(wl.n_chunks)]


def layer_seed(wl: Workload, layer: int) -> int:
    """Seed of layer `layer` of a multi-layer workload (layer 0 keeps the
    workload's own seed, so it is the one-layer batch)."""
    return wl.seed + 1000003 * layer


def make_layer_batches(wl: Workload | str) -> List["Batch"]:
    """One batch per layer: the same request layout, independent weights,
    hidden states and per-chunk caches."""
    if isinstance(wl, str):
        wl = get_workload(wl)
    return [make_batch(wl, seed=layer_seed(wl, l)) for l in range(wl.n_layers)]


def make_batch(wl: Workload | str, seed: Optional[int] = None) -> Batch:
    """Draw one synthetic request batch for workload `wl`.

    Non-pool workloads: fresh context hidden X ~ N(0, 1) per slot; the cached
    hidden of slot s >= 1 is X + sigma * N(0, 1); slot 0 caches X itself.
    Pool workloads: pool chunk c has cached hidden H_c ~ N(0, 1); request r uses
    fresh X = H_c in slot 0 and X = H_c + sigma * N(0, 1) in every later slot.
    Query hidden ~ N(0, 1).  Weights ~ N(0, 1/hidden).
    """
    if isinstance(wl, str):
        wl = get_workload(wl)
    if seed is not None:
        wl = dataclasses.replace(wl, seed=seed)
    sd = wl.seed
    m = wl.n_chunks
    lens = list(wl.chunk_lens)
    n_ctx = sum(lens)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)

    # pool layout: every pool chunk id -> its length
    if wl.pool_chunks:
        if len(set(lens)) != 1:
            raise ValueError("pool workloads need equal chunk lengths")
        n_pool = wl.pool_chunks
        pool_len = [lens[0]] * n_pool
    else:
        n_pool = wl.n_req * m
        pool_len = [lens[s] for _ in range(wl.n_req) for s in range(m)]
    pool_cu = np.concatenate([[0], np.cumsum(pool_len)]).astype(np.int32)
    pool_pos = np.concatenate([np.arange(n, dtype=np.int32) for n in pool_len])

    tq = [wl.query_len(r) for r in range(wl.n_req)]
    T = [n_ctx + q for q in tq]
    cu_T = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    total = int(cu_T[-1])

    H = wl.hidden
    x = np.empty((total, H), dtype=np.float32)
    pool_hidden = np.empty((int(pool_cu[-1]), H), dtype=np.float32)
    # Every draw has its own key, so the draws run on a thread pool (the
    # generator releases the GIL) without changing any value.
    pool = _pool()

    if wl.pool_chunks:
        def fill_pool(c):
            pool_hidden[pool_cu[c]:pool_cu[c + 1]] = _normal(sd, "pool_hidden", (pool_len[c], H), c)
        list(pool.map(fill_pool, range(n_pool)))

    table = []
    jobs = []
    for r in range(wl.n_req):
        ids = _chunk_ids(wl, r)
        for s in range(m):
            c = ids[s]
            rows = slice(int(cu_T[r] + starts[s]), int(cu_T[r] + starts[s + 1]))
            jobs.append((r, s, c, rows))
            table.append([int(pool_cu[c]), rows.start, int(starts[s]), lens[s], c, 0, 0, 0])

    def fill_slot(job):
        r, s, c, rows = job
        if wl.pool_chunks:
            base = pool_hidden[pool_cu[c]:pool_cu[c + 1]]
            if s == 0:
                x[rows] = base
            else:
                x[rows] = base + np.float32(wl.sigma) * _normal(sd, "fresh_noise", base.shape, r, s)
        else:
            fresh = _normal(sd, "fresh_hidden", (lens[s], H), r, s)
            x[rows] = fresh
            if s == 0:
                pool_hidden[pool_cu[c]:pool_cu[c + 1]] = fresh
            else:
                pool_hidden[pool_cu[c]:pool_cu[c + 1]] = fresh + np.float32(wl.sigma) * _normal(
                    sd, "cached_noise", fresh.shape, r, s)

    def fill_query(r):
        x[cu_T[r] + n_ctx:cu_T[r + 1]] = _normal(sd, "query_hidden", (tq[r], H), r)

    list(pool.map(fill_slot, jobs))
    list(pool.map(fill_query, range(wl.n_req)))

    n_out = (wl.n_q_heads + 2 * wl.n_kv_heads) * wl.head_dim
    w = _normal(sd, "w_qkv", (n_out, H), std=1.0 / np.sqrt(H))

    return Batch(
        wl=wl,
        cu_T=cu_T,
        n_ctx=np.full(wl.n_req, n_ctx, dtype=np.int32),
        chunk_table=np.asarray(table, dtype=np.int32).reshape(-1, 8),
        pool_cu=pool_cu,
        pool_pos=pool_pos,
        pool_hidden=_encode_rows(pool_hidden, wl.dtype),
        x=_encode_rows(x, wl.dtype),
        w_qkv=_encode_rows(w, wl.dtype),
    )


def random_scores(n: int, seed: int, ties: int = 0, distinct_levels: Optional[int] = None) -> np.ndarray:
    """float32 scores for selection tests; optionally with forced ties."""
    g = _rng(seed, "scores", n)
    if distinct_levels:
        s = g.integers(0, distinct_levels, size=n).astype(np.float32) / np.float32(distinct_levels)
    else:
        s = g.standard_normal(n).astype(np.float32)
    if ties and n > 1:
        idx = g.choice(n, size=min(ties, n), replace=False)
        s[idx] = s[idx[0]]
    return s


def random_normal(shape: Sequence[int], seed: int, name: str = "tensor", std: float = 1.0) -> np.ndarray:
    """Plain float32 N(0, std^2) tensor for stage-isolated tests."""
    return _normal(seed, name, tuple(shape), std=std)


def random_codes(shape: Sequence[int], seed: int, name: str = "codes") -> np.ndarray:
    return _rng(seed, name).integers(0, 256, size=tuple(shape), dtype=np.uint8)


def random_rows(n_total: int, count: int, seed: int, name: str = "rows") -> np.ndarray:
    """`count` distinct row indices in [0, n_total), ascending."""
    g = _rng(seed, name, n_total, count)
    return np.sort(g.choice(n_total, size=count, replace=False)).astype(np.int32)
