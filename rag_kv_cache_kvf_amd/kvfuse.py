"""ctypes binding of libkvfuse (include/kvfuse.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and the current HIP stream to
the C entry point of the same name, and raises KvfError on a non-OK status.
Nothing here computes; the library must be built (`__graft_entry__.build()`)
or importing this module fails.
"""
from __future__ import annotations

import contextlib
import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

# KVF_LIBRARY selects another build of the same library (an instrumented
# one, say); by default the one built in this directory.
_LIB_PATH = os.environ.get("KVF_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libkvfuse.so")

KVF_OK, KVF_ERR_INVALID_ARG, KVF_ERR_UNSUPPORTED, KVF_ERR_WORKSPACE, KVF_ERR_HIP = range(5)
KVF_F32, KVF_BF16 = 0, 1
KVF_SCORE_DEVIATION, KVF_SCORE_ATTN_MASS, KVF_SCORE_KEY_NORM = 0, 1, 2
KVF_SCORE_ACCUMULATE = 0x100
KVF_OUT_Q, KVF_OUT_K, KVF_OUT_V = 1, 2, 4
KVF_MAX_REQ = 64


class KvfError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {status_name(status)}: {msg}")
        self.status = status


def load_library(path: str = _LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libkvfuse is not built ({path} missing); run __graft_entry__.build()")
    return ctypes.CDLL(path)


_lib = load_library()


# ----------------------------------------------------------------------------
# C structs
# ----------------------------------------------------------------------------
class LayerDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class BatchDesc(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("cu_T", ctypes.POINTER(ctypes.c_int32)),
                ("n_ctx", ctypes.POINTER(ctypes.c_int32))]


class KiviDesc(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_min", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_min", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("n_pool_chunks", ctypes.c_int32), ("bits", ctypes.c_int32)]


class Q8CacheDesc(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_stats", ctypes.c_void_p), ("v_stats", ctypes.c_void_p),
                ("rows", ctypes.c_int64)]


class StaticRules(ctypes.Structure):
    _fields_ = [("sink", ctypes.c_int32), ("boundary", ctypes.c_int32), ("seam", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_LP = ctypes.POINTER(LayerDesc)
_BP = ctypes.POINTER(BatchDesc)
_IP = ctypes.POINTER(ctypes.c_int32)

_SIGS = {
    "kvf_rope_table": (_I32, [ctypes.c_double, _I32, _I32, _P, _P, _P]),
    "kvf_rerotate": (_I32, [_LP, _P, _I32, _I32, _P, _P, ctypes.POINTER(KiviDesc), _I64, _P, _P,
                            _I32, _P, _P, _I64, _I32, _P]),
    "kvf_rerotate_deviation": (_I32, [_LP, _BP, _P, _I32, _I32, _P, _P, ctypes.POINTER(KiviDesc), _I64,
                                      _P, _P, _I32, _P, _P, _I64, _I32, _P, _P, _I32, _P, _P]),
    "kvf_score": (_I32, [_I32, _LP, _BP, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "kvf_rerotate_score_attn_mass": (_I32, [_LP, _BP, _P, _I32, _I32, _P, _I64, _P, _P, _I32, _P, _I64,
                                            _P, _I32, _P, _I32, _P, _P, _SZ, _P]),
    "kvf_score_workspace_size": (_SZ, [_I32, _LP, _BP, _I32]),
    "kvf_score_attn_mass_noalloc": (_I32, [_LP, _BP, _P, _P, _I32, _P, _P, _I32, _P]),
    "kvf_select_topk": (_I32, [_P, _P, _BP, _IP, _P, _P, _P, _P, _P, _SZ, _P]),
    "kvf_select_topk_segmented": (_I32, [_P, _P, _BP, _P, _I32, _IP, _P, _P, _P, _P]),
    "kvf_select_static": (_I32, [_BP, _P, _I32, ctypes.POINTER(StaticRules), _P, _P]),
    "kvf_static_counts": (_I32, [_BP, _P, _I32, ctypes.POINTER(StaticRules), _IP]),
    "kvf_select_workspace_size": (_SZ, [_BP]),
    "kvf_recompute_qkv": (_I32, [_LP, _P, _I64, _P, _P, _I32, _P, ctypes.c_uint32, _P, _P, _I32,
                                 _P, _P, _P, _P, _I64, _P, _SZ, _P]),
    "kvf_recompute_workspace_size": (_SZ, [_LP, _I32, ctypes.c_uint32]),
    "kvf_scatter_kv": (_I32, [_LP, _P, _P, _I64, _P, _P, _I64, _P, _I32, _P, _P, _I64, _P]),
    "kvf_sparse_q_attention": (_I32, [_LP, _BP, _P, _P, _IP, _P, _P, ctypes.c_float, _P, _P, _P,
                                      _SZ, _P]),
    "kvf_attention_workspace_size": (_SZ, [_LP, _BP, _IP]),
    "kvf_rerotate_q8": (_I32, [_LP, _P, _I32, _I32, _P, _P, ctypes.POINTER(KiviDesc), _I64, _P, _P,
                               _I32, ctypes.POINTER(Q8CacheDesc), _P]),
    "kvf_rerotate_q8_deviation": (_I32, [_LP, _BP, _P, _I32, _I32, _P, _P, ctypes.POINTER(KiviDesc),
                                         _I64, _P, _P, _I32, ctypes.POINTER(Q8CacheDesc), _P, _P,
                                         _I32, _P, _P]),
    "kvf_score_q8": (_I32, [_I32, _LP, _BP, ctypes.POINTER(Q8CacheDesc), _P, _P, _P, _P]),
    "kvf_scatter_kv_q8": (_I32, [_LP, _P, _P, _I64, _P, _P, _I64, _P, _I32,
                                 ctypes.POINTER(Q8CacheDesc), _P]),
    "kvf_sparse_q_attention_q8": (_I32, [_LP, _BP, _P, _P, _IP, ctypes.POINTER(Q8CacheDesc),
                                         ctypes.c_float, _P, _P, _P, _SZ, _P]),
    "kvf_kivi_encode": (_I32, [_LP, _P, _P, _P, _I32, _I64, _I32, ctypes.POINTER(KiviDesc), _P]),
    "kvf_recompute_budget": (_I32, [_I32, _I32]),
    "kvf_anchor_budget": (_I32, [_I32, _I32, _I32]),
    "kvf_status_string": (ctypes.c_char_p, [_I32]),
    "kvf_last_error": (ctypes.c_char_p, []),
    "kvf_abi_version": (_I32, []),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def status_name(status: int) -> str:
    return _lib.kvf_status_string(status).decode()


def last_error() -> str:
    return _lib.kvf_last_error().decode()


def abi_version() -> int:
    return _lib.kvf_abi_version()


def recompute_budget(n_ctx: int, ratio_pct: int) -> int:
    return _lib.kvf_recompute_budget(n_ctx, ratio_pct)


def anchor_budget(length: int, ra_num: int, ra_den: int) -> int:
    return _lib.kvf_anchor_budget(length, ra_num, ra_den)


def _check(status: int, func: str):
    if status != KVF_OK:
        raise KvfError(status, func, last_error())


# ----------------------------------------------------------------------------
# prepared calls: the arguments of a call marshalled once
# ----------------------------------------------------------------------------
class Prepared:
    """One library call with its arguments converted once (device pointers,
    ctypes structs and arrays); calling it runs the C entry point on the
    current HIP stream, or on `stream`.  The tensors behind the pointers
    must stay alive and keep their storage while it is used; `keep` holds
    the ones the binding created itself."""
    __slots__ = ("fn", "args", "name", "keep")

    def __init__(self, fn, args, name, keep=()):
        self.fn, self.args, self.name, self.keep = fn, args, name, keep

    def __call__(self, stream=None):
        _check(self.fn(*self.args, _stream(stream)), self.name)


_preparing = False


@contextlib.contextmanager
def preparing():
    """Inside this context the entry points below return a Prepared call
    instead of running it."""
    global _preparing
    old, _preparing = _preparing, True
    try:
        yield
    finally:
        _preparing = old


def _run(fn, args: tuple, name: str, stream, keep=()):
    if _preparing:
        return Prepared(fn, args, name, keep)
    _check(fn(*args, _stream(stream)), name)
    return None


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Layer:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str          # "f32" | "bf16"

    def desc(self) -> LayerDesc:
        return LayerDesc(self.hidden, self.n_q_heads, self.n_kv_heads, self.head_dim,
                         KVF_BF16 if self.dtype == "bf16" else KVF_F32)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


class Batch:
    """Host-side request layout (cu_T, n_ctx) held as ctypes arrays."""

    def __init__(self, cu_T: Sequence[int], n_ctx: Sequence[int]):
        self.cu_T_list = [int(v) for v in cu_T]
        self.n_ctx_list = [int(v) for v in n_ctx]
        n = len(self.n_ctx_list)
        self._cu = (ctypes.c_int32 * (n + 1))(*self.cu_T_list)
        self._nc = (ctypes.c_int32 * max(n, 1))(*self.n_ctx_list)
        self.desc = BatchDesc(n, ctypes.cast(self._cu, _IP), ctypes.cast(self._nc, _IP))

    @property
    def n_req(self) -> int:
        return len(self.n_ctx_list)

    def n_query(self, r: int) -> int:
        return self.cu_T_list[r + 1] - self.cu_T_list[r] - self.n_ctx_list[r]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _int_array(vals: Sequence[int]):
    return (ctypes.c_int32 * max(len(vals), 1))(*[int(v) for v in vals])


def _rows(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else int(t.shape[0])


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------
def rope_table(base: float, head_dim: int, n_pos: int, cos_out: torch.Tensor,
               sin_out: torch.Tensor, stream=None):
    return _run(_lib.kvf_rope_table, (float(base), head_dim, n_pos, _ptr(cos_out), _ptr(sin_out)),
                "kvf_rope_table", stream)


def rerotate(layer: Layer, chunks: torch.Tensor, max_chunk_len: int,
             pool_k: Optional[torch.Tensor], pool_v: Optional[torch.Tensor],
             rope_cos: torch.Tensor, rope_sin: torch.Tensor, fused_k: torch.Tensor,
             fused_v: Optional[torch.Tensor], kivi: Optional[dict] = None, k_only: bool = False,
             stream=None):
    """chunks: int32 [n_chunks, 8] device tensor (kvf_chunk rows).
    kivi: dict of k_codes, v_codes ([rows, Hkv, d * bits / 8] uint8), k_min,
    k_scale ([n_pool, Hkv, d]), v_min, v_scale ([rows, Hkv]); the code width
    follows from the shapes.  k_only: keys only (values already in place;
    pool_v / fused_v unused; pool_k may be fused_k)."""
    kd = None
    pool_rows = _rows(pool_k)
    if kivi is not None:
        kd = ctypes.byref(_kivi_desc(kivi))
        pool_rows = int(kivi["k_codes"].shape[0])
    d = layer.desc()
    return _run(_lib.kvf_rerotate, (ctypes.byref(d), _ptr(chunks), int(chunks.shape[0]), max_chunk_len,
                             _ptr(pool_k), _ptr(pool_v), kd, pool_rows, _ptr(rope_cos),
                             _ptr(rope_sin), int(rope_cos.shape[0]), _ptr(fused_k), _ptr(fused_v),
                             _rows(fused_k), 1 if k_only else 0), "kvf_rerotate", stream)


def rerotate_deviation(layer: Layer, batch: Batch, chunks: torch.Tensor, max_chunk_len: int,
                       pool_k: Optional[torch.Tensor], pool_v: Optional[torch.Tensor],
                       rope_cos: torch.Tensor, rope_sin: torch.Tensor, fused_k: torch.Tensor,
                       fused_v: Optional[torch.Tensor], k_fresh: torch.Tensor, scores: torch.Tensor,
                       kivi: Optional[dict] = None, k_only: bool = False,
                       eligible: Optional[torch.Tensor] = None, accumulate: bool = False,
                       stream=None):
    """kvf_rerotate_deviation: rerotate() plus the deviation score of every
    re-positioned context row against k_fresh ([fused rows, Hkv, d])."""
    kd = None
    pool_rows = _rows(pool_k)
    if kivi is not None:
        kd = ctypes.byref(_kivi_desc(kivi))
        pool_rows = int(kivi["k_codes"].shape[0])
    d = layer.desc()
    return _run(_lib.kvf_rerotate_deviation,
                (ctypes.byref(d), ctypes.byref(batch.desc), _ptr(chunks), int(chunks.shape[0]),
                 max_chunk_len, _ptr(pool_k), _ptr(pool_v), kd, pool_rows, _ptr(rope_cos),
                 _ptr(rope_sin), int(rope_cos.shape[0]), _ptr(fused_k), _ptr(fused_v), _rows(fused_k),
                 1 if k_only else 0, _ptr(k_fresh), _ptr(eligible), 1 if accumulate else 0,
                 _ptr(scores)), "kvf_rerotate_deviation", stream, keep=(d, batch))


def rerotate_score_attn_mass(layer: Layer, batch: Batch, chunks: torch.Tensor, max_chunk_len: int,
                             pool_k: torch.Tensor, rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                             fused_k: torch.Tensor, q_u: torch.Tensor, scores: torch.Tensor,
                             workspace: Optional[torch.Tensor], n_last_q: int = 0,
                             eligible: Optional[torch.Tensor] = None, accumulate: bool = False,
                             stream=None):
    """kvf_rerotate_score_attn_mass: keys-only re-positioning of the chunks
    (pool_k -> fused_k; pool_k may be fused_k) and the attention-mass score
    in one pass."""
    d = layer.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _run(_lib.kvf_rerotate_score_attn_mass,
                (ctypes.byref(d), ctypes.byref(batch.desc), _ptr(chunks), int(chunks.shape[0]),
                 max_chunk_len, _ptr(pool_k), _rows(pool_k), _ptr(rope_cos), _ptr(rope_sin),
                 int(rope_cos.shape[0]), _ptr(fused_k), _rows(fused_k), _ptr(q_u), n_last_q,
                 _ptr(eligible), 1 if accumulate else 0,
                 _ptr(scores), _ptr(workspace), ws_bytes), "kvf_rerotate_score_attn_mass", stream,
                keep=(d, batch))


def score_attn_mass_noalloc(layer: Layer, batch: Batch, fused_k: torch.Tensor, q_u: torch.Tensor,
                            scores: torch.Tensor, n_last_q: int = 0,
                            eligible: Optional[torch.Tensor] = None, accumulate: bool = False,
                            stream=None):
    """kvf_score_attn_mass_noalloc: the attention-mass score without a
    caller workspace (the library's per-GPU scratch array)."""
    d = layer.desc()
    return _run(_lib.kvf_score_attn_mass_noalloc,
                (ctypes.byref(d), ctypes.byref(batch.desc), _ptr(fused_k), _ptr(q_u), n_last_q,
                 _ptr(eligible), _ptr(scores), 1 if accumulate else 0),
                "kvf_score_attn_mass_noalloc", stream, keep=(d, batch))


def score_workspace_size(mode: int, layer: Layer, batch: Batch, n_last_q: int = 0) -> int:
    d = layer.desc()
    return int(_lib.kvf_score_workspace_size(mode, ctypes.byref(d), ctypes.byref(batch.desc), n_last_q))


def score(mode: int, layer: Layer, batch: Batch, fused_k: torch.Tensor,
          k_fresh: Optional[torch.Tensor], q_u: Optional[torch.Tensor], scores: torch.Tensor,
          workspace: Optional[torch.Tensor] = None, n_last_q: int = 0,
          eligible: Optional[torch.Tensor] = None, accumulate: bool = False, stream=None):
    """eligible: uint8 [sum N] (0 = not scored, NaN); accumulate: add to scores."""
    d = layer.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    flags = mode | (KVF_SCORE_ACCUMULATE if accumulate else 0)
    return _run(_lib.kvf_score, (flags, ctypes.byref(d), ctypes.byref(batch.desc), _ptr(fused_k),
                          _ptr(k_fresh), _ptr(q_u), n_last_q, _ptr(eligible), _ptr(scores),
                          _ptr(workspace), ws_bytes,), "kvf_score", stream)


def select_topk(scores: Optional[torch.Tensor], batch: Batch, k_per_req: Sequence[int],
                out_idx: torch.Tensor, out_rows: Optional[torch.Tensor] = None,
                out_pos: Optional[torch.Tensor] = None, forced: Optional[torch.Tensor] = None,
                out_mask: Optional[torch.Tensor] = None, stream=None):
    """forced: uint8 [sum N] mask of positions ranked above every score;
    out_mask: uint8 [sum N], 1 at the picks."""
    ka = _int_array(k_per_req)
    return _run(_lib.kvf_select_topk, (_ptr(scores), _ptr(forced), ctypes.byref(batch.desc), ka,
                                _ptr(out_idx), _ptr(out_rows), _ptr(out_pos), _ptr(out_mask),
                                None, 0,), "kvf_select_topk", stream)


def select_topk_segmented(scores: Optional[torch.Tensor], batch: Batch, segs: torch.Tensor,
                          k_per_req: Sequence[int], out_idx: torch.Tensor,
                          out_rows: Optional[torch.Tensor] = None,
                          out_pos: Optional[torch.Tensor] = None,
                          forced: Optional[torch.Tensor] = None, stream=None):
    """segs: int32 [n_segs, 8] device tensor (kvf_segment rows)."""
    ka = _int_array(k_per_req)
    return _run(_lib.kvf_select_topk_segmented, (_ptr(scores), _ptr(forced), ctypes.byref(batch.desc),
                                          _ptr(segs), int(segs.shape[0]), ka, _ptr(out_idx),
                                          _ptr(out_rows), _ptr(out_pos),), "kvf_select_topk_segmented", stream)


def select_static(batch: Batch, chunks: torch.Tensor, rules: Sequence[int], mask: torch.Tensor,
                  stream=None):
    """rules: (sink, boundary, seam); chunks: int32 [n_chunks, 8] device tensor."""
    r = StaticRules(*[int(v) for v in rules])
    return _run(_lib.kvf_select_static, (ctypes.byref(batch.desc), _ptr(chunks), int(chunks.shape[0]),
                                  ctypes.byref(r), _ptr(mask),), "kvf_select_static", stream)


def static_counts(batch: Batch, chunks_host, rules: Sequence[int]) -> list:
    """Per-request count of kvf_select_static's marks; chunks_host: int32
    [n_chunks, 8] host array (numpy or CPU tensor)."""
    import numpy as np
    ch = np.ascontiguousarray(np.asarray(chunks_host, dtype=np.int32))
    if ch.ndim != 2 or ch.shape[1] != 8:
        raise ValueError("chunks_host must be int32 [n_chunks, 8]")
    r = StaticRules(*[int(v) for v in rules])
    out = (ctypes.c_int32 * max(batch.n_req, 1))()
    _check(_lib.kvf_static_counts(ctypes.byref(batch.desc), ch.ctypes.data, int(ch.shape[0]),
                                  ctypes.byref(r), out), "kvf_static_counts")
    return [int(out[i]) for i in range(batch.n_req)]


def recompute_qkv(layer: Layer, x: torch.Tensor, row_src: Optional[torch.Tensor],
                  row_pos: torch.Tensor, w_qkv: torch.Tensor, out_mask: int,
                  rope_cos: torch.Tensor, rope_sin: torch.Tensor,
                  q_out: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None,
                  v_out: Optional[torch.Tensor] = None, M: Optional[int] = None,
                  workspace: Optional[torch.Tensor] = None, kv_out_row: Optional[torch.Tensor] = None,
                  stream=None):
    """workspace: kvf_recompute_workspace_size bytes, zeroed before its first
    use; allocated here when omitted and needed (pass one to keep the call
    allocation-free).
    kv_out_row: destination rows of K/V in k_out / v_out (e.g. the fused cache)."""
    d = layer.desc()
    M = int(row_pos.shape[0]) if M is None else M
    if workspace is None:
        need = recompute_workspace_size(layer, M, out_mask)
        if need:
            workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    kv_rows = 0
    if kv_out_row is not None:
        kv_rows = min(_rows(t) for t in (k_out, v_out) if t is not None)
    return _run(_lib.kvf_recompute_qkv,
                (ctypes.byref(d), _ptr(x), _rows(x), _ptr(row_src), _ptr(row_pos), M, _ptr(w_qkv),
                 out_mask, _ptr(rope_cos), _ptr(rope_sin), _rows(rope_cos), _ptr(q_out),
                 _ptr(k_out), _ptr(v_out), _ptr(kv_out_row), kv_rows, _ptr(workspace), ws_bytes),
                "kvf_recompute_qkv", stream, keep=(workspace,))


def recompute_workspace_size(layer: Layer, M: int, out_mask: int) -> int:
    d = layer.desc()
    return int(_lib.kvf_recompute_workspace_size(ctypes.byref(d), M, out_mask))


def scatter_kv(layer: Layer, k_src: Optional[torch.Tensor], k_src_row: Optional[torch.Tensor],
               v_src: Optional[torch.Tensor], v_src_row: Optional[torch.Tensor],
               dst_row: torch.Tensor, fused_k: torch.Tensor, fused_v: torch.Tensor,
               M: Optional[int] = None, stream=None):
    d = layer.desc()
    M = int(dst_row.shape[0]) if M is None else M
    return _run(_lib.kvf_scatter_kv, (ctypes.byref(d), _ptr(k_src), _ptr(k_src_row), _rows(k_src),
                               _ptr(v_src), _ptr(v_src_row), _rows(v_src), _ptr(dst_row), M,
                               _ptr(fused_k), _ptr(fused_v), _rows(fused_k),), "kvf_scatter_kv", stream)


def attention_workspace_size(layer: Layer, batch: Batch, cu_q: Sequence[int]) -> int:
    d = layer.desc()
    return int(_lib.kvf_attention_workspace_size(ctypes.byref(d), ctypes.byref(batch.desc),
                                                 _int_array(cu_q)))


def sparse_q_attention(layer: Layer, batch: Batch, q: torch.Tensor, q_pos: torch.Tensor,
                       cu_q: Sequence[int], fused_k: torch.Tensor, fused_v: torch.Tensor,
                       sm_scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """workspace: attention_workspace_size bytes, zero-filled when allocated
    (the call leaves it zeroed); None runs without key splitting."""
    d = layer.desc()
    cq = _int_array(cu_q)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _run(_lib.kvf_sparse_q_attention, (ctypes.byref(d), ctypes.byref(batch.desc), _ptr(q),
                                       _ptr(q_pos), cq, _ptr(fused_k), _ptr(fused_v),
                                       float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                       ws_bytes,), "kvf_sparse_q_attention", stream)


def _kivi_desc(k: dict) -> KiviDesc:
    bits = 8 * int(k["k_codes"].shape[-1]) // int(k["k_min"].shape[-1])
    return KiviDesc(_ptr(k["k_codes"]), _ptr(k["v_codes"]), _ptr(k["k_min"]), _ptr(k["k_scale"]),
                    _ptr(k["v_min"]), _ptr(k["v_scale"]), int(k["k_min"].shape[0]), bits)


def kivi_encode(layer: Layer, pool_k: torch.Tensor, pool_v: torch.Tensor, pool_cu: torch.Tensor,
                max_chunk_len: int, out: dict, stream=None):
    """out: the kivi dict of rerotate, allocated by the caller; the code
    width follows from the shapes of k_codes and k_min."""
    d = layer.desc()
    n_pool = int(pool_cu.shape[0]) - 1
    od = _kivi_desc(out)
    return _run(_lib.kvf_kivi_encode, (ctypes.byref(d), _ptr(pool_k), _ptr(pool_v), _ptr(pool_cu),
                                n_pool, _rows(pool_k), max_chunk_len, ctypes.byref(od),), "kvf_kivi_encode", stream)


# ----------------------------------------------------------------------------
# int8-resident fused cache
# ----------------------------------------------------------------------------
def q8_cache(rows: int, n_kv_heads: int, head_dim: int, device="cuda") -> dict:
    """A zeroed int8-resident fused cache (kvf_q8_cache): k_codes, v_codes
    uint8 [rows, Hkv, d]; k_stats, v_stats float32 [rows, Hkv, 2] (min, scale)."""
    codes = (rows, n_kv_heads, head_dim)
    stats = (rows, n_kv_heads, 2)
    return {"k_codes": torch.zeros(codes, dtype=torch.uint8, device=device),
            "v_codes": torch.zeros(codes, dtype=torch.uint8, device=device),
            "k_stats": torch.zeros(stats, dtype=torch.float32, device=device),
            "v_stats": torch.zeros(stats, dtype=torch.float32, device=device)}


def _q8_desc(c: dict) -> Q8CacheDesc:
    return Q8CacheDesc(_ptr(c["k_codes"]), _ptr(c["v_codes"]), _ptr(c["k_stats"]),
                       _ptr(c["v_stats"]), int(c["k_codes"].shape[0]))


def rerotate_q8_deviation(layer: Layer, batch: Batch, chunks: torch.Tensor, max_chunk_len: int,
                          pool_k: Optional[torch.Tensor], pool_v: Optional[torch.Tensor],
                          rope_cos: torch.Tensor, rope_sin: torch.Tensor, fused: dict,
                          k_fresh: torch.Tensor, scores: torch.Tensor, kivi: Optional[dict] = None,
                          eligible: Optional[torch.Tensor] = None, accumulate: bool = False,
                          stream=None):
    """kvf_rerotate_q8_deviation: rerotate_q8() plus the deviation score of
    every re-positioned context row against k_fresh (bf16 [rows, Hkv, d])."""
    kd = None
    pool_rows = _rows(pool_k)
    if kivi is not None:
        kd = ctypes.byref(_kivi_desc(kivi))
        pool_rows = int(kivi["k_codes"].shape[0])
    d = layer.desc()
    fd = _q8_desc(fused)
    return _run(_lib.kvf_rerotate_q8_deviation,
                (ctypes.byref(d), ctypes.byref(batch.desc), _ptr(chunks), int(chunks.shape[0]),
                 max_chunk_len, _ptr(pool_k), _ptr(pool_v), kd, pool_rows, _ptr(rope_cos),
                 _ptr(rope_sin), int(rope_cos.shape[0]), ctypes.byref(fd), _ptr(k_fresh),
                 _ptr(eligible), 1 if accumulate else 0, _ptr(scores)),
                "kvf_rerotate_q8_deviation", stream, keep=(d, fd, batch))


def rerotate_q8(layer: Layer, chunks: torch.Tensor, max_chunk_len: int,
                pool_k: Optional[torch.Tensor], pool_v: Optional[torch.Tensor],
                rope_cos: torch.Tensor, rope_sin: torch.Tensor, fused: dict,
                kivi: Optional[dict] = None, stream=None):
    """kvf_rerotate_q8: S1 into the int8-resident cache `fused` (q8_cache)
    from a dense bf16 per-chunk cache or an 8-bit KIVI one (`kivi`)."""
    kd = None
    pool_rows = _rows(pool_k)
    if kivi is not None:
        kd = ctypes.byref(_kivi_desc(kivi))
        pool_rows = int(kivi["k_codes"].shape[0])
    d = layer.desc()
    fd = _q8_desc(fused)
    return _run(_lib.kvf_rerotate_q8, (ctypes.byref(d), _ptr(chunks), int(chunks.shape[0]),
                                       max_chunk_len, _ptr(pool_k), _ptr(pool_v), kd, pool_rows,
                                       _ptr(rope_cos), _ptr(rope_sin), int(rope_cos.shape[0]),
                                       ctypes.byref(fd)), "kvf_rerotate_q8", stream, keep=(d, fd))


def score_q8(mode: int, layer: Layer, batch: Batch, fused: dict, k_fresh: Optional[torch.Tensor],
             scores: torch.Tensor, eligible: Optional[torch.Tensor] = None,
             accumulate: bool = False, stream=None):
    """kvf_score_q8: deviation or key-norm score over the int8-resident cache."""
    d = layer.desc()
    fd = _q8_desc(fused)
    flags = mode | (KVF_SCORE_ACCUMULATE if accumulate else 0)
    return _run(_lib.kvf_score_q8, (flags, ctypes.byref(d), ctypes.byref(batch.desc), ctypes.byref(fd),
                                    _ptr(k_fresh), _ptr(eligible), _ptr(scores)), "kvf_score_q8",
                stream, keep=(d, fd, batch))


def scatter_kv_q8(layer: Layer, k_src: Optional[torch.Tensor], k_src_row: Optional[torch.Tensor],
                  v_src: Optional[torch.Tensor], v_src_row: Optional[torch.Tensor],
                  dst_row: torch.Tensor, fused: dict, M: Optional[int] = None, stream=None):
    """kvf_scatter_kv_q8: bf16 rows encoded into the int8-resident cache."""
    d = layer.desc()
    fd = _q8_desc(fused)
    M = int(dst_row.shape[0]) if M is None else M
    return _run(_lib.kvf_scatter_kv_q8, (ctypes.byref(d), _ptr(k_src), _ptr(k_src_row), _rows(k_src),
                                         _ptr(v_src), _ptr(v_src_row), _rows(v_src), _ptr(dst_row), M,
                                         ctypes.byref(fd)), "kvf_scatter_kv_q8", stream, keep=(d, fd))


def sparse_q_attention_q8(layer: Layer, batch: Batch, q: torch.Tensor, q_pos: torch.Tensor,
                          cu_q: Sequence[int], fused: dict, sm_scale: float, out: torch.Tensor,
                          lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """kvf_sparse_q_attention_q8: the attention call over the int8-resident
    cache (workspace as for sparse_q_attention)."""
    d = layer.desc()
    fd = _q8_desc(fused)
    cq = _int_array(cu_q)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _run(_lib.kvf_sparse_q_attention_q8, (ctypes.byref(d), ctypes.byref(batch.desc), _ptr(q),
                                                 _ptr(q_pos), cq, ctypes.byref(fd), float(sm_scale),
                                                 _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes),
                "kvf_sparse_q_attention_q8", stream, keep=(d, fd, batch, cq))
