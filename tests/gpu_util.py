"""Helpers shared by the GPU parity tests (tensor transfer and error metrics)."""
from __future__ import annotations

import numpy as np

from oracle import fusion, storage

TOL = {"bf16": 2e-2, "f32": 1e-4}     # max |gpu - oracle| / rms(oracle)


def to_gpu(a: np.ndarray, dtype: str = None):
    import torch
    if dtype == "bf16" or (dtype is None and a.dtype == np.uint16):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def from_gpu(t) -> np.ndarray:
    """GPU tensor -> float64 numpy (bf16 decoded exactly)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return storage.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def raw(t) -> np.ndarray:
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    gpu = np.asarray(gpu, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(gpu - ref))) / max(rms, 1e-30)


def assert_close(gpu, ref, dtype: str, what: str, tol: float = None):
    e = rel_err(gpu, ref)
    t = TOL[dtype] if tol is None else tol
    where = ""
    if np.size(ref):
        d = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
        idx = np.unravel_index(int(np.argmax(d)), d.shape)
        where = f" at {tuple(int(i) for i in idx)} gpu={float(np.asarray(gpu)[idx]):.6g} ref={float(np.asarray(ref)[idx]):.6g}"
    print(f"[parity] {what}: max|d|/rms = {e:.3e} (tol {t:.1e}){where}", flush=True)
    assert e <= t, f"{what}: relative error {e:.3e} > {t:.1e}"


def rel_err_vectors(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over output vectors (last axis) of max|d| / rms(reference vector)."""
    ref = np.asarray(ref, dtype=np.float64)
    gpu = np.asarray(gpu, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    r = ref.reshape(-1, ref.shape[-1])
    g = gpu.reshape(-1, ref.shape[-1])
    floor = 1e-3 * float(np.sqrt(np.mean(r * r))) + 1e-30
    rms = np.maximum(np.sqrt(np.mean(r * r, axis=1)), floor)
    return float(np.max(np.max(np.abs(g - r), axis=1) / rms))


def assert_close_vectors(gpu, ref, dtype: str, what: str, tol: float = None):
    """Attention outputs: the RMS is taken per output vector (one token, one
    head).  Outputs of rows that see few keys are an order of magnitude
    larger than those of long rows, so a single RMS over the tensor would be
    exceeded by the bf16 storage rounding of those few vectors alone."""
    e = rel_err_vectors(gpu, ref)
    whole = rel_err(gpu, ref)
    t = TOL[dtype] if tol is None else tol
    print(f"[parity] {what}: max over vectors of max|d|/rms(vector) = {e:.3e} (tol {t:.1e}); "
          f"whole-tensor max|d|/rms = {whole:.3e}", flush=True)
    assert e <= t, f"{what}: per-vector relative error {e:.3e} > {t:.1e}"


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return storage.encode(x, dtype)


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    return storage.decode(a, dtype)


def check_selection(name, sel_gpu, gs, rs, ks, n_ctx):
    """GPU picks = TopK of the GPU's own scores, bit for bit; differences from
    the oracle's picks only where the scores' error can reorder them."""
    delta = float(np.max(np.abs(gs - rs)))
    off = 0
    for r, k in enumerate(ks):
        n = int(n_ctx[r])
        g_r, o_r = gs[off:off + n], rs[off:off + n]
        want = fusion.select_topk(g_r.astype(np.float32), k)
        assert np.array_equal(sel_gpu[r], want), f"{name} req {r}: not the TopK of its own scores"
        ref_sel = fusion.select_topk(o_r.astype(np.float32), k)
        diff = np.setxor1d(sel_gpu[r], ref_sel)
        if k and len(diff):
            kth = np.sort(o_r)[::-1][k - 1]
            far = np.abs(o_r[diff] - kth).max()
            assert far <= 2 * delta, f"{name} req {r}: a pick {far:.3g} from the k-th score (2 max|d| = {2 * delta:.3g})"
        print(f"[info] {name} req {r}: {len(diff) // 2} of {k} picks differ from the oracle's "
              f"(scores max|d| {delta:.3g})", flush=True)
        off += n
