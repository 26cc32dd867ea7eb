"""Helpers shared by the GPU parity tests (tensor transfer and error metrics)."""
from __future__ import annotations

import numpy as np

from oracle import storage

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
    print(f"[parity] {what}: max|d|/rms = {e:.3e} (tol {t:.1e})", flush=True)
    assert e <= t, f"{what}: relative error {e:.3e} > {t:.1e}"


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    return storage.encode(x, dtype)


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    return storage.decode(a, dtype)
