"""Storage encodings read and written by the oracle (test infrastructure).

The oracle computes in float64.  It reads the stored fp32 / bf16 inputs
exactly (both are exactly representable in float64) and, where a stored
input has to be produced (the per-chunk caches built ahead of serving),
rounds float64 results to the storage format with round-to-nearest-even.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    raise ValueError(dtype)


def round_f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, one round-to-nearest-even step.

    Rounds the float64 value directly to 8 significant bits (no intermediate
    float32 rounding, which could double-round).  Values must lie in the
    normal bf16 range or be zero; the oracle's data never leaves it.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                    # x = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # 8 significant bits, RNE
    u = r.astype(np.float32).view(np.uint32)     # exact: 8 bits fit in fp32
    return (u >> np.uint32(16)).astype(np.uint16)


def round_f64_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage encoding (float32 array or bf16 bits)."""
    if dtype == "f32":
        return round_f64_to_f32(x)
    if dtype == "bf16":
        return round_f64_to_bf16_bits(x)
    raise ValueError(dtype)
