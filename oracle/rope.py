"""Rotary position embedding, float64 (test infrastructure).

[KVB] section 3.2, Eq. 3: queries and keys are rotated by a matrix that
depends on the token position t and a base frequency; the dot product of a
rotated query at s and a rotated key at t depends only on t - s.  The page
does not fix the pairing or the frequency schedule.  This oracle takes the
rotate-half form used by HuggingFace RoPE models (the models that page
targets): channel j is paired with channel j + d/2, the pair rotates by the
angle t * theta_j with theta_j = base ** (-2 j / d), j < d/2, and no
frequency scaling is applied.

Pins (tests/test_oracle_rope.py): equality with multiplication by the complex
exponential exp(i t theta_j) on z_j = x_j + i x_{j+d/2}; R(a) R(b) = R(a + b);
R(0) = I; norm preservation; the relative-offset property of Eq. 3; the
page's worked case of a key cached at position 50 reused at 1050 through
the correction R^1000.
"""
from __future__ import annotations

import numpy as np


def inverse_frequencies(head_dim: int, base: float) -> np.ndarray:
    """theta_j = base ** (-2 j / d) for j in [0, d/2), float64."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * j / head_dim)


def angles(pos: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """[n, d/2] rotation angles pos * theta_j (float64)."""
    pos = np.asarray(pos, dtype=np.float64).reshape(-1)
    return pos[:, None] * inverse_frequencies(head_dim, base)[None, :]


def rotate(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Apply R(pos_n) to every head vector of row n.

    x: [n, H, d] float64; pos: [n] positions (may be any real offset,
    including the negative or delta rotations used for re-positioning).
    Returns a new float64 array.
    """
    x = np.asarray(x, dtype=np.float64)
    n, h, d = x.shape
    half = d // 2
    a = angles(pos, d, base)                      # [n, d/2]
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    lo = x[..., :half]
    hi = x[..., half:]
    out = np.empty_like(x)
    out[..., :half] = lo * c - hi * s
    out[..., half:] = hi * c + lo * s
    return out
