"""KIVI-style asymmetric int8 / int4 cache encoding (test infrastructure).

[KVB] section 4.5, Eq. 7: a cached value x is stored as the integer
round((x - min) / (max - min) * (2^b - 1)); keys take their min/max per head
channel over the tokens of a chunk, values per token; b is 8 or 4.  With
levels = 2^b - 1, codes lie in [0, levels] and the stored statistics are
float32 (min, scale) with scale = (max - min) / levels, so that the decoded
value is min + code * scale.  4-bit codes are stored two to a byte (pack4):
channel 2i in the low nibble, channel 2i + 1 in the high nibble.

Statistics groups:
  K: one (min, scale) per (pool chunk, kv head, channel), over the chunk's
     tokens.
  V: one (min, scale) per (cached token, kv head), over the head channels.

Encoding takes an integer decision from floating point, so it is computed in
float32, the precision of the library's encoder, with the operations in this
order: range = max - min; scale = range / levels; inv = levels / range;
code = round_half_even((x - min) * inv), clamped to [0, levels]; a group
with range 0 gets scale 0 and codes 0.  Decoding is float64.

Pins (tests/test_oracle_kivi.py): codes lie in [0, levels]; the group minimum
decodes exactly to min and the maximum to code `levels`; |decode(encode(x)) -
x| <= scale / 2 (+ float32 rounding); constant groups decode exactly; the
4-bit packing of a hand-written example and its inverse.
"""
from __future__ import annotations

import numpy as np


def levels(bits: int) -> int:
    if bits not in (4, 8):
        raise ValueError("KIVI codes are 8 or 4 bits")
    return (1 << bits) - 1


def _encode_groups(x: np.ndarray, axis, bits: int = 8) -> tuple:
    """Encode float32 `x`, reducing statistics over `axis`."""
    top = np.float32(levels(bits))
    x = np.asarray(x, dtype=np.float32)
    mn = x.min(axis=axis, keepdims=True)
    mx = x.max(axis=axis, keepdims=True)
    rng = (mx - mn).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = np.where(rng > 0, rng / top, np.float32(0.0)).astype(np.float32)
        inv = np.where(rng > 0, top / rng, np.float32(0.0)).astype(np.float32)
    t = ((x - mn).astype(np.float32) * inv).astype(np.float32)
    code = np.clip(np.rint(t), 0, top).astype(np.uint8)
    return code, mn, scale


def encode_keys(k: np.ndarray, pool_cu: np.ndarray, bits: int = 8) -> tuple:
    """k: [pool_rows, Hkv, d] float32 -> (codes uint8 same shape, one code
    per byte, k_min [n_pool, Hkv, d] f32, k_scale [n_pool, Hkv, d] f32)."""
    k = np.asarray(k, dtype=np.float32)
    n_pool = len(pool_cu) - 1
    codes = np.empty(k.shape, dtype=np.uint8)
    kmin = np.empty((n_pool,) + k.shape[1:], dtype=np.float32)
    kscale = np.empty_like(kmin)
    for c in range(n_pool):
        a, b = int(pool_cu[c]), int(pool_cu[c + 1])
        code, mn, sc = _encode_groups(k[a:b], axis=0, bits=bits)
        codes[a:b] = code
        kmin[c] = mn[0]
        kscale[c] = sc[0]
    return codes, kmin, kscale


def encode_values(v: np.ndarray, bits: int = 8) -> tuple:
    """v: [pool_rows, Hkv, d] float32 -> (codes, v_min [pool_rows, Hkv],
    v_scale [pool_rows, Hkv])."""
    code, mn, sc = _encode_groups(v, axis=2, bits=bits)
    return code, mn[..., 0], sc[..., 0]


def pack4(codes: np.ndarray) -> np.ndarray:
    """4-bit codes (one per byte, last axis even) -> two per byte: byte i of
    the last axis holds channel 2i in bits 0-3 and channel 2i + 1 in bits 4-7."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2 or (c > 15).any():
        raise ValueError("pack4 takes 4-bit codes over an even last axis")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def decode_keys(codes: np.ndarray, kmin: np.ndarray, kscale: np.ndarray,
                pool_cu: np.ndarray) -> np.ndarray:
    out = np.empty(codes.shape, dtype=np.float64)
    for c in range(len(pool_cu) - 1):
        a, b = int(pool_cu[c]), int(pool_cu[c + 1])
        out[a:b] = kmin[c].astype(np.float64) + codes[a:b].astype(np.float64) * kscale[c].astype(np.float64)
    return out


def decode_values(codes: np.ndarray, vmin: np.ndarray, vscale: np.ndarray) -> np.ndarray:
    return (vmin.astype(np.float64)[..., None]
            + codes.astype(np.float64) * vscale.astype(np.float64)[..., None])
