"""INT4-quantised KV cache (oracle; test infrastructure only).

[EX] "Who uses it" and "Further reading" pair EAGLE with KV-cache quantisation (INT4 /
INT3 caches that free memory for the draft head); no format is given.  Reading: each
(slot, KV head) row of head_dim values is stored as head_dim signed 4-bit integers q in
[-8, 7] with one float32 scale s, packed two per byte (element 2j in the low nibble of
byte j, element 2j+1 in the high nibble, two's complement).  The value attention uses
is the float32 product s * q rounded to the nearest bfloat16 (ties to even), so that
the attention arithmetic downstream is that of a bfloat16 cache.
"""
from __future__ import annotations

import numpy as np


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """[..., d/2] uint8 -> [..., d] int8 (low nibble first, 4-bit two's complement)."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    vals = np.stack([lo, hi], axis=-1).reshape(*p.shape[:-1], 2 * p.shape[-1])
    return np.where(vals >= 8, vals - 16, vals).astype(np.int8)


def bf16_nearest(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 of each float32 value (ties to even), as float64.  A normal value
    f * 2^e (f in [0.5, 1)) keeps 8 significant bits: rint(f * 256) / 256 * 2^e, with rint
    rounding halves to even.  (Subnormal inputs do not occur for these caches.)"""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    f, e = np.frexp(x)
    return np.ldexp(np.rint(f * 256.0) / 256.0, e)


def dequant_int4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[..., d/2] packed values and [...] float32 scales -> [..., d] float64 values."""
    q = unpack_int4(packed).astype(np.float32)
    s = np.asarray(scales, dtype=np.float32)[..., None]
    return bf16_nearest(s * q)
