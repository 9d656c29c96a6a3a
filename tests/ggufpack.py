"""Test-side packers: known field values -> GGUF block bytes.

These run in the opposite direction to the oracle's decoders (values -> bytes
instead of bytes -> values), written from the public GGUF block description,
so a mistake in a decoder is not mirrored here.  Used to build hand-made
blocks whose decoded values are known in advance.
"""
from __future__ import annotations

import numpy as np


def f16_bits(x: float) -> int:
    return int(np.array([x], dtype=np.float16).view(np.uint16)[0])


def f16_value(bits: int) -> float:
    return float(np.array([bits], dtype=np.uint16).view(np.float16)[0])


def pack_q4k(d_bits: int, dmin_bits: int, sc, mn, u) -> np.ndarray:
    """One 144-byte Q4_K block from f16 bit patterns, 8 scales, 8 mins (0..63)
    and 256 quants (0..15)."""
    sc = [int(v) for v in sc]
    mn = [int(v) for v in mn]
    u = [int(v) for v in u]
    assert len(sc) == 8 and len(mn) == 8 and len(u) == 256
    assert all(0 <= v < 64 for v in sc + mn) and all(0 <= v < 16 for v in u)
    b = np.zeros(144, np.uint8)
    b[0], b[1] = d_bits & 255, d_bits >> 8
    b[2], b[3] = dmin_bits & 255, dmin_bits >> 8
    S = [0] * 12
    for j in range(4):
        S[j] |= sc[j]
        S[j + 4] |= mn[j]
    for j in range(4, 8):
        S[j + 4] = (sc[j] & 15) | ((mn[j] & 15) << 4)
        S[j - 4] |= (sc[j] >> 4) << 6
        S[j] |= (mn[j] >> 4) << 6
    b[4:16] = S
    for i in range(256):
        j, l = divmod(i, 32)
        pos = 16 + 32 * (j // 2) + l
        if j % 2 == 0:
            b[pos] |= u[i]
        else:
            b[pos] |= u[i] << 4
    return b


def pack_q6k(d_bits: int, sc, q) -> np.ndarray:
    """One 210-byte Q6_K block from an f16 bit pattern, 16 int8 scales and 256
    6-bit quants (0..63; the weight is d*scale*(q-32))."""
    sc = [int(v) for v in sc]
    q = [int(v) for v in q]
    assert len(sc) == 16 and len(q) == 256
    assert all(-128 <= v < 128 for v in sc) and all(0 <= v < 64 for v in q)
    b = np.zeros(210, np.uint8)
    for i in range(256):
        h, r = divmod(i, 128)
        k, l = divmod(r, 32)
        lo, hi = q[i] & 15, q[i] >> 4
        pos = 64 * h + 32 * (k & 1) + l
        b[pos] |= lo if k < 2 else lo << 4
        b[128 + 32 * h + l] |= hi << (2 * k)
    b[192:208] = np.array(sc, np.int8).view(np.uint8)
    b[208], b[209] = d_bits & 255, d_bits >> 8
    return b


def pack_q8k(d: float, q) -> np.ndarray:
    """One 292-byte Q8_K record from an f32 scale and 256 int8 quants; the
    16 sums are filled in."""
    q = np.asarray(q, np.int64)
    assert q.size == 256 and q.min() >= -128 and q.max() <= 127
    b = np.zeros(292, np.uint8)
    b[0:4] = np.array([d], np.float32).view(np.uint8)
    b[4:260] = q.astype(np.int8).view(np.uint8)
    bs = q.reshape(16, 16).sum(axis=1)
    b[260:292] = bs.astype(np.int16).view(np.uint8)
    return b
