"""Test-side encoders for the q4_K / q5_K / q6_K superblock formats.

Written independently of the oracle's decoders (the oracle decodes bytes into
fields; this module packs fields into bytes) from the public GGUF K-quant
definitions.  A round trip fields -> bytes -> oracle decode -> fields pins the
oracle's bit extraction, and the dequantised values built here from the fields
(in numpy f64) are the brute-force side of the matmul pins.
"""
from __future__ import annotations

import numpy as np


def f16_bits(x: float) -> int:
    return int(np.array([x], dtype=np.float16).view(np.uint16)[0])


def q4k_encode(d_bits: int, dmin_bits: int, sc, mn, q) -> np.ndarray:
    """Pack one q4_K superblock (144 B).

    sc, mn: eight 6-bit sub-block scales and mins; q: 256 4-bit quants.
    Layout: d (f16) | dmin (f16) | 12 scale bytes | 128 quant bytes.
    Scale bytes: byte j (j<4) holds sc[j] in bits 0..5 and the top two bits of
    sc[j+4] in bits 6..7; byte j+4 likewise for mn; byte j+8 holds the low
    nibbles of sc[j+4] (bits 0..3) and mn[j+4] (bits 4..7).
    Quant byte 32*g + l holds element 64*g + l (low nibble) and 64*g + 32 + l
    (high nibble).
    """
    sc = [int(v) for v in sc]; mn = [int(v) for v in mn]; q = [int(v) for v in q]
    assert len(sc) == 8 and len(mn) == 8 and len(q) == 256
    assert all(0 <= v < 64 for v in sc + mn) and all(0 <= v < 16 for v in q)
    b = np.zeros(144, np.uint8)
    b[0] = d_bits & 0xFF; b[1] = d_bits >> 8
    b[2] = dmin_bits & 0xFF; b[3] = dmin_bits >> 8
    s = np.zeros(12, np.int64)
    for j in range(4):
        s[j] = sc[j] | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = mn[j] | ((mn[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4)
    b[4:16] = s
    for g in range(4):
        for l in range(32):
            b[16 + 32 * g + l] = q[64 * g + l] | (q[64 * g + 32 + l] << 4)
    return b


def q5k_encode(d_bits: int, dmin_bits: int, sc, mn, q) -> np.ndarray:
    """Pack one q5_K superblock (176 B).

    sc, mn: eight 6-bit sub-block scales and mins; q: 256 5-bit quants.
    Layout: d (f16) | dmin (f16) | 12 scale bytes (packed as in q4_K) |
    32 high-bit bytes | 128 low-nibble bytes (arranged as the q4_K quants).
    High-bit byte l holds, in bit 2*g, the fifth bit of element 64*g + l and,
    in bit 2*g + 1, that of element 64*g + 32 + l.
    """
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 32 for v in q)
    head = q4k_encode(d_bits, dmin_bits, sc, mn, [v & 15 for v in q])
    qh = np.zeros(32, np.int64)
    for g in range(4):
        for l in range(32):
            qh[l] |= (q[64 * g + l] >> 4) << (2 * g)
            qh[l] |= (q[64 * g + 32 + l] >> 4) << (2 * g + 1)
    b = np.zeros(176, np.uint8)
    b[0:16] = head[0:16]
    b[16:48] = qh
    b[48:176] = head[16:144]
    return b


def q6k_encode(d_bits: int, sc, q) -> np.ndarray:
    """Pack one q6_K superblock (210 B).

    sc: sixteen int8 sub-scales (one per 16 elements); q: 256 6-bit quants.
    Layout: ql[128] | qh[64] | scales[16] | d (f16).  Element e = 128*h +
    32*s + l stores its low nibble in ql[64*h + l + 32*(s % 2)] (low nibble
    for s < 2, high nibble otherwise) and its top two bits in bits 2s, 2s+1 of
    qh[32*h + l].
    """
    sc = [int(v) for v in sc]; q = [int(v) for v in q]
    assert len(sc) == 16 and len(q) == 256
    assert all(-128 <= v < 128 for v in sc) and all(0 <= v < 64 for v in q)
    ql = np.zeros(128, np.int64); qh = np.zeros(64, np.int64)
    for e in range(256):
        h, r = divmod(e, 128)
        s, l = divmod(r, 32)
        lo, hi = q[e] & 15, q[e] >> 4
        ql[64 * h + l + 32 * (s % 2)] |= lo << (4 if s >= 2 else 0)
        qh[32 * h + l] |= hi << (2 * s)
    b = np.zeros(210, np.uint8)
    b[0:128] = ql; b[128:192] = qh
    b[192:208] = np.array(sc, np.int64).astype(np.int8).view(np.uint8)
    b[208] = d_bits & 0xFF; b[209] = d_bits >> 8
    return b


def random_q4k(rng, od: int, id_: int):
    """Random q4_K matrix as (bytes [od, nsb*144], dequantised f64 [od, id], fields)."""
    nsb = id_ // 256
    raw = np.zeros((od, nsb * 144), np.uint8)
    w = np.zeros((od, id_), np.float64)
    for o in range(od):
        for s in range(nsb):
            d = np.float16(rng.uniform(1e-3, 1e-2)); dm = np.float16(rng.uniform(1e-3, 1e-2))
            sc = rng.integers(0, 64, 8); mn = rng.integers(0, 64, 8); q = rng.integers(0, 16, 256)
            raw[o, s * 144:(s + 1) * 144] = q4k_encode(f16_bits(d), f16_bits(dm), sc, mn, q)
            j = np.arange(256) // 32
            w[o, s * 256:(s + 1) * 256] = float(d) * sc[j] * q - float(dm) * mn[j]
    return raw, w


def random_q5k(rng, od: int, id_: int):
    """Random q5_K matrix as (bytes [od, nsb*176], dequantised f64 [od, id])."""
    nsb = id_ // 256
    raw = np.zeros((od, nsb * 176), np.uint8)
    w = np.zeros((od, id_), np.float64)
    for o in range(od):
        for s in range(nsb):
            d = np.float16(rng.uniform(1e-3, 1e-2)); dm = np.float16(rng.uniform(1e-3, 1e-2))
            sc = rng.integers(0, 64, 8); mn = rng.integers(0, 64, 8); q = rng.integers(0, 32, 256)
            raw[o, s * 176:(s + 1) * 176] = q5k_encode(f16_bits(d), f16_bits(dm), sc, mn, q)
            j = np.arange(256) // 32
            w[o, s * 256:(s + 1) * 256] = float(d) * sc[j] * q - float(dm) * mn[j]
    return raw, w


def random_q6k(rng, od: int, id_: int):
    """Random q6_K matrix as (bytes [od, nsb*210], dequantised f64 [od, id])."""
    nsb = id_ // 256
    raw = np.zeros((od, nsb * 210), np.uint8)
    w = np.zeros((od, id_), np.float64)
    for o in range(od):
        for s in range(nsb):
            d = np.float16(rng.uniform(1e-3, 1e-2))
            sc = rng.integers(-128, 128, 16); q = rng.integers(0, 64, 256)
            raw[o, s * 210:(s + 1) * 210] = q6k_encode(f16_bits(d), sc, q)
            w[o, s * 256:(s + 1) * 256] = float(d) * sc[np.arange(256) // 16] * (q - 32)
    return raw, w
