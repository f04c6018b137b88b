"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and writes them into the documented
byte positions of the two K-quant superblock formats; it holds none of the
method's arithmetic (no decoding, no quantisation, no dot products), so the
CPU oracle and the HIP library can both consume its output without sharing
any code with each other.

Recipe (stands in for the real 7B / 14B GGUF models, which are not
available):
  * seed = crc32("<config>/<layer>/<tensor>") into numpy's PCG64;
  * q4_K (144 B per 256 weights): f16 d and dmin drawn from U(1e-3, 1e-2),
    the 12 packed scale/min bytes and the 128 quant bytes uniform over
    0..255 (so every 6-bit scale/min and 4-bit quant is uniform);
  * q6_K (210 B per 256 weights): the 128 ql bytes, 64 qh bytes and 16
    int8 sub-scales uniform over all byte values, f16 d from U(1e-3, 1e-2);
  * q5_K (176 B per 256 weights): as q4_K, with the 32 fifth-bit bytes
    uniform too (every 5-bit quant uniform);
  * activations ~ N(0, 1) f32; RMSNorm weight ~ U(0.5, 1.5); eps = 1e-6.
"""
from __future__ import annotations

import zlib

import numpy as np

Q4K_BYTES = 144
Q5K_BYTES = 176
Q6K_BYTES = 210
EPS = 1e-6

# Shapes of the five workloads (tokens, hidden, ffn, weights per layer).
CONFIGS = {
    "tiny": dict(n=32, hidden=256, od=512),
    "ffn7b": dict(n=3314, hidden=3584, ffn=18944),
    "attn7b": dict(n=3314, hidden=3584, kv=512),
    "decode14b": dict(n=1, hidden=5120, ffn=13824, attn_v=1024, vocab=152064),
    "chain7b": dict(n=3314, hidden=3584, ffn=18944, kv=512, layers=28),
}


def rng_for(config: str, layer: int, tensor: str) -> np.random.Generator:
    seed = zlib.crc32(f"{config}/{layer}/{tensor}".encode())
    return np.random.Generator(np.random.PCG64(seed))


def _uniform_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).copy()


def _f16_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    v = rng.uniform(1e-3, 1e-2, size=n).astype(np.float16)
    return v.view(np.uint8).reshape(n, 2)


def q4k_weights(rng: np.random.Generator, od: int, id_: int) -> np.ndarray:
    """Raw q4_K superblocks, row-major [od][id/256], returned as uint8 [od, id/256*144]."""
    assert id_ % 256 == 0
    nsb = od * (id_ // 256)
    raw = _uniform_bytes(rng, nsb * Q4K_BYTES).reshape(nsb, Q4K_BYTES)
    raw[:, 0:2] = _f16_bytes(rng, nsb)   # d
    raw[:, 2:4] = _f16_bytes(rng, nsb)   # dmin
    return raw.reshape(od, (id_ // 256) * Q4K_BYTES)


def q5k_weights(rng: np.random.Generator, od: int, id_: int) -> np.ndarray:
    """Raw q5_K superblocks, row-major [od][id/256], returned as uint8 [od, id/256*176]."""
    assert id_ % 256 == 0
    nsb = od * (id_ // 256)
    raw = _uniform_bytes(rng, nsb * Q5K_BYTES).reshape(nsb, Q5K_BYTES)
    raw[:, 0:2] = _f16_bytes(rng, nsb)   # d
    raw[:, 2:4] = _f16_bytes(rng, nsb)   # dmin
    return raw.reshape(od, (id_ // 256) * Q5K_BYTES)


def q6k_weights(rng: np.random.Generator, od: int, id_: int) -> np.ndarray:
    """Raw q6_K superblocks, row-major [od][id/256], returned as uint8 [od, id/256*210]."""
    assert id_ % 256 == 0
    nsb = od * (id_ // 256)
    raw = _uniform_bytes(rng, nsb * Q6K_BYTES).reshape(nsb, Q6K_BYTES)
    raw[:, 208:210] = _f16_bytes(rng, nsb)   # d
    return raw.reshape(od, (id_ // 256) * Q6K_BYTES)


def weights(wtype: str, rng: np.random.Generator, od: int, id_: int) -> np.ndarray:
    return {"q4_K": q4k_weights, "q5_K": q5k_weights, "q6_K": q6k_weights}[wtype](rng, od, id_)


def activations(rng: np.random.Generator, n: int, d: int) -> np.ndarray:
    return rng.standard_normal(size=(n, d), dtype=np.float32)


def rms_weight(rng: np.random.Generator, d: int) -> np.ndarray:
    return rng.uniform(0.5, 1.5, size=d).astype(np.float32)
