"""CPU oracle for the q8-plane producers, the q4_K / q5_K / q6_K matmuls and
the f32-activation q6_K GEMV.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product
library (``quantized_matmul_rmsnorm_amd``) never does, and the two share no
code.  The arithmetic lives in ``oracle.c`` (plain scalar C, built with
``-O2 -ffp-contract=off``); this module only marshals numpy arrays.

Every function cites the passage of the engineering-log pages it follows in
``oracle.c``.  Pins: ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, OpenMP over output rows)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-std=c11", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f32.restype = ctypes.c_float
        lib.oracle_q4k_fields.argtypes = [P, P, P, P, P, P]
        lib.oracle_q5k_fields.argtypes = [P, P, P, P, P, P]
        lib.oracle_q6k_fields.argtypes = [P, P, P, P]
        lib.oracle_dequant_q4k.argtypes = [P, I64, I64, P]
        lib.oracle_dequant_q5k.argtypes = [P, I64, I64, P]
        lib.oracle_dequant_q6k.argtypes = [P, I64, I64, P]
        lib.oracle_rmsnorm.argtypes = [P, P, I64, I64, ctypes.c_float, P]
        lib.oracle_swiglu.argtypes = [P, P, I64, I64, P]
        lib.oracle_quantize.argtypes = [P, I64, I64, P, P, P]
        lib.oracle_gemm_q4k.argtypes = [P, P, P, P, I64, P, I64, P, I64, P, P]
        lib.oracle_gemm_q5k.argtypes = [P, P, P, P, I64, P, I64, P, I64, P, P]
        lib.oracle_gemm_q6k.argtypes = [P, P, P, I64, P, I64, P, I64, P, P]
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def f16_to_f32(h: int) -> float:
    return float(_load().oracle_f16_to_f32(int(h) & 0xFFFF))


def q4k_fields(block: np.ndarray):
    """Decode one 144-byte q4_K superblock -> (d, dmin, sc[8], m[8], q[256])."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    assert b.size == 144
    d = np.zeros(1, np.float32); dm = np.zeros(1, np.float32)
    sc = np.zeros(8, np.uint8); mn = np.zeros(8, np.uint8); q = np.zeros(256, np.uint8)
    _load().oracle_q4k_fields(_p(b), _p(d), _p(dm), _p(sc), _p(mn), _p(q))
    return float(d[0]), float(dm[0]), sc, mn, q


def q5k_fields(block: np.ndarray):
    """Decode one 176-byte q5_K superblock -> (d, dmin, sc[8], m[8], q[256] in [0,31])."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    assert b.size == 176
    d = np.zeros(1, np.float32); dm = np.zeros(1, np.float32)
    sc = np.zeros(8, np.uint8); mn = np.zeros(8, np.uint8); q = np.zeros(256, np.uint8)
    _load().oracle_q5k_fields(_p(b), _p(d), _p(dm), _p(sc), _p(mn), _p(q))
    return float(d[0]), float(dm[0]), sc, mn, q


def q6k_fields(block: np.ndarray):
    """Decode one 210-byte q6_K superblock -> (d, sc[16] int8, q[256] in [0,63])."""
    b = np.ascontiguousarray(block, dtype=np.uint8)
    assert b.size == 210
    d = np.zeros(1, np.float32); sc = np.zeros(16, np.int8); q = np.zeros(256, np.uint8)
    _load().oracle_q6k_fields(_p(b), _p(d), _p(sc), _p(q))
    return float(d[0]), sc, q


def dequant(wtype: str, raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """f64 dequantised weight matrix [rows][cols]."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    w = np.zeros((rows, cols), np.float64)
    fn = {"q4_K": _load().oracle_dequant_q4k, "q5_K": _load().oracle_dequant_q5k,
          "q6_K": _load().oracle_dequant_q6k}[wtype]
    fn(_p(raw), rows, cols, _p(w))
    return w


def gemv_f32(wtype: str, raw: np.ndarray, rows: int, cols: int, x: np.ndarray) -> np.ndarray:
    """out[o] = sum_k w[o][k] * x[k] in f64, w the dequantised weight and x the
    f32 activation as given (not quantised): what the decode arm computes on
    its f32-activation path below the shape gate ("72 · D3-7 ...", section 2,
    Excerpt A).  The plain definition: the f64 dequantisation above, then one
    matrix-vector product."""
    x = np.ascontiguousarray(x, np.float32).astype(np.float64)
    assert x.shape == (cols,)
    return dequant(wtype, raw, rows, cols) @ x


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32); w = np.ascontiguousarray(w, np.float32)
    n, d = x.shape
    y = np.zeros_like(x)
    _load().oracle_rmsnorm(_p(x), _p(w), n, d, ctypes.c_float(eps), _p(y))
    return y


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, np.float32); u = np.ascontiguousarray(u, np.float32)
    n, d = g.shape
    y = np.zeros_like(g)
    _load().oracle_swiglu(_p(g), _p(u), n, d, _p(y))
    return y


def quantize(y: np.ndarray):
    """Block-32 q8 plane of y [n][d] -> (Q int8 [n][d], D f32 [n][d/32], S int32 [n][d/32])."""
    y = np.ascontiguousarray(y, np.float32)
    n, d = y.shape
    assert d % 32 == 0
    q = np.zeros((n, d), np.int8)
    D = np.zeros((n, d // 32), np.float32)
    S = np.zeros((n, d // 32), np.int32)
    _load().oracle_quantize(_p(y), n, d, _p(q), _p(D), _p(S))
    return q, D, S


def _idx(v, limit):
    if v is None:
        return np.arange(limit, dtype=np.int64)
    v = np.ascontiguousarray(v, dtype=np.int64)
    assert v.ndim == 1 and (v.size == 0 or (v.min() >= 0 and v.max() < limit))
    return v


def gemm(wtype: str, Q, D, S, raw, od: int, id_: int, tok=None, outs=None,
         with_mag: bool = False):
    """out[i][j] for t = tok[i], o = outs[j] (all tokens / outputs when None):
    the plane's values D * q times the dequantised weight, with f64 block terms
    and an f64 sum, stored as f32.  With with_mag, also returns mag [i][j] =
    sum over blocks of |block term| (f64), the magnitude that any f32
    evaluation of the per-block rescale rounds against.

    Q/D/S: the q8 plane (int8 [n][id], f32 [n][id/32], int32 [n][id/32]);
    raw: the [od][id/256] superblocks as bytes.
    """
    Q = np.ascontiguousarray(Q, np.int8); D = np.ascontiguousarray(D, np.float32)
    raw = np.ascontiguousarray(raw, np.uint8)
    n = Q.shape[0]
    assert Q.shape[1] == id_ and id_ % 256 == 0
    bpb = {"q4_K": 144, "q5_K": 176, "q6_K": 210}[wtype]
    assert raw.size == od * (id_ // 256) * bpb
    tok = _idx(tok, n); outs = _idx(outs, od)
    out = np.zeros((tok.size, outs.size), np.float32)
    mag = np.zeros((tok.size, outs.size), np.float64) if with_mag else None
    mp = _p(mag) if with_mag else None
    if wtype == "q4_K":
        S = np.ascontiguousarray(S, np.int32)
        _load().oracle_gemm_q4k(_p(Q), _p(D), _p(S), _p(raw), id_, _p(tok), tok.size,
                                _p(outs), outs.size, _p(out), mp)
    elif wtype == "q5_K":
        S = np.ascontiguousarray(S, np.int32)
        _load().oracle_gemm_q5k(_p(Q), _p(D), _p(S), _p(raw), id_, _p(tok), tok.size,
                                _p(outs), outs.size, _p(out), mp)
    elif wtype == "q6_K":
        _load().oracle_gemm_q6k(_p(Q), _p(D), _p(raw), id_, _p(tok), tok.size,
                                _p(outs), outs.size, _p(out), mp)
    else:
        raise ValueError(wtype)
    return (out, mag) if with_mag else out
