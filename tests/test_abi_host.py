"""CPU tests of the C ABI: every declared symbol is exported, and the host logic
(argument/shape/type validation, plane cache, dead-key refusal, statistics,
scratch cap) behaves as include/mmq.h states.  Uses MMQ_CTX_DRYRUN contexts:
bookkeeping runs, nothing touches a device (pointers are plain integers).
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import quantized_matmul_rmsnorm_amd as mmq
from quantized_matmul_rmsnorm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mmq\w+|mmvq\w+)\s*\(", text)))


def test_header_declares_the_exported_list():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    dyn = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in dyn, name
        assert getattr(ctypes.CDLL(_lib.LIB_PATH), name) is not None


def test_peak_library_exports_its_header():
    """libmmq_peak.so (the benchmark's measured MFMA ceilings) exports exactly
    what include/mmq_peak.h declares, and rejects bad arguments without a
    launch (no device is touched: the checks come first)."""
    from quantized_matmul_rmsnorm_amd import build as _b
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mmq_peak.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(mmq\w+)\s*\(", text)))
    assert declared == ["mmq_peak_chains", "mmq_peak_mfma_f16", "mmq_peak_mfma_i8", "mmq_peak_mix",
                        "mmq_peak_probe", "mmq_peak_probe_count", "mmq_peak_probe_info",
                        "mmq_peak_read"]
    out = subprocess.run(["nm", "-D", "--defined-only", _b.LIB_PEAK], capture_output=True,
                         text=True, check=True).stdout
    dyn = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(declared) <= dyn
    lib = ctypes.CDLL(_b.LIB_PEAK)
    assert lib.mmq_peak_chains() == 8
    for fn in (lib.mmq_peak_mfma_f16, lib.mmq_peak_mfma_i8):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        assert fn(None, 1, 1, None) == -1
        assert fn(ctypes.c_void_p(0x1000), 0, 1, None) == -1
        assert fn(ctypes.c_void_p(0x1000), 1, 0, None) == -1
        assert fn(ctypes.c_void_p(0x1000), 1, (1 << 20) + 1, None) == -1
    mix = lib.mmq_peak_mix
    mix.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert mix(None, 1, 1, 0, None) == -1
    assert mix(ctypes.c_void_p(0x1000), 0, 1, 0, None) == -1
    assert mix(ctypes.c_void_p(0x1000), 1, 0, 0, None) == -1
    assert mix(ctypes.c_void_p(0x1000), 1, (1 << 20) + 1, 0, None) == -1
    assert mix(ctypes.c_void_p(0x1000), 1, 1, 4, None) == -1
    assert mix(ctypes.c_void_p(0x1000), 1, 1, -1, None) == -1
    count = lib.mmq_peak_probe_count()
    assert count >= 10
    info = lib.mmq_peak_probe_info
    info.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int),
                     ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    names = set()
    for i in range(count):
        nm, th, ti, mw = ctypes.c_char_p(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        assert info(i, ctypes.byref(nm), ctypes.byref(th), ctypes.byref(ti), ctypes.byref(mw)) == 0
        assert th.value in (256, 512, 1024) and ti.value in (1, 2) and 0 <= mw.value <= th.value // 64
        names.add(nm.value.decode())
    assert len(names) == count
    nm, th, ti, mw = ctypes.c_char_p(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    assert info(count, ctypes.byref(nm), ctypes.byref(th), ctypes.byref(ti), ctypes.byref(mw)) == -1
    probe = lib.mmq_peak_probe
    probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert probe(-1, ctypes.c_void_p(0x1000), 1, 1, None) == -1
    assert probe(count, ctypes.c_void_p(0x1000), 1, 1, None) == -1
    assert probe(0, None, 1, 1, None) == -1
    assert probe(0, ctypes.c_void_p(0x1000), 0, 1, None) == -1
    assert probe(0, ctypes.c_void_p(0x1000), 1, (1 << 20) + 1, None) == -1
    rd = lib.mmq_peak_read
    rd.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p]
    assert rd(None, 16, ctypes.c_void_p(0x1000), 1, 8, None) == -1
    assert rd(ctypes.c_void_p(0x1000), 24, ctypes.c_void_p(0x1000), 1, 8, None) == -1
    assert rd(ctypes.c_void_p(0x1000), 0, ctypes.c_void_p(0x1000), 1, 8, None) == -1
    assert rd(ctypes.c_void_p(0x1000), 16, None, 1, 8, None) == -1
    assert rd(ctypes.c_void_p(0x1000), 16, ctypes.c_void_p(0x1000), 0, 8, None) == -1
    assert rd(ctypes.c_void_p(0x1000), 16, ctypes.c_void_p(0x1000), 1, 5, None) == -1


def test_no_device_is_reported():
    with pytest.raises(mmq.MmqError) as e:
        mmq.mmq_create(999, 0)
    assert e.value.status == mmq.MMQ_E_DEVICE
    with pytest.raises(mmq.MmqError) as e:
        mmq.mmq_create(0, 0x100)
    assert e.value.status == mmq.MMQ_E_ARG


@pytest.fixture
def ctx():
    c = mmq.mmq_create(0, mmq.MMQ_CTX_DRYRUN)
    yield c
    mmq.mmq_destroy(c)


def _w(ctx, wtype=mmq.MMQ_Q4_K, rows=512, cols=256, uses=0):
    bpb = {mmq.MMQ_Q4_K: 144, mmq.MMQ_Q5_K: 176, mmq.MMQ_Q6_K: 210}[wtype]
    raw = np.zeros(rows * cols // 256 * bpb, np.uint8)
    return mmq.mmq_register_weight(ctx, wtype, rows, cols, raw, uses)


def _status(fn, *a):
    try:
        fn(*a)
    except mmq.MmqError as e:
        return e.status
    return mmq.MMQ_OK


def test_plane_rows():
    assert [mmq.mmq_plane_rows(n) for n in (0, 1, 31, 32, 33, 3314)] == [0, 32, 32, 32, 64, 3328]


def test_shape_and_argument_validation(ctx):
    X, W, Y = 0x10000, 0x20000, 0x30000
    assert _status(mmq.mmq_quant_rms, ctx, X, W, Y, 4, 300, 1e-6, 0) == mmq.MMQ_E_SHAPE
    assert _status(mmq.mmq_quant_rms, ctx, X, W, Y, 0, 256, 1e-6, 0) == mmq.MMQ_E_SHAPE
    assert _status(mmq.mmq_quant_rms, ctx, X + 4, W, Y, 4, 256, 1e-6, 0) == mmq.MMQ_E_ARG
    assert _status(mmq.mmq_quant_swiglu, ctx, X, 0, Y, 4, 256, 0) == mmq.MMQ_E_ARG
    assert _status(mmq.mmq_quant_f32, ctx, 0, 4, 256) == mmq.MMQ_E_ARG
    st = mmq.mmq_stats(ctx)
    assert st["launches_quant_rms"] == st["launches_quant_swiglu"] == st["launches_quant_f32"] == 0


def test_registration_validation(ctx):
    raw = np.zeros(144 * 4, np.uint8)
    assert _status(mmq.mmq_register_weight, ctx, 11, 4, 256, raw) == mmq.MMQ_E_TYPE
    assert _status(mmq.mmq_register_weight, ctx, mmq.MMQ_Q4_K, 4, 300, raw) == mmq.MMQ_E_SHAPE
    assert _status(mmq.mmq_register_weight, ctx, mmq.MMQ_Q4_K, 0, 256, raw) == mmq.MMQ_E_SHAPE
    assert _status(mmq.mmq_register_weight, ctx, mmq.MMQ_Q4_K, 4, 256, raw, 0x8) == mmq.MMQ_E_ARG
    w4 = _w(ctx, mmq.MMQ_Q4_K, 512, 256)
    # q4_K one-token GEMV layout: 16 B of codes + 2 B (sc, m) per 32 weights, (d, dmin) per 256
    w4v = _w(ctx, mmq.MMQ_Q4_K, 300, 512, mmq.MMQ_USE_GEMV)
    assert mmq.mmq_weight_bytes(w4v) == 300 * 16 * (16 + 2) + 300 * 2 * 8
    mmq.mmq_weight_free(w4v)
    w6 = _w(ctx, mmq.MMQ_Q6_K, 1000, 512)
    # q4_K: f16 tiles (2 B/weight) + scales + mins; q6_K adds the GEMV layout
    assert mmq.mmq_weight_bytes(w4) == 512 * 256 * 2 + 16 * 1 * 64 * 4 + 16 * 1 * 512 * 2
    rows_pad = 1024
    # q6_K matmul tiles: f16 centred codes (2 B/weight), d per row and
    # superblock, and 16 f16 sub-scales per row and superblock
    gemm6 = rows_pad * 512 * 2 + (rows_pad // 32) * 2 * 32 * 4 + rows_pad * 2 * 16 * 2
    gemv6 = 1000 * 16 * (16 + 8 + 2) + 1000 * 2 * 4
    assert mmq.mmq_weight_bytes(w6) == gemm6 + gemv6
    assert mmq.mmq_stats(ctx)["weight_bytes"] == mmq.mmq_weight_bytes(w4) + mmq.mmq_weight_bytes(w6)
    mmq.mmq_weight_free(w4)
    assert mmq.mmq_stats(ctx)["weight_bytes"] == mmq.mmq_weight_bytes(w6)
    mmq.mmq_weight_free(w6)


def test_packed_q4k_registration(ctx):
    """MMQ_USE_GEMM_PACKED: q4_K only, only beside MMQ_USE_GEMM, refused before
    any allocation; the tiles take half a byte per weight plus 8 f16
    sub-scales per row and superblock, beside the same scales and mins; the
    matmul accepts the weight like any other."""
    P, G = mmq.MMQ_USE_GEMM_PACKED, mmq.MMQ_USE_GEMM
    raw4, raw5, raw6 = (np.zeros(b * 4, np.uint8) for b in (144, 176, 210))
    assert _status(mmq.mmq_register_weight, ctx, mmq.MMQ_Q4_K, 4, 256, raw4, P) == mmq.MMQ_E_ARG
    assert _status(mmq.mmq_register_weight, ctx, mmq.MMQ_Q4_K, 4, 256, raw4,
                   P | mmq.MMQ_USE_GEMV) == mmq.MMQ_E_ARG
    assert _status(mmq.mmq_register_weight, ctx, mmq.MMQ_Q6_K, 4, 256, raw6, G | P) == mmq.MMQ_E_TYPE
    assert _status(mmq.mmq_register_weight, ctx, mmq.MMQ_Q5_K, 4, 256, raw5, G | P) == mmq.MMQ_E_TYPE
    assert mmq.mmq_stats(ctx)["weight_bytes"] == 0
    w = _w(ctx, mmq.MMQ_Q4_K, 1000, 512, G | P)
    rows_pad, nsb = 1024, 2
    packed = rows_pad * 512 // 2 + rows_pad * nsb * 16 + (rows_pad // 32) * nsb * (64 * 4 + 512 * 2)
    assert mmq.mmq_weight_bytes(w) == packed
    wf = _w(ctx, mmq.MMQ_Q4_K, 1000, 512, G)
    assert mmq.mmq_weight_bytes(wf) == rows_pad * 512 * 2 + (rows_pad // 32) * nsb * (64 * 4 + 512 * 2)
    assert mmq.mmq_weight_bytes(wf) / mmq.mmq_weight_bytes(w) > 2.9
    # with the GEMV layout too: both sets of tiles
    wb = _w(ctx, mmq.MMQ_Q4_K, 1000, 512, G | P | mmq.MMQ_USE_GEMV)
    assert mmq.mmq_weight_bytes(wb) == packed + 1000 * 16 * (16 + 2) + 1000 * 2 * 8
    A, O = 0x100000, 0x200000
    assert _status(mmq.mmq_gemm_q4k, ctx, w, A, 300, O) == mmq.MMQ_OK
    assert _status(mmq.mmq_gemm_q6k, ctx, w, A, 300, O) == mmq.MMQ_E_TYPE
    assert _status(mmq.mmvq_q4k, ctx, w, A, O) == mmq.MMQ_E_TYPE      # no GEMV tiles
    assert _status(mmq.mmvq_q4k, ctx, wb, A, O) == mmq.MMQ_OK
    assert mmq.mmq_stats(ctx)["launches_gemm_q4k"] == 1
    for h in (w, wf, wb):
        mmq.mmq_weight_free(h)
    assert mmq.mmq_stats(ctx)["weight_bytes"] == 0


def test_q5k_is_a_decode_only_type(ctx):
    raw = np.zeros(176 * 4, np.uint8)
    # no matmul tiles for q5_K: asking for them is a type error, before any allocation
    for uses in (mmq.MMQ_USE_GEMM, mmq.MMQ_USE_GEMM | mmq.MMQ_USE_GEMV):
        assert _status(mmq.mmq_register_weight, ctx, mmq.MMQ_Q5_K, 4, 256, raw, uses) == mmq.MMQ_E_TYPE
    assert mmq.mmq_stats(ctx)["weight_bytes"] == 0
    # default uses = the GEMV: 16 B of low nibbles + 4 B of fifth bits + 2 B (sc, m) per 32
    # weights, (d, dmin) per 256
    w5 = _w(ctx, mmq.MMQ_Q5_K, 300, 512)
    assert mmq.mmq_weight_bytes(w5) == 300 * 16 * (16 + 4 + 2) + 300 * 2 * 8
    w4 = _w(ctx, mmq.MMQ_Q4_K, 64, 512, mmq.MMQ_USE_GEMV)
    A, O = 0x100000, 0x200000
    assert _status(mmq.mmq_gemm_q4k, ctx, w5, A, 8, O) == mmq.MMQ_E_TYPE
    assert _status(mmq.mmq_gemm_q6k, ctx, w5, A, 8, O) == mmq.MMQ_E_TYPE
    assert _status(mmq.mmvq_q4k, ctx, w5, A, O) == mmq.MMQ_E_TYPE
    assert _status(mmq.mmvq_q6k, ctx, w5, A, O) == mmq.MMQ_E_TYPE
    assert _status(mmq.mmvq_q5k, ctx, w4, A, O) == mmq.MMQ_E_TYPE
    assert _status(mmq.mmvq_q5k, ctx, w5, A + 4, O) == mmq.MMQ_E_ARG
    assert _status(mmq.mmvq_q5k, ctx, w5, A, O) == mmq.MMQ_OK
    st = mmq.mmq_stats(ctx)
    assert st["launches_mmvq_q5k"] == 1 and st["launches_mmvq_q4k"] == 0
    assert st["cache_misses"] == 1      # the activation was quantised standalone
    with pytest.raises(ValueError):     # the binding checks 176 B per superblock
        mmq.mmq_register_weight(ctx, mmq.MMQ_Q5_K, 4, 256, np.zeros(144 * 4, np.uint8))
    mmq.mmq_weight_free(w5)
    mmq.mmq_weight_free(w4)


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    for name in ("MMQ_Q4_K", "MMQ_Q5_K", "MMQ_Q6_K", "MMQ_USE_GEMM", "MMQ_USE_GEMV", "MMQ_USE_GEMM_PACKED",
                 "MMQ_DECODE_F32_GATE", "MMQ_PLANE_ROWS", "MMQ_NOALLOC_MAX_COLS"):
        m = re.search(rf"#define {name}\s+\(?(-?\d+)", text)
        assert m, name
        assert int(m.group(1)) == getattr(mmq, name), name


def test_decode_q6k_routing(ctx):
    """The routed q6_K decode arm takes the f32-activation GEMV only below the
    od*id gate, for a written activation with no recorded plane; otherwise
    the quantised GEMV (which quantises on a miss and hits a recorded plane)."""
    gv = mmq.MMQ_USE_GEMV
    small = _w(ctx, mmq.MMQ_Q6_K, 512, 3584, gv)          # 1.8M < gate
    big = _w(ctx, mmq.MMQ_Q6_K, 8192, 5120, gv)           # 41.9M >= gate
    wide = _w(ctx, mmq.MMQ_Q6_K, 16, 16640, gv)           # small, but x too wide for LDS
    assert 512 * 3584 < mmq.MMQ_DECODE_F32_GATE <= 8192 * 5120
    X, X2, X3, Y, W, O = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000

    def delta(fn, *a):
        before = mmq.mmq_stats(ctx)
        fn(*a)
        after = mmq.mmq_stats(ctx)
        return {k: after[k] - before[k] for k in ("launches_gemv_f32", "launches_mmvq_q6k",
                                                 "launches_quant_f32", "cache_hits", "cache_misses")}

    # small, written, no plane: the f32 path, nothing quantised or recorded
    d = delta(mmq.mmq_decode_q6k, ctx, small, X, O)
    assert d == {"launches_gemv_f32": 1, "launches_mmvq_q6k": 0, "launches_quant_f32": 0,
                 "cache_hits": 0, "cache_misses": 0}
    # large: the quantised GEMV, quantising x on the miss
    d = delta(mmq.mmq_decode_q6k, ctx, big, X2, O)
    assert d["launches_mmvq_q6k"] == 1 and d["cache_misses"] == 1 and d["launches_gemv_f32"] == 0
    # small, but x2 (id 5120) now has no plane of width 3584; x3 gets one first
    mmq.mmq_quant_f32(ctx, X3, 1, 3584)
    d = delta(mmq.mmq_decode_q6k, ctx, small, X3, O)
    assert d["launches_mmvq_q6k"] == 1 and d["cache_hits"] == 1 and d["launches_gemv_f32"] == 0
    # a skip-write producer's output: never read as f32, served from its plane
    mmq.mmq_quant_rms(ctx, X, W, Y, 1, 3584, 1e-6, 0)
    d = delta(mmq.mmq_decode_q6k, ctx, small, Y, O)
    assert d["launches_mmvq_q6k"] == 1 and d["cache_hits"] == 1 and d["launches_gemv_f32"] == 0
    # the explicit f32 path refuses it (and launches nothing)
    assert _status(mmq.mmq_gemv_q6k_f32, ctx, small, Y, O) == mmq.MMQ_E_DEAD_WRITE
    # too wide for the staged activation: explicit call refused, routed call quantises
    assert _status(mmq.mmq_gemv_q6k_f32, ctx, wide, X, O) == mmq.MMQ_E_SHAPE
    d = delta(mmq.mmq_decode_q6k, ctx, wide, X, O)
    assert d["launches_mmvq_q6k"] == 1 and d["launches_gemv_f32"] == 0
    # type and registration checks
    w4 = _w(ctx, mmq.MMQ_Q4_K, 64, 256, gv)
    w6g = _w(ctx, mmq.MMQ_Q6_K, 64, 256, mmq.MMQ_USE_GEMM)
    for fn in (mmq.mmq_gemv_q6k_f32, mmq.mmq_decode_q6k):
        assert _status(fn, ctx, w4, X, O) == mmq.MMQ_E_TYPE
        assert _status(fn, ctx, w6g, X, O) == mmq.MMQ_E_TYPE
        assert _status(fn, ctx, small, X + 4, O) == mmq.MMQ_E_ARG
    for w in (small, big, wide, w4, w6g):
        mmq.mmq_weight_free(w)


def test_consumer_type_checks(ctx):
    w4 = _w(ctx, mmq.MMQ_Q4_K, 512, 256)
    w6g = _w(ctx, mmq.MMQ_Q6_K, 64, 256, mmq.MMQ_USE_GEMM)
    A, O = 0x100000, 0x200000
    assert _status(mmq.mmq_gemm_q6k, ctx, w4, A, 8, O) == mmq.MMQ_E_TYPE
    assert _status(mmq.mmq_gemm_q4k, ctx, w6g, A, 8, O) == mmq.MMQ_E_TYPE
    assert _status(mmq.mmvq_q6k, ctx, w6g, A, O) == mmq.MMQ_E_TYPE     # not registered for GEMV
    assert _status(mmq.mmvq_q4k, ctx, w4, A, O) == mmq.MMQ_E_TYPE      # q4_K default: matmul only
    assert _status(mmq.mmvq_q4k, ctx, w6g, A, O) == mmq.MMQ_E_TYPE     # wrong type
    w4v = _w(ctx, mmq.MMQ_Q4_K, 64, 256, mmq.MMQ_USE_GEMV)
    assert _status(mmq.mmvq_q6k, ctx, w4v, A, O) == mmq.MMQ_E_TYPE
    assert _status(mmq.mmvq_q4k, ctx, w4v, A, O) == mmq.MMQ_OK
    assert mmq.mmq_stats(ctx)["launches_mmvq_q4k"] == 1
    assert _status(mmq.mmq_gemm_q4k, ctx, w4, A, 0, O) == mmq.MMQ_E_SHAPE
    other = mmq.mmq_create(0, mmq.MMQ_CTX_DRYRUN)
    try:
        assert _status(mmq.mmq_gemm_q4k, other, w4, A, 8, O) == mmq.MMQ_E_ARG
    finally:
        mmq.mmq_destroy(other)


def test_attention_chain_counts(ctx):
    """rms plane shared by q, k, v (3 hits); o's input misses once, then hits."""
    wq, wk = _w(ctx, mmq.MMQ_Q4_K, 512, 256), _w(ctx, mmq.MMQ_Q4_K, 128, 256)
    wv = _w(ctx, mmq.MMQ_Q6_K, 128, 256)
    X, W, Y, ATT, OUT = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    mmq.mmq_quant_rms(ctx, X, W, Y, 40, 256, 1e-6, 0)
    mmq.mmq_gemm_q4k(ctx, wq, Y, 40, OUT)
    mmq.mmq_gemm_q4k(ctx, wk, Y, 40, OUT)
    mmq.mmq_gemm_q6k(ctx, wv, Y, 40, OUT)
    mmq.mmq_gemm_q4k(ctx, wq, ATT, 40, OUT)
    mmq.mmq_gemm_q4k(ctx, wq, ATT, 40, OUT)
    st = mmq.mmq_stats(ctx)
    assert (st["cache_hits"], st["cache_misses"], st["launches_quant_rms"],
            st["launches_quant_f32"], st["launches_gemm_q4k"], st["launches_gemm_q6k"]) == (4, 1, 1, 1, 4, 1)
    assert st["cache_entries"] == 2
    mmq.mmq_cache_clear(ctx)
    assert mmq.mmq_stats(ctx)["cache_entries"] == 0


def test_dead_write_refusal_and_revival(ctx, capfd):
    w = _w(ctx, mmq.MMQ_Q4_K, 128, 256)
    Y = 0x1000000
    n, d = 100, 256
    mmq.mmq_quant_swiglu(ctx, 0x10000, 0x20000, Y, n, d, 0)          # dead [Y, Y + 102400)
    before = mmq.mmq_stats(ctx)
    assert _status(mmq.mmq_quant_f32, ctx, Y, n, d) == mmq.MMQ_E_DEAD_WRITE
    assert _status(mmq.mmq_quant_f32, ctx, Y + 4096, 10, d) == mmq.MMQ_E_DEAD_WRITE
    assert _status(mmq.mmq_gemm_q4k, ctx, w, Y, n - 1, 0x9000000) == mmq.MMQ_E_DEAD_WRITE
    mmq.mmq_gemm_q4k(ctx, w, Y, n, 0x9000000)                          # the recorded plane serves
    after = mmq.mmq_stats(ctx)
    assert after["cache_refusals"] - before["cache_refusals"] == 3
    assert after["launches_quant_f32"] == before["launches_quant_f32"]
    assert after["launches_gemm_q4k"] == before["launches_gemm_q4k"] + 1
    assert "refused" in capfd.readouterr().err
    # a real write into the middle revives exactly those bytes
    mid = Y + 40 * d * 4
    mmq.mmq_quant_rms(ctx, 0x10000, 0x20000, mid, 10, d, 1e-6, 1)
    assert _status(mmq.mmq_quant_f32, ctx, mid, 10, d) == mmq.MMQ_OK
    assert _status(mmq.mmq_quant_f32, ctx, mid - 1024, 1, d) == mmq.MMQ_E_DEAD_WRITE
    assert _status(mmq.mmq_quant_f32, ctx, mid + 10 * d * 4, 1, d) == mmq.MMQ_E_DEAD_WRITE
    # invalidate drops the dead range that starts at the key; clear drops all
    mmq.mmq_cache_invalidate(ctx, Y)
    assert _status(mmq.mmq_quant_f32, ctx, Y, 1, d) == mmq.MMQ_OK
    mmq.mmq_quant_swiglu(ctx, 0x10000, 0x20000, Y, n, d, 0)
    mmq.mmq_cache_clear(ctx)
    assert _status(mmq.mmq_quant_f32, ctx, Y, n, d) == mmq.MMQ_OK


def test_lru_eviction_keeps_recent_entries(ctx):
    w = _w(ctx, mmq.MMQ_Q4_K, 128, 256)
    keys = [0x1000000 * (i + 1) for i in range(10)]
    for k in keys:
        mmq.mmq_quant_f32(ctx, k, 8, 256)
    assert mmq.mmq_stats(ctx)["cache_entries"] == 8
    h0 = mmq.mmq_stats(ctx)["cache_hits"]
    mmq.mmq_gemm_q4k(ctx, w, keys[-1], 8, 0x9000000)    # recent: hit
    assert mmq.mmq_stats(ctx)["cache_hits"] == h0 + 1
    m0 = mmq.mmq_stats(ctx)["cache_misses"]
    mmq.mmq_gemm_q4k(ctx, w, keys[0], 8, 0x9000000)     # evicted: miss, re-quantised
    assert mmq.mmq_stats(ctx)["cache_misses"] == m0 + 1


def test_producer_replaces_stale_overlapping_entries(ctx):
    w = _w(ctx, mmq.MMQ_Q4_K, 128, 256)
    Y = 0x1000000
    mmq.mmq_quant_rms(ctx, 0x10000, 0x20000, Y, 64, 256, 1e-6, 1)
    mmq.mmq_quant_f32(ctx, Y + 256 * 4, 8, 256)          # plane of a sub-range of y
    mmq.mmq_quant_rms(ctx, 0x10000, 0x20000, Y, 64, 256, 1e-6, 1)   # y rewritten
    m0 = mmq.mmq_stats(ctx)["cache_misses"]
    mmq.mmq_gemm_q4k(ctx, w, Y + 256 * 4, 8, 0x9000000)  # stale sub-range plane was dropped
    assert mmq.mmq_stats(ctx)["cache_misses"] == m0 + 1


def test_consumer_output_drops_stale_planes_and_revives_dead_bytes(ctx):
    """A matmul's out that overwrites a key buffer: the old plane no longer
    serves (a miss re-quantises), and dead bytes it writes become readable."""
    w = _w(ctx, mmq.MMQ_Q4_K, 256, 256)          # out rows: n x 256 floats = n x 1 KiB
    K, n, d = 0x1000000, 8, 256
    mmq.mmq_quant_f32(ctx, K, n, d)               # plane of K recorded (live)
    mmq.mmq_gemm_q4k(ctx, w, 0x2000000, n, K)     # out = K: its contents change
    m0, h0 = mmq.mmq_stats(ctx)["cache_misses"], mmq.mmq_stats(ctx)["cache_hits"]
    mmq.mmq_gemm_q4k(ctx, w, K, n, 0x3000000)     # must not reuse K's old plane
    st = mmq.mmq_stats(ctx)
    assert (st["cache_misses"], st["cache_hits"]) == (m0 + 1, h0)
    # a dead key that a matmul has since written is readable again, exactly there
    Y = 0x5000000
    mmq.mmq_quant_rms(ctx, 0x10000, 0x20000, Y, 2 * n, d, 1e-6, 0)   # dead [Y, Y + 16 KiB)
    assert _status(mmq.mmq_quant_f32, ctx, Y, n, d) == mmq.MMQ_E_DEAD_WRITE
    mmq.mmq_gemm_q4k(ctx, w, 0x2000000, n, Y)     # writes [Y, Y + 8 KiB)
    assert _status(mmq.mmq_quant_f32, ctx, Y, n, d) == mmq.MMQ_OK
    assert _status(mmq.mmq_quant_f32, ctx, Y + n * d * 4, n, d) == mmq.MMQ_E_DEAD_WRITE
    # the one-token GEMV's output counts as a write too
    wv = _w(ctx, mmq.MMQ_Q6_K, 256, 256)
    Z = 0x7000000
    mmq.mmq_quant_swiglu(ctx, 0x10000, 0x30000, Z, 1, d, 0)         # dead [Z, Z + 1 KiB)
    mmq.mmvq_q6k(ctx, wv, 0x2000000, Z)
    assert _status(mmq.mmq_quant_f32, ctx, Z, 1, d) == mmq.MMQ_OK


def test_producers_refuse_dead_inputs(ctx, capfd):
    """RMSNorm and SwiGLU read their f32 inputs: a skip-write buffer (never
    written) as x, w, gate or up is refused before any launch."""
    Y, n, d = 0x1000000, 4, 256
    mmq.mmq_quant_swiglu(ctx, 0x10000, 0x20000, Y, n, d, 0)         # dead [Y, Y + 4 KiB)
    before = mmq.mmq_stats(ctx)
    for call in ((mmq.mmq_quant_rms, ctx, Y, 0x30000, 0x40000, n, d, 1e-6, 1),
                 (mmq.mmq_quant_rms, ctx, 0x30000, Y + 512, 0x40000, n, d, 1e-6, 1),
                 (mmq.mmq_quant_swiglu, ctx, Y, 0x30000, 0x40000, n, d, 1),
                 (mmq.mmq_quant_swiglu, ctx, 0x30000, Y + 1024, 0x40000, 1, d, 0)):
        assert _status(*call) == mmq.MMQ_E_DEAD_WRITE
    after = mmq.mmq_stats(ctx)
    assert after["cache_refusals"] == before["cache_refusals"] + 4
    for k in ("launches_quant_rms", "launches_quant_swiglu", "degraded_writes"):
        assert after[k] == before[k]
    assert "refused" in capfd.readouterr().err
    # inputs next to the dead range are fine
    mmq.mmq_quant_rms(ctx, Y + n * d * 4, 0x30000, 0x40000, n, d, 1e-6, 1)


def test_invalidate_drops_every_piece_of_the_dead_range(ctx):
    """After a partial write splits a dead range, invalidating its key drops
    the pieces on both sides; other producers' dead ranges stay."""
    w = _w(ctx, mmq.MMQ_Q4_K, 256, 256)
    Y, V, d = 0x1000000, 0x4000000, 256
    mmq.mmq_quant_rms(ctx, 0x10000, 0x20000, Y, 16, d, 1e-6, 0)     # dead [Y, Y + 16 KiB)
    mmq.mmq_quant_rms(ctx, 0x10000, 0x20000, V, 4, d, 1e-6, 0)      # another dead key
    mmq.mmq_gemm_q4k(ctx, w, 0x2000000, 4, Y + 4096)                # writes 4 KiB in the middle
    assert _status(mmq.mmq_quant_f32, ctx, Y + 12288, 4, d) == mmq.MMQ_E_DEAD_WRITE
    mmq.mmq_cache_invalidate(ctx, Y)
    assert _status(mmq.mmq_quant_f32, ctx, Y, 4, d) == mmq.MMQ_OK
    assert _status(mmq.mmq_quant_f32, ctx, Y + 12288, 4, d) == mmq.MMQ_OK
    assert _status(mmq.mmq_quant_f32, ctx, V, 4, d) == mmq.MMQ_E_DEAD_WRITE


def test_noalloc_decode_host_logic(ctx):
    """The allocation-free GEMV: a hit on a recorded plane, a miss that records
    nothing, dead-key refusal and the column limit, all before any launch."""
    d = 512
    w = _w(ctx, mmq.MMQ_Q6_K, 128, d)
    X = 0x1000000
    before = mmq.mmq_stats(ctx)
    mmq.mmvq_q6k_noalloc(ctx, w, X, 0x9000000)                      # miss: nothing recorded
    st = mmq.mmq_stats(ctx)
    assert (st["cache_misses"], st["launches_quant_f32"], st["launches_mmvq_q6k"],
            st["cache_entries"], st["plane_bytes"]) == (
        before["cache_misses"] + 1, before["launches_quant_f32"] + 1,
        before["launches_mmvq_q6k"] + 1, before["cache_entries"], before["plane_bytes"])
    mmq.mmq_quant_f32(ctx, X, 1, d)                                  # now a recorded plane
    h0 = mmq.mmq_stats(ctx)["cache_hits"]
    mmq.mmvq_q6k_noalloc(ctx, w, X, 0x9000000)                      # hit
    assert mmq.mmq_stats(ctx)["cache_hits"] == h0 + 1
    Y = 0x2000000
    mmq.mmq_quant_rms(ctx, 0x10000, 0x20000, Y, 4, d, 1e-6, 0)      # dead [Y, Y + 8 KiB)
    assert _status(mmq.mmvq_q6k_noalloc, ctx, w, Y + 4096, 0x9000000) == mmq.MMQ_E_DEAD_WRITE
    wide = _w(ctx, mmq.MMQ_Q6_K, 4, mmq.MMQ_NOALLOC_MAX_COLS + 256)
    before = mmq.mmq_stats(ctx)
    assert _status(mmq.mmvq_q6k_noalloc, ctx, wide, X, 0x9000000) == mmq.MMQ_E_SHAPE
    assert "exceeds" in mmq.last_error()
    assert mmq.mmq_stats(ctx) == before
    assert _status(mmq.mmvq_q6k_noalloc, ctx, _w(ctx, mmq.MMQ_Q6_K, 4, 256, mmq.MMQ_USE_GEMM),
                   X, 0x9000000) == mmq.MMQ_E_TYPE                  # no GEMV tiles


def test_scratch_cap(ctx):
    mmq.mmq_set_scratch_cap(ctx, 64 * 1024)
    assert _status(mmq.mmq_quant_f32, ctx, 0x100000, 32, 512) == mmq.MMQ_OK     # ~21 KB
    assert _status(mmq.mmq_quant_f32, ctx, 0x200000, 1024, 512) == mmq.MMQ_E_OOM
    st = mmq.mmq_stats(ctx)
    assert st["plane_bytes"] <= 64 * 1024 and st["launches_quant_f32"] == 1
    mmq.mmq_set_scratch_cap(ctx, -1)
    assert _status(mmq.mmq_quant_f32, ctx, 0x200000, 1024, 512) == mmq.MMQ_OK


def test_export_needs_a_plane_aligned_buffers_and_a_device(ctx):
    assert _status(mmq.mmq_plane_export, ctx, 0x100000, 8, 256, 0, 0x1000, 0x2000, 0x3000) == mmq.MMQ_E_ARG
    mmq.mmq_quant_f32(ctx, 0x100000, 8, 256)
    # the scales and sums are written as 4-byte words
    for dq, s in ((0x2002, 0x3000), (0x2000, 0x3001)):
        rc = _lib.lib.mmq_plane_export(ctx, 0x100000, 8, 256, 0, 0x1000, dq, s, None)
        assert rc == mmq.MMQ_E_ARG
    rc = _lib.lib.mmq_plane_export(ctx, 0x100000, 8, 256, 0, 0x1000, 0x2000, 0x3000, None)
    assert rc == mmq.MMQ_E_DEVICE


def test_degradation_ladder_follows_the_consumer_set(ctx, capfd):
    """Skip-write is honoured only while every consumer reads planes; a foreign
    (f32-reading) consumer makes write_y=0 and MMQ_WRITE_AUTO write y as well."""
    w = _w(ctx, mmq.MMQ_Q4_K, 128, 256)
    X, W, Y, O = 0x100000, 0x200000, 0x1000000, 0x3000000
    assert mmq.mmq_plane_only(ctx)
    mmq.mmq_quant_rms(ctx, X, W, Y, 8, 256, 1e-6, mmq.MMQ_WRITE_AUTO)
    assert _status(mmq.mmq_quant_f32, ctx, Y, 8, 256) == mmq.MMQ_E_DEAD_WRITE   # skipped: dead
    mmq.mmq_cache_clear(ctx)
    assert _status(mmq.mmq_register_foreign_consumer, ctx, 7) == mmq.MMQ_E_ARG
    capfd.readouterr()
    mmq.mmq_register_foreign_consumer(ctx, mmq.MMQ_FOREIGN_F32)
    assert "f32" in capfd.readouterr().err
    assert not mmq.mmq_plane_only(ctx)
    mmq.mmq_quant_rms(ctx, X, W, Y, 8, 256, 1e-6, 0)        # degraded: y written, entry live
    mmq.mmq_gemm_q4k(ctx, w, Y, 8, O)                        # hit
    assert _status(mmq.mmq_quant_f32, ctx, Y, 8, 256) == mmq.MMQ_OK    # not dead
    mmq.mmq_quant_swiglu(ctx, X, W, Y, 8, 256, mmq.MMQ_WRITE_AUTO)
    st = mmq.mmq_stats(ctx)
    assert st["degraded_writes"] == 2 and st["cache_refusals"] == 1 and st["cache_hits"] == 1
    assert _status(mmq.mmq_quant_rms, ctx, X, W, Y, 8, 256, 1e-6, 2) == mmq.MMQ_E_ARG


def test_auto_falls_back_to_unfused_without_plane_memory(ctx, capfd):
    """MMQ_WRITE_AUTO: no plane memory -> y written alone, nothing recorded; a
    consumer then quantises y itself and fails loudly if it cannot either."""
    w = _w(ctx, mmq.MMQ_Q4_K, 128, 256)
    X, W, Y, O = 0x100000, 0x200000, 0x1000000, 0x3000000
    mmq.mmq_set_scratch_cap(ctx, 0)
    capfd.readouterr()
    assert _status(mmq.mmq_quant_rms, ctx, X, W, Y, 8, 256, 1e-6, mmq.MMQ_WRITE_AUTO) == mmq.MMQ_OK
    assert "without a plane" in capfd.readouterr().err
    st = mmq.mmq_stats(ctx)
    assert st["unfused_fallbacks"] == 1 and st["cache_entries"] == 0
    assert st["launches_quant_rms"] == 1
    assert _status(mmq.mmq_gemm_q4k, ctx, w, Y, 8, O) == mmq.MMQ_E_OOM     # miss, no memory
    # an explicit skip-write request does not fall back: it fails before any launch
    assert _status(mmq.mmq_quant_rms, ctx, X, W, Y, 8, 256, 1e-6, 0) == mmq.MMQ_E_OOM
    mmq.mmq_set_scratch_cap(ctx, -1)
    mmq.mmq_quant_rms(ctx, X, W, Y, 8, 256, 1e-6, mmq.MMQ_WRITE_AUTO)
    assert mmq.mmq_stats(ctx)["cache_entries"] == 1


def test_split_k_scratch_is_checked_before_any_launch(ctx):
    """A matmul with few output tiles holds K-split partials in the context's
    scratch; a cap that cannot hold them fails before anything is enqueued."""
    w = _w(ctx, mmq.MMQ_Q6_K, 3584, 18944, mmq.MMQ_USE_GEMM)
    A, O = 0x100000, 0x200000
    plane = mmq.mmq_plane_rows(8) * 18944 * 5 // 4
    mmq.mmq_set_scratch_cap(ctx, plane + 3584 * 8 * 4)        # room for one split only
    st0 = mmq.mmq_stats(ctx)
    assert _status(mmq.mmq_gemm_q6k, ctx, w, A, 8, O) == mmq.MMQ_E_OOM
    st1 = mmq.mmq_stats(ctx)
    assert st1["launches_gemm_q6k"] == st0["launches_gemm_q6k"]
    assert st1["cache_misses"] == st0["cache_misses"] and st1["launches_quant_f32"] == 0
    mmq.mmq_set_scratch_cap(ctx, -1)
    mmq.mmq_gemm_q6k(ctx, w, A, 8, O)
    part = mmq.mmq_stats(ctx)["plane_bytes"] - plane
    assert part % (3584 * 8 * 4) == 0 and part // (3584 * 8 * 4) >= 2     # 3584*8 is a multiple of 64
    # many output tiles whose last round is well filled: no split, no partials
    c2 = mmq.mmq_create(0, mmq.MMQ_CTX_DRYRUN)
    try:
        plane = mmq.mmq_plane_rows(3314) * 3584 * 5 // 4
        w2 = _w(c2, mmq.MMQ_Q4_K, 3584, 3584, mmq.MMQ_USE_GEMM)     # 728 tiles: 2.84 rounds
        mmq.mmq_gemm_q4k(c2, w2, A, 3314, O)
        assert mmq.mmq_stats(c2)["plane_bytes"] == plane
        # 3848 tiles = 15 rounds + 8: the 8 leftover tiles run K-split (14 superblocks ->
        # 14 splits) into compact 128 x 128 partial tiles
        w3 = _w(c2, mmq.MMQ_Q4_K, 18944, 3584, mmq.MMQ_USE_GEMM)
        mmq.mmq_gemm_q4k(c2, w3, A, 3314, O)
        assert mmq.mmq_stats(c2)["plane_bytes"] == plane + 14 * 8 * 128 * 128 * 4
    finally:
        mmq.mmq_destroy(c2)


def test_small_n_routing(ctx):
    """On a weight registered for both paths the GEMV path serves the call
    when one pass of the LDS holds the tokens (8 at width 5120, 4 at 18944),
    or when two passes do and n <= 8 or rows * cols <= 16M; otherwise (and
    always beyond 16 tokens) the matmul tiles."""
    both = mmq.MMQ_USE_GEMM | mmq.MMQ_USE_GEMV
    w = _w(ctx, mmq.MMQ_Q4_K, 256, 5120, both)            # 1.3M weights
    wg = _w(ctx, mmq.MMQ_Q4_K, 256, 5120, mmq.MMQ_USE_GEMM)
    wd = _w(ctx, mmq.MMQ_Q6_K, 256, 18944, both)           # 4.8M weights, 4 tokens per pass
    wb = _w(ctx, mmq.MMQ_Q4_K, 3328, 5120, both)           # 17.0M weights
    wl = _w(ctx, mmq.MMQ_Q6_K, 1024, 18944, both)          # 19.4M weights, 4 tokens per pass
    A, O = 0x100000, 0x4000000
    for n, weight, fn, routed in [(1, w, mmq.mmq_gemm_q4k, 1), (8, w, mmq.mmq_gemm_q4k, 1),
                                  (9, w, mmq.mmq_gemm_q4k, 1), (16, w, mmq.mmq_gemm_q4k, 1),
                                  (17, w, mmq.mmq_gemm_q4k, 0), (4, wg, mmq.mmq_gemm_q4k, 0),
                                  (8, wb, mmq.mmq_gemm_q4k, 1), (9, wb, mmq.mmq_gemm_q4k, 0),
                                  (4, wd, mmq.mmq_gemm_q6k, 1), (5, wd, mmq.mmq_gemm_q6k, 1),
                                  (8, wd, mmq.mmq_gemm_q6k, 1), (9, wd, mmq.mmq_gemm_q6k, 0),
                                  (8, wl, mmq.mmq_gemm_q6k, 1), (9, wl, mmq.mmq_gemm_q6k, 0)]:
        before = mmq.mmq_stats(ctx)["small_n_gemv"]
        fn(ctx, weight, A + n * 0x10000000, n, O)
        assert mmq.mmq_stats(ctx)["small_n_gemv"] - before == routed, (n, routed)


def test_failed_producer_leaves_dead_marks(ctx):
    """A producer that fails before its launch (no plane memory) must not
    revive the dead range of a buffer it never wrote."""
    X, W, Y = 0x100000, 0x200000, 0x1000000
    mmq.mmq_quant_rms(ctx, X, W, Y, 8, 256, 1e-6, 0)           # Y promised unread
    mmq.mmq_set_scratch_cap(ctx, mmq.mmq_stats(ctx)["plane_bytes"])
    assert _status(mmq.mmq_quant_rms, ctx, X, W, Y, 64, 2048, 1e-6, 1) == mmq.MMQ_E_OOM
    assert _status(mmq.mmq_quant_f32, ctx, Y, 8, 256) == mmq.MMQ_E_DEAD_WRITE
    mmq.mmq_set_scratch_cap(ctx, -1)


def test_binding_checks_the_raw_buffer_size(ctx):
    with pytest.raises(ValueError):
        mmq.mmq_register_weight(ctx, mmq.MMQ_Q4_K, 4, 256, np.zeros(144 * 3, np.uint8))
    w = mmq.mmq_register_weight(ctx, mmq.MMQ_Q6_K, 2, 512, bytes(2 * 2 * 210))
    mmq.mmq_weight_free(w)


def test_size_limits_of_the_32_bit_buffer_offsets(ctx):
    """The matmul addresses its tiles and the plane with 32-bit buffer offsets,
    so registration refuses matmul tiles of 4 GiB or more and a matmul call
    refuses a plane of 2 GiB or more, both with MMQ_E_SHAPE and a message that
    says how to split; nothing is launched and no plane is recorded."""
    out = ctypes.c_void_p()
    # 2^20 x 2048 q4_K: f16 tiles of exactly 4 GiB (the raw buffer is never
    # read: the shape is refused first, so a dummy address stands in for it)
    rc = _lib.lib.mmq_register_weight(ctx, mmq.MMQ_Q4_K, 1 << 20, 2048, ctypes.c_void_p(0x1000),
                                      mmq.MMQ_USE_GEMM, ctypes.byref(out))
    assert rc == mmq.MMQ_E_SHAPE and "4 GiB" in _lib.last_error()
    assert out.value is None
    # one row fewer than a 128-row tile group below the limit is accepted
    rc = _lib.lib.mmq_register_weight(ctx, mmq.MMQ_Q4_K, (1 << 20) - 128, 2048,
                                      ctypes.c_void_p(0x1000), mmq.MMQ_USE_GEMM, ctypes.byref(out))
    assert rc == mmq.MMQ_OK
    big = out.value
    # GEMV-only registration has no matmul tiles and no such limit
    rc = _lib.lib.mmq_register_weight(ctx, mmq.MMQ_Q6_K, 1 << 20, 2048, ctypes.c_void_p(0x1000),
                                      mmq.MMQ_USE_GEMV, ctypes.byref(out))
    assert rc == mmq.MMQ_OK
    mmq.mmq_weight_free(out.value)
    w = _w(ctx, mmq.MMQ_Q4_K, 128, 2048)
    st0 = mmq.mmq_stats(ctx)
    n = (1 << 31) // 2048             # plane of exactly 2 GiB of codes
    assert _status(mmq.mmq_gemm_q4k, ctx, w, 0x10000000, n, 0x20000000) == mmq.MMQ_E_SHAPE
    assert "2 GiB" in _lib.last_error()
    st1 = mmq.mmq_stats(ctx)
    assert st1["launches_gemm_q4k"] == st0["launches_gemm_q4k"]
    assert st1["launches_quant_f32"] == st0["launches_quant_f32"]
    assert st1["cache_entries"] == st0["cache_entries"]
    # 32 tokens fewer (the plane's row padding) fits
    assert _status(mmq.mmq_gemm_q4k, ctx, w, 0x10000000, n - 32, 0x20000000) == mmq.MMQ_OK
    mmq.mmq_weight_free(w)
    mmq.mmq_weight_free(big)
