"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Inputs come from synth.py (seeded); expected values come only from oracle/.
Planes are compared on the canonical export; matmuls against the oracle run on
the GPU's exported plane (which isolates the matmul from producer rounding).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_rmsnorm_amd as mmq
import synth
from tests.gpu_util import (GemmRef, assert_fused_close, assert_gemm_close, assert_plane_equal,
                            dev_tensor, export_plane, gemm_ref)

pytestmark = pytest.mark.gpu
EPS = synth.EPS
WT = {"q4_K": 12, "q6_K": 14}


@pytest.fixture(scope="module")
def _module_ctx():
    c = mmq.mmq_create(0, 0)
    yield c
    mmq.mmq_destroy(c)


@pytest.fixture
def ctx(_module_ctx):
    # each test is its own execution window: buffers freed by an earlier test
    # may come back at the same addresses
    mmq.mmq_cache_clear(_module_ctx)
    return _module_ctx


def _act(tag, n, d, spread=True):
    rng = synth.rng_for("test", n * 100003 + d, tag)
    y = synth.activations(rng, n, d)
    if spread:  # rows and blocks of very different magnitude, a few all-zero blocks
        y *= rng.uniform(0.05, 20.0, (n, 1)).astype(np.float32)
        y.reshape(n, -1, 32)[:, ::7, :] *= np.float32(1e-3)
        if n * d >= 64:
            y.reshape(-1, 32)[::13] = 0.0
    return np.ascontiguousarray(y, np.float32)


# ------------------------------------------------------------------ producers
@pytest.mark.parametrize("n,d", [(1, 256), (37, 512), (64, 3584), (3, 5120), (5, 18944),
                                 (3314, 3584)])
def test_quant_f32_bit_exact(ctx, n, d):
    y = _act("qf32", n, d)
    x = dev_tensor(y)
    mmq.mmq_quant_f32(ctx, x, n, d)
    assert_plane_equal(export_plane(ctx, x, n, d), oracle.quantize(y), f"quant_f32 {n}x{d}")


def test_quant_f32_special_values(ctx):
    n, d = 5, 256
    y = np.zeros((n, d), np.float32)
    y[0, :32] = 1e-40                     # subnormal block
    y[0, 32:64] = np.linspace(-3e-39, 3e-39, 32)
    y[1, :32] = 3e38                      # near the top of the range
    y[1, 40] = -1e-30                     # lone tiny value
    y[2, ::2] = 2.5                       # ties around the code grid
    y[2, 1::2] = 127.0
    y[3] = np.float32(7.0) / np.float32(3.0)
    tiny = np.float32(2.0 ** -149)            # scale underflow: amax / 127 rounds to 0
    y[4, 0], y[4, 5] = 10 * tiny, -3 * tiny
    y[4, 32], y[4, 33] = 63 * tiny, -63 * tiny
    y[4, 64], y[4, 65], y[4, 66] = 190 * tiny, 64 * tiny, -3 * tiny   # D = 2^-149, clamped code
    y[4, 96:128] = -tiny
    x = dev_tensor(y)
    mmq.mmq_quant_f32(ctx, x, n, d)
    assert_plane_equal(export_plane(ctx, x, n, d), oracle.quantize(y), "special values")


# up to 4 rows take the 8-wave form (d up to 16384, its 64 rounds at 3 x 16384;
# 4 rows at 4096, and 5 rows at 4096 take the 4-wave form); d 8192 and 16384
# fill the 8- and 16-round register forms of the 4-wave form; 16640 and 18944
# re-read x for the second pass
@pytest.mark.parametrize("n,d", [(37, 512), (128, 3584), (1, 5120), (3314, 3584), (2, 8192),
                                 (3, 16384), (2, 16640), (2, 18944), (4, 4096), (5, 4096),
                                 (9, 16384)])
def test_quant_rms_fused_and_cross_mode(ctx, n, d):
    rng = synth.rng_for("test", n, f"rms{d}")
    xh = synth.activations(rng, n, d)
    wh = synth.rms_weight(rng, d)
    y_ref = oracle.rmsnorm(xh, wh, EPS)
    ref = oracle.quantize(y_ref)
    x, w = dev_tensor(xh), dev_tensor(wh)
    y1 = torch.empty((n, d), dtype=torch.float32, device="cuda")
    y0 = torch.empty((n, d), dtype=torch.float32, device="cuda")
    mmq.mmq_quant_rms(ctx, x, w, y1, n, d, EPS, 1)
    p1 = export_plane(ctx, y1, n, d)
    mmq.mmq_quant_rms(ctx, x, w, y0, n, d, EPS, 0)
    p0 = export_plane(ctx, y0, n, d)
    y_gpu = y1.cpu().numpy()
    mmq.mmq_quant_f32(ctx, y1, n, d)          # standalone quantise of the written y
    pf = export_plane(ctx, y1, n, d)
    assert_plane_equal(p0, p1, "write_y=0 vs 1")
    assert_plane_equal(pf, p1, "standalone vs fused")
    assert_plane_equal(oracle.quantize(y_gpu), p1, "oracle quantiser on the GPU's y")
    assert_fused_close(p1, ref, y_gpu, y_ref, f"rms {n}x{d}")
    rel = np.abs(y_gpu.astype(np.float64) - y_ref) / np.maximum(np.abs(y_ref), 1e-30)
    assert rel.max() < 4e-7


@pytest.mark.parametrize("n,d", [(37, 512), (64, 18944), (1, 13824), (3314, 18944)])
def test_quant_swiglu_fused_and_cross_mode(ctx, n, d):
    rng = synth.rng_for("test", n, f"swiglu{d}")
    gh = synth.activations(rng, n, d)
    uh = synth.activations(rng, n, d)
    y_ref = oracle.swiglu(gh, uh)
    ref = oracle.quantize(y_ref)
    g, u = dev_tensor(gh), dev_tensor(uh)
    y1 = torch.empty((n, d), dtype=torch.float32, device="cuda")
    y0 = torch.empty((n, d), dtype=torch.float32, device="cuda")
    mmq.mmq_quant_swiglu(ctx, g, u, y1, n, d, 1)
    p1 = export_plane(ctx, y1, n, d)
    mmq.mmq_quant_swiglu(ctx, g, u, y0, n, d, 0)
    p0 = export_plane(ctx, y0, n, d)
    y_gpu = y1.cpu().numpy()
    mmq.mmq_quant_f32(ctx, y1, n, d)
    pf = export_plane(ctx, y1, n, d)
    assert_plane_equal(p0, p1, "write_y=0 vs 1")
    assert_plane_equal(pf, p1, "standalone vs fused")
    assert_fused_close(p1, ref, y_gpu, y_ref, f"swiglu {n}x{d}")
    rel = np.abs(y_gpu.astype(np.float64) - y_ref) / np.maximum(np.abs(y_ref), 1e-30)
    assert np.quantile(rel, 0.999999) < 1e-6


def test_padded_rows_zero_after_poisoned_slot(ctx):
    """A slot that held a bigger plane is reused for a smaller one: the padded
    rows must come back zero, not stale."""
    d = 512
    mmq.mmq_cache_clear(ctx)
    big = dev_tensor(_act("poison", 64, d) + np.float32(5.0))
    keys = [big]
    mmq.mmq_quant_f32(ctx, big, 64, d)
    # fill every slot with non-zero planes, then clear and write a 37-row plane
    for i in range(8):
        t = dev_tensor(_act(f"poison{i}", 64, d) + np.float32(3.0))
        keys.append(t)
        mmq.mmq_quant_f32(ctx, t, 64, d)
    mmq.mmq_cache_clear(ctx)
    xh = synth.activations(synth.rng_for("test", 0, "padrms"), 37, d)
    wh = synth.rms_weight(synth.rng_for("test", 1, "padrms"), d)
    y = torch.empty((37, d), dtype=torch.float32, device="cuda")
    mmq.mmq_quant_rms(ctx, dev_tensor(xh), dev_tensor(wh), y, 37, d, EPS, 0)
    q, D, S = export_plane(ctx, y, 37, d, include_pad=True)
    assert q.shape[0] == 64
    assert not q[37:].any() and not D[37:].any() and not S[37:].any()
    assert q[:37].any()


# ------------------------------------------------------------------ matmuls
def _gemm_case(ctx, wtype, n, od, id_, tag):
    rng = synth.rng_for("test", n * 7 + od, f"{tag}{wtype}{id_}")
    raw = synth.weights(wtype, rng, od, id_)
    ah = _act(tag, n, id_)
    w = mmq.mmq_register_weight(ctx, WT[wtype], od, id_, raw, 1)
    a = dev_tensor(ah)
    out = torch.full((n, od), float("nan"), dtype=torch.float32, device="cuda")
    fn = mmq.mmq_gemm_q4k if wtype == "q4_K" else mmq.mmq_gemm_q6k
    fn(ctx, w, a, n, out)
    torch.cuda.synchronize()
    plane = export_plane(ctx, a, n, id_)
    return w, raw, plane, out.cpu().numpy()


@pytest.mark.parametrize("wtype", ["q4_K", "q6_K"])
@pytest.mark.parametrize("n,od,id_", [(1, 128, 256), (37, 256, 512), (200, 384, 1024),
                                      (130, 1000, 768), (16, 32, 2304)])
def test_gemm_parity(ctx, wtype, n, od, id_):
    w, raw, (q, D, S), got = _gemm_case(ctx, wtype, n, od, id_, "gemm")
    ref = gemm_ref(wtype, q, D, S, raw, od, id_)
    assert_gemm_close(got, ref, f"{wtype} n={n} od={od} id={id_}")
    mmq.mmq_weight_free(w)


def test_tiny_chain_rms_plane_q4k(ctx):
    """The tiny workload end to end: 32 tokens x hidden 256, the RMSNorm
    producer (weight in [0.5, 1.5), eps 1e-6) into a skip-write plane, then the
    q4_K 512 x 256 matmul, which finds that plane in the cache.  The plane
    equals the one written with y and meets the fused bar against the oracle;
    the matmul meets the element-wise bar on it."""
    cfg = synth.CONFIGS["tiny"]
    n, d, od = cfg["n"], cfg["hidden"], cfg["od"]
    rng = synth.rng_for("test", n, "tinychain")
    xh = synth.activations(rng, n, d)
    wh = synth.rms_weight(rng, d)
    raw = synth.q4k_weights(rng, od, d)
    y_ref = oracle.rmsnorm(xh, wh, EPS)
    w = mmq.mmq_register_weight(ctx, mmq.MMQ_Q4_K, od, d, raw, mmq.MMQ_USE_GEMM)
    x, g = dev_tensor(xh), dev_tensor(wh)
    y0 = torch.empty((n, d), dtype=torch.float32, device="cuda")   # never written
    y1 = torch.empty((n, d), dtype=torch.float32, device="cuda")
    out = torch.full((n, od), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmq_quant_rms(ctx, x, g, y0, n, d, EPS, 0)
    hits, misses = mmq.mmq_stats(ctx)["cache_hits"], mmq.mmq_stats(ctx)["cache_misses"]
    mmq.mmq_gemm_q4k(ctx, w, y0, n, out)
    st = mmq.mmq_stats(ctx)
    assert (st["cache_hits"], st["cache_misses"]) == (hits + 1, misses)
    p0 = export_plane(ctx, y0, n, d)
    mmq.mmq_quant_rms(ctx, x, g, y1, n, d, EPS, 1)
    p1 = export_plane(ctx, y1, n, d)
    torch.cuda.synchronize()
    assert_plane_equal(p0, p1, "tiny: skip-write vs written plane")
    assert_fused_close(p1, oracle.quantize(y_ref), y1.cpu().numpy(), y_ref, "tiny rms")
    ref = gemm_ref("q4_K", *p0, raw, od, d)
    assert_gemm_close(out.cpu().numpy(), ref, "tiny q4_K 512x256")
    mmq.mmq_weight_free(w)


@pytest.mark.parametrize("wtype", ["q4_K", "q6_K", "q4_K packed"])
def test_gemm_degenerate_activation_rows(ctx, wtype):
    """Rows the plane encodes at its edges: all zero (D = 0, S = 0), one
    nonzero block among zero blocks, one nonzero value per block, and row
    scales from 1e-20 to 1e20; n = 40 (a ragged token tile), od = 200."""
    n, od, id_ = 40, 200, 1024
    rng = synth.rng_for("test", n, f"degen{wtype}")
    y = synth.activations(rng, n, id_)
    y[0] = 0.0
    y[1] = 0.0
    y[1, 256:288] = y[2, 256:288]
    y[3] = 0.0
    y[3, ::32] = np.linspace(-5.0, 5.0, id_ // 32, dtype=np.float32)
    y[4] *= np.float32(1e20)
    y[5] *= np.float32(1e-20)
    y[6, :512] = 0.0
    y = np.ascontiguousarray(y, np.float32)
    packed = wtype.endswith("packed")
    wtype = wtype.split()[0]
    raw = synth.weights(wtype, synth.rng_for("test", od, f"degenw{wtype}"), od, id_)
    w = mmq.mmq_register_weight(ctx, WT[wtype], od, id_, raw,
                                mmq.MMQ_USE_GEMM | (mmq.MMQ_USE_GEMM_PACKED if packed else 0))
    a = dev_tensor(y)
    out = torch.full((n, od), float("nan"), dtype=torch.float32, device="cuda")
    (mmq.mmq_gemm_q4k if wtype == "q4_K" else mmq.mmq_gemm_q6k)(ctx, w, a, n, out)
    torch.cuda.synchronize()
    q, D, S = export_plane(ctx, a, n, id_)
    assert_plane_equal((q, D, S), oracle.quantize(y), "degenerate rows plane")
    got = out.cpu().numpy()
    assert not got[0].any() and np.isfinite(got).all()
    ref = gemm_ref(wtype, q, D, S, raw, od, id_)
    assert_gemm_close(got, ref, f"degenerate rows {wtype}")
    # the 1e-20 row also at its own unit scale, where the +1 of the bar would
    # otherwise accept anything
    s5 = 1e20
    assert_gemm_close(got[5].astype(np.float64) * s5,
                      GemmRef(ref.out[5].astype(np.float64) * s5, ref.mag[5] * s5, ref.nsb),
                      f"degenerate row 5 at unit scale {wtype}")
    mmq.mmq_weight_free(w)


@pytest.mark.parametrize("wtype,n,od,id_", [("q4_K", 2, 1000, 5120), ("q6_K", 3, 300, 13824),
                                            ("q4_K", 5, 13824, 5120), ("q6_K", 8, 3584, 18944),
                                            ("q6_K", 4, 3584, 18944),
                                            ("q6_K", 6, 64, 256), ("q4_K", 1, 700, 2048),
                                            ("q4_K", 7, 33, 20480), ("q4_K", 12, 3584, 3584),
                                            ("q6_K", 16, 512, 3584), ("q4_K", 11, 600, 13824),
                                            ("q4_K", 9, 4096, 5120)])
def test_gemm_small_n_gemv_path(ctx, wtype, n, od, id_):
    """A weight registered for both paths runs on the dot4 GEMV kernels when
    one pass of the LDS holds the n tokens, or two passes do and n <= 8 or
    od * id <= 16M (the 18944-wide plane holds 4 tokens, so n = 8 there takes
    two passes; n = 9 on 4096 x 5120 takes the matmul tiles); the outputs of
    either path meet the matmul bar."""
    rng = synth.rng_for("test", n * 7 + od, f"smalln{wtype}{id_}")
    raw = synth.weights(wtype, rng, od, id_)
    w = mmq.mmq_register_weight(ctx, WT[wtype], od, id_, raw, mmq.MMQ_USE_GEMM | mmq.MMQ_USE_GEMV)
    a = dev_tensor(_act("smalln", n, id_))
    out = torch.full((n, od), float("nan"), dtype=torch.float32, device="cuda")
    before = mmq.mmq_stats(ctx)["small_n_gemv"]
    (mmq.mmq_gemm_q4k if wtype == "q4_K" else mmq.mmq_gemm_q6k)(ctx, w, a, n, out)
    torch.cuda.synchronize()
    rec = id_ // 32 * 40                     # LDS bytes per token: 40 B per 32-block
    per_pass = max([t for t in (2, 4, 8) if t * rec <= 160 * 1024], default=0)
    passes = -(-n // per_pass) if per_pass else 0
    gemv = n <= 16 and (passes == 1 or (passes == 2 and (n <= 8 or od * id_ <= 16_000_000)))
    assert mmq.mmq_stats(ctx)["small_n_gemv"] == before + (1 if gemv else 0)
    q, D, S = export_plane(ctx, a, n, id_)
    ref = gemm_ref(wtype, q, D, S, raw, od, id_)
    assert_gemm_close(out.cpu().numpy(), ref, f"small-n {wtype} n={n} {od}x{id_}")
    mmq.mmq_weight_free(w)


@pytest.mark.parametrize("wtype,n,od,id_", [("q6_K", 8, 3584, 18944), ("q4_K", 3, 18944, 3584),
                                            ("q4_K", 70, 512, 2560), ("q6_K", 1, 1000, 5120),
                                            ("q4_K", 130, 384, 4864), ("q6_K", 9, 1001, 2560)])
def test_gemm_split_k_parity(ctx, wtype, n, od, id_):
    """Few output tiles: the matmul splits K across workgroups (partials summed
    in split order by a second kernel), including splits of unequal length."""
    w, raw, (q, D, S), got = _gemm_case(ctx, wtype, n, od, id_, "splitk")
    before = mmq.mmq_stats(ctx)["plane_bytes"]
    assert before > mmq.mmq_plane_rows(n) * id_ * 1.25   # the partial scratch is held too
    ref = gemm_ref(wtype, q, D, S, raw, od, id_)
    assert_gemm_close(got, ref, f"split-K {wtype} n={n} {od}x{id_}")
    mmq.mmq_weight_free(w)


@pytest.mark.parametrize("wtype", ["q4_K", "q6_K"])
def test_gemm_tail_round_split(ctx, wtype):
    """258 output tiles on 256 CUs: 256 run whole, the 2 leftover tiles (the
    last output tile, both token tiles) run K-split into compact partial tiles
    summed by the tile reduce.  All outputs of the leftover tiles are checked,
    plus sampled others."""
    n, od, id_ = 256, 16512, 1024
    w, raw, (q, D, S), got = _gemm_case(ctx, wtype, n, od, id_, "tail")
    rng = np.random.default_rng(11)
    outs = np.unique(np.concatenate([np.arange(16384, od), rng.integers(0, 16384, 200)]))
    ref = gemm_ref(wtype, q, D, S, raw, od, id_, outs=outs)
    assert_gemm_close(got[:, outs], ref, f"tail split {wtype}")
    mmq.mmq_weight_free(w)


@pytest.mark.parametrize("wtype,od,id_", [("q4_K", 18944, 3584), ("q6_K", 3584, 18944),
                                          ("q4_K", 3584, 3584), ("q4_K", 512, 3584),
                                          ("q6_K", 512, 3584)])
def test_gemm_full_size_sampled(ctx, wtype, od, id_):
    n = 3314
    w, raw, (q, D, S), got = _gemm_case(ctx, wtype, n, od, id_, "full")
    rng = np.random.default_rng(od + id_)
    tok = np.unique(np.concatenate([[0, 1, 31, 32, 127, 128, 3199, 3200, 3313],
                                    rng.integers(0, n, 7)]))
    outs = np.unique(np.concatenate([[0, 31, 32, 127, 128, od - 1],
                                     rng.integers(0, od, 250)]))
    ref = gemm_ref(wtype, q, D, S, raw, od, id_, tok=tok, outs=outs)
    assert_gemm_close(got[np.ix_(tok, outs)], ref, f"{wtype} {od}x{id_} sampled")
    assert np.isfinite(got).all()
    mmq.mmq_weight_free(w)


# ------------------------------------------------------------------ packed q4_K tiles
PACKED_SHAPES = [(1, 128, 256), (37, 256, 512), (200, 384, 1024), (130, 1000, 768),
                 (16, 32, 2304), (70, 512, 2560), (130, 384, 4864), (3, 18944, 3584),
                 (3314, 512, 3584), (3314, 3584, 3584), (3314, 18944, 3584)]


@pytest.mark.parametrize("n,od,id_", PACKED_SHAPES)
def test_gemm_packed_q4k_bit_identical(ctx, n, od, id_):
    """A q4_K weight registered with its 4-bit codes (MMQ_USE_GEMM_PACKED)
    returns the same bits as from the f16 tiles on every output: ragged
    shapes, the K split (few output tiles), full rounds, and the tail split of
    the 18944 x 3584 gate at 3314 tokens; small shapes also meet the oracle's
    bar on every output.  The tiles take about a third of the bytes."""
    rng = synth.rng_for("test", n * 7 + od, f"packed{id_}")
    raw = synth.weights("q4_K", rng, od, id_)
    wf = mmq.mmq_register_weight(ctx, WT["q4_K"], od, id_, raw, mmq.MMQ_USE_GEMM)
    wp = mmq.mmq_register_weight(ctx, WT["q4_K"], od, id_, raw,
                                 mmq.MMQ_USE_GEMM | mmq.MMQ_USE_GEMM_PACKED)
    assert mmq.mmq_weight_bytes(wf) > 2.9 * mmq.mmq_weight_bytes(wp)
    a = dev_tensor(_act("packed", n, id_))
    of = torch.full((n, od), float("nan"), dtype=torch.float32, device="cuda")
    op = torch.full((n, od), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmq_gemm_q4k(ctx, wf, a, n, of)
    mmq.mmq_gemm_q4k(ctx, wp, a, n, op)
    torch.cuda.synchronize()
    assert torch.isfinite(op).all()
    assert torch.equal(of, op), f"packed {n}x{od}x{id_}: not bit-identical to the f16 tiles"
    if n * od * id_ <= 200_000_000:
        q, D, S = export_plane(ctx, a, n, id_)
        ref = gemm_ref("q4_K", q, D, S, raw, od, id_)
        assert_gemm_close(op.cpu().numpy(), ref, f"packed q4_K n={n} {od}x{id_}")
    mmq.mmq_weight_free(wf)
    mmq.mmq_weight_free(wp)


# ------------------------------------------------------------------ one-token GEMV
# one shape per register-array size (rounds of 64 blocks per row 1..12, the
# plane staged in LDS), then the re-reading form for longer rows (13 and 16
# rounds); 20000 rows make waves walk several rows with the next row in flight
GEMV_SHAPES = [(64, 256), (4100, 4096), (1000, 5120), (1024, 5120), (20000, 5120), (777, 8192),
               (9000, 10240), (130, 12288), (300, 13824), (65, 16384), (50, 18432), (33, 20480),
               (40, 22528), (70, 24576), (33, 26624), (20, 32768)]


@pytest.mark.parametrize("od,id_", GEMV_SHAPES)
def test_mmvq_parity(ctx, od, id_):
    rng = synth.rng_for("test", od, f"mmvq{id_}")
    raw = synth.q6k_weights(rng, od, id_)
    w = mmq.mmq_register_weight(ctx, 14, od, id_, raw, 2)
    ah = _act("mmvq", 1, id_)
    a = dev_tensor(ah)
    out = torch.full((od,), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmvq_q6k(ctx, w, a, out)
    q, D, S = export_plane(ctx, a, 1, id_)
    ref = gemm_ref("q6_K", q, D, S, raw, od, id_)[0]
    assert_gemm_close(out.cpu().numpy(), ref, f"mmvq {od}x{id_}")
    mmq.mmq_weight_free(w)


@pytest.mark.parametrize("od,id_", GEMV_SHAPES + [(5120, 5120), (13824, 5120)])
def test_mmvq_q4k_parity(ctx, od, id_):
    rng = synth.rng_for("test", od, f"mmvq4{id_}")
    raw = synth.q4k_weights(rng, od, id_)
    w = mmq.mmq_register_weight(ctx, 12, od, id_, raw, 2)
    ah = _act("mmvq4", 1, id_)
    a = dev_tensor(ah)
    out = torch.full((od,), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmvq_q4k(ctx, w, a, out)
    q, D, S = export_plane(ctx, a, 1, id_)
    ref = gemm_ref("q4_K", q, D, S, raw, od, id_)[0]
    assert_gemm_close(out.cpu().numpy(), ref, f"mmvq q4_K {od}x{id_}")
    mmq.mmq_weight_free(w)


@pytest.mark.parametrize("od,id_", GEMV_SHAPES + [(5120, 13824), (13824, 5120)])
def test_mmvq_q5k_parity(ctx, od, id_):
    rng = synth.rng_for("test", od, f"mmvq5{id_}")
    raw = synth.q5k_weights(rng, od, id_)
    w = mmq.mmq_register_weight(ctx, mmq.MMQ_Q5_K, od, id_, raw, 0)
    ah = _act("mmvq5", 1, id_)
    a = dev_tensor(ah)
    out = torch.full((od,), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmvq_q5k(ctx, w, a, out)
    q, D, S = export_plane(ctx, a, 1, id_)
    ref = gemm_ref("q5_K", q, D, S, raw, od, id_)[0]
    assert_gemm_close(out.cpu().numpy(), ref, f"mmvq q5_K {od}x{id_}")
    assert mmq.mmq_stats(ctx)["launches_mmvq_q5k"] >= 1
    mmq.mmq_weight_free(w)


# the f32-activation q6_K GEMV: register-sized rows, ragged row counts, the
# widest staged activation (16384) and the decode shapes below the gate
GEMV_F32_SHAPES = [(1, 256), (64, 256), (37, 1024), (512, 3584), (1000, 5120), (1024, 5120),
                   (3, 16384), (4100, 4096), (20000, 768)]


def _assert_f32_gemv_close(got, raw, od, id_, x, what):
    ref = oracle.gemv_f32("q6_K", raw, od, id_, x)
    scale = np.abs(oracle.dequant("q6_K", raw, od, id_)) @ np.abs(x.astype(np.float64))
    err = np.abs(got.astype(np.float64) - ref)
    # f32 products and sums of exact weights: well inside 2^-14 of the absolute sum
    assert np.all(err <= 2.0 ** -14 * scale + 1e-30), (what, float((err / (scale + 1e-30)).max()))
    assert_gemm_close(got, GemmRef(ref.astype(np.float32), scale, id_ // 256), what)


@pytest.mark.parametrize("od,id_", GEMV_F32_SHAPES)
def test_gemv_f32_parity(ctx, od, id_):
    raw = synth.q6k_weights(synth.rng_for("test", od, f"gemvf32{id_}"), od, id_)
    w = mmq.mmq_register_weight(ctx, mmq.MMQ_Q6_K, od, id_, raw, mmq.MMQ_USE_GEMV)
    xh = _act("gemvf32", 1, id_)[0]
    x = dev_tensor(xh)
    out = torch.full((od,), float("nan"), dtype=torch.float32, device="cuda")
    st0 = mmq.mmq_stats(ctx)
    mmq.mmq_gemv_q6k_f32(ctx, w, x, out)
    st1 = mmq.mmq_stats(ctx)
    assert st1["launches_gemv_f32"] - st0["launches_gemv_f32"] == 1
    assert st1["launches_quant_f32"] == st0["launches_quant_f32"]     # nothing quantised
    _assert_f32_gemv_close(out.cpu().numpy(), raw, od, id_, xh, f"gemv f32 {od}x{id_}")
    mmq.mmq_weight_free(w)


def test_decode_q6k_routes_bit_identically(ctx):
    """The routed decode arm returns exactly what the path it takes returns:
    the f32 GEMV below the gate, the quantised GEMV above it or when the
    activation already has a plane."""
    for od, id_ in ((512, 3584), (1024, 5120), (8192, 3584)):
        raw = synth.q6k_weights(synth.rng_for("test", od, f"route{id_}"), od, id_)
        w = mmq.mmq_register_weight(ctx, mmq.MMQ_Q6_K, od, id_, raw, mmq.MMQ_USE_GEMV)
        xh = _act("route", 1, id_)[0]
        x = dev_tensor(xh)
        routed = torch.empty((od,), dtype=torch.float32, device="cuda")
        direct = torch.empty_like(routed)
        mmq.mmq_cache_clear(ctx)
        mmq.mmq_decode_q6k(ctx, w, x, routed)
        small = od * id_ < mmq.MMQ_DECODE_F32_GATE
        assert small == (od != 8192)
        if small:
            mmq.mmq_gemv_q6k_f32(ctx, w, x, direct)
        else:
            mmq.mmvq_q6k(ctx, w, x, direct)
        torch.cuda.synchronize()
        assert torch.equal(routed, direct), (od, id_)
        if small:
            _assert_f32_gemv_close(routed.cpu().numpy(), raw, od, id_, xh, "routed f32")
            # with a plane recorded for x, the same call takes the quantised GEMV
            mmq.mmq_quant_f32(ctx, x, 1, id_)
            mmq.mmq_decode_q6k(ctx, w, x, routed)
            mmq.mmvq_q6k(ctx, w, x, direct)
            torch.cuda.synchronize()
            assert torch.equal(routed, direct)
        mmq.mmq_cache_clear(ctx)
        mmq.mmq_weight_free(w)


def test_mmvq_q5k_extreme_codes(ctx):
    """Every code at 31 (all fifth bits set) and at 0, with sub-scales and mins
    at 63: the fifth bit carries weight 16 in every nibble group."""
    od, id_ = 96, 1024
    raw = synth.q5k_weights(synth.rng_for("test", od, "mmvq5x"), od, id_).reshape(od, -1, 176)
    raw[:, :, 4:16] = 0xFF                      # every 6-bit scale and min = 63
    raw[: od // 2, :, 16:176] = 0xFF            # rows 0..47: every code 31
    raw[od // 2:, :, 16:176] = 0x00             # rows 48..95: every code 0
    raw = np.ascontiguousarray(raw.reshape(od, -1))
    w = mmq.mmq_register_weight(ctx, mmq.MMQ_Q5_K, od, id_, raw, 0)
    ah = _act("mmvq5x", 1, id_)
    a = dev_tensor(ah)
    out = torch.full((od,), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmvq_q5k(ctx, w, a, out)
    q, D, S = export_plane(ctx, a, 1, id_)
    ref = gemm_ref("q5_K", q, D, S, raw, od, id_)[0]
    assert_gemm_close(out.cpu().numpy(), ref, "mmvq q5_K extreme codes")
    mmq.mmq_weight_free(w)


@pytest.mark.parametrize("wtype", ["q4_K", "q6_K"])
@pytest.mark.parametrize("n", [1, 3])
def test_gemv_degenerate_activation_rows(ctx, wtype, n):
    """The one-token GEMV (n = 1) and the few-token GEMV (n = 3) on rows with
    zero blocks, a block scaled by 1e20 and one by 1e-20, and (n = 3) an
    all-zero row: outputs finite and within the element-wise bar."""
    od, id_ = 300, 5120
    y = synth.activations(synth.rng_for("test", n, f"gvdegen{wtype}"), n, id_)
    y[0, :1024] = 0.0
    y[0, 1024:1056] *= np.float32(1e20)
    y[0, 2048:2080] *= np.float32(1e-20)
    if n > 1:
        y[1] = 0.0
    y = np.ascontiguousarray(y, np.float32)
    raw = synth.weights(wtype, synth.rng_for("test", od, f"gvdegenw{wtype}"), od, id_)
    w = mmq.mmq_register_weight(ctx, WT[wtype], od, id_, raw, mmq.MMQ_USE_GEMM | mmq.MMQ_USE_GEMV)
    a = dev_tensor(y)
    out = torch.full((n, od), float("nan"), dtype=torch.float32, device="cuda")
    before = mmq.mmq_stats(ctx)["small_n_gemv"]
    (mmq.mmq_gemm_q4k if wtype == "q4_K" else mmq.mmq_gemm_q6k)(ctx, w, a, n, out)
    torch.cuda.synchronize()
    assert mmq.mmq_stats(ctx)["small_n_gemv"] == before + 1   # the GEMV path ran
    q, D, S = export_plane(ctx, a, n, id_)
    assert_plane_equal((q, D, S), oracle.quantize(y), "degenerate rows plane")
    got = out.cpu().numpy()
    ref = gemm_ref(wtype, q, D, S, raw, od, id_)
    assert np.isfinite(got).all()
    assert_gemm_close(got, ref, f"GEMV degenerate rows {wtype} n={n}")
    if n > 1:
        assert not got[1].any()
    mmq.mmq_weight_free(w)


def test_decode_ffn_chain_q4k_gate_up_q6k_down(ctx):
    """14B decode FFN at one token: RMSNorm(5120) -> plane shared by gate and up
    (q4_K GEMV, two hits) -> SwiGLU(13824) of their outputs -> plane -> down
    (q6_K GEMV, one hit).  Each GEMV is checked on the plane it consumed."""
    c = mmq.mmq_create(0, 0)
    try:
        xh = synth.activations(synth.rng_for("decode14b", 1, "x"), 1, 5120)
        wn = synth.rms_weight(synth.rng_for("decode14b", 1, "norm"), 5120)
        shapes = {"gate": ("q4_K", 13824, 5120), "up": ("q4_K", 13824, 5120),
                  "down": ("q6_K", 5120, 13824)}
        raws, ws = {}, {}
        for k, (wt, od, id_) in shapes.items():
            raws[k] = synth.weights(wt, synth.rng_for("decode14b", 1, k), od, id_)
            ws[k] = mmq.mmq_register_weight(c, WT[wt], od, id_, raws[k], mmq.MMQ_USE_GEMV)
        y = torch.empty((1, 5120), dtype=torch.float32, device="cuda")
        ysw = torch.empty((1, 13824), dtype=torch.float32, device="cuda")
        outs = {k: torch.full((od,), float("nan"), dtype=torch.float32, device="cuda")
                for k, (_, od, _) in shapes.items()}
        mmq.mmq_quant_rms(c, dev_tensor(xh), dev_tensor(wn), y, 1, 5120, EPS, 0)
        mmq.mmvq_q4k(c, ws["gate"], y, outs["gate"])
        mmq.mmvq_q4k(c, ws["up"], y, outs["up"])
        mmq.mmq_quant_swiglu(c, outs["gate"].view(1, -1), outs["up"].view(1, -1), ysw, 1, 13824, 0)
        mmq.mmvq_q6k(c, ws["down"], ysw, outs["down"])
        st = mmq.mmq_stats(c)
        assert st["cache_hits"] == 3 and st["cache_misses"] == 0 and st["launches_quant_f32"] == 0
        assert st["launches_mmvq_q4k"] == 2 and st["launches_mmvq_q6k"] == 1
        p1 = export_plane(c, y, 1, 5120)
        p2 = export_plane(c, ysw, 1, 13824)
        assert_fused_close(p1, oracle.quantize(oracle.rmsnorm(xh, wn, EPS)), what="decode rms")
        g, u = outs["gate"].cpu().numpy(), outs["up"].cpu().numpy()
        for k in ("gate", "up"):
            ref = gemm_ref("q4_K", *p1, raws[k], 13824, 5120)[0]
            assert_gemm_close(outs[k].cpu().numpy(), ref, k)
        # the SwiGLU plane is the fused quantisation of the GPU's own gate/up outputs
        assert_fused_close(p2, oracle.quantize(oracle.swiglu(g[None], u[None])), what="decode swiglu")
        ref = gemm_ref("q6_K", *p2, raws["down"], 5120, 13824)[0]
        assert_gemm_close(outs["down"].cpu().numpy(), ref, "down")
        for wt in ws.values():
            mmq.mmq_weight_free(wt)
    finally:
        mmq.mmq_destroy(c)


def test_mmvq_decode_chain_full_size(ctx):
    """14B decode: rms(5120) plane shared by attn_v and lm_head (hits), SwiGLU(13824)
    plane feeding ffn_down; lm_head checked on sampled rows."""
    c = mmq.mmq_create(0, 0)
    try:
        rng = synth.rng_for("decode14b", 0, "x")
        xh = synth.activations(rng, 1, 5120)
        wn = synth.rms_weight(synth.rng_for("decode14b", 0, "norm"), 5120)
        gh = synth.activations(synth.rng_for("decode14b", 0, "gate"), 1, 13824)
        uh = synth.activations(synth.rng_for("decode14b", 0, "up"), 1, 13824)
        shapes = {"attn_v": (1024, 5120), "lm_head": (152064, 5120), "ffn_down": (5120, 13824)}
        raws, ws = {}, {}
        for k, (od, id_) in shapes.items():
            raws[k] = synth.q6k_weights(synth.rng_for("decode14b", 0, k), od, id_)
            ws[k] = mmq.mmq_register_weight(c, 14, od, id_, raws[k], 2)
        y = torch.empty((1, 5120), dtype=torch.float32, device="cuda")
        y2 = torch.empty((1, 13824), dtype=torch.float32, device="cuda")
        outs = {k: torch.empty((od,), dtype=torch.float32, device="cuda") for k, (od, _) in shapes.items()}
        mmq.mmq_quant_rms(c, dev_tensor(xh), dev_tensor(wn), y, 1, 5120, EPS, 0)
        mmq.mmvq_q6k(c, ws["attn_v"], y, outs["attn_v"])
        mmq.mmvq_q6k(c, ws["lm_head"], y, outs["lm_head"])
        mmq.mmq_quant_swiglu(c, dev_tensor(gh), dev_tensor(uh), y2, 1, 13824, 0)
        mmq.mmvq_q6k(c, ws["ffn_down"], y2, outs["ffn_down"])
        st = mmq.mmq_stats(c)
        assert st["cache_hits"] == 3 and st["cache_misses"] == 0 and st["launches_quant_f32"] == 0
        p1 = export_plane(c, y, 1, 5120)
        p2 = export_plane(c, y2, 1, 13824)
        assert_fused_close(p1, oracle.quantize(oracle.rmsnorm(xh, wn, EPS)), what="decode rms")
        for k, (od, id_) in shapes.items():
            q, D, S = p1 if id_ == 5120 else p2
            rows = None if od <= 8192 else np.unique(np.concatenate(
                [[0, od - 1], np.random.default_rng(5).integers(0, od, 2000)]))
            ref = gemm_ref("q6_K", q, D, S, raws[k], od, id_, outs=rows)[0]
            got = outs[k].cpu().numpy()
            assert_gemm_close(got if rows is None else got[rows], ref, k)
        for wt in ws.values():
            mmq.mmq_weight_free(wt)
    finally:
        mmq.mmq_destroy(c)


# ------------------------------------------------------------------ cache semantics on the device
def test_attention_projection_cache_counts():
    """The 7B attention projections at 3314 tokens: the rms plane is shared by
    q, k, v (three hits); o misses and quantises its input once; outputs match
    the oracle on the shared plane (sampled tokens x outputs)."""
    c = mmq.mmq_create(0, 0)
    try:
        n, d = 3314, 3584
        xh = synth.activations(synth.rng_for("attn", 0, "x"), n, d)
        wn = synth.rms_weight(synth.rng_for("attn", 0, "norm"), d)
        ah = synth.activations(synth.rng_for("attn", 0, "attn_out"), n, d)
        specs = {"q": ("q4_K", 3584), "k": ("q4_K", 512), "v": ("q6_K", 512), "o": ("q4_K", 3584)}
        raws = {k: synth.weights(t, synth.rng_for("attn", 0, k), od, d) for k, (t, od) in specs.items()}
        ws = {k: mmq.mmq_register_weight(c, WT[t], od, d, raws[k], 1) for k, (t, od) in specs.items()}
        y = torch.empty((n, d), dtype=torch.float32, device="cuda")
        a = dev_tensor(ah)
        outs = {k: torch.empty((n, od), dtype=torch.float32, device="cuda") for k, (t, od) in specs.items()}
        mmq.mmq_quant_rms(c, dev_tensor(xh), dev_tensor(wn), y, n, d, EPS, 0)
        for k in ("q", "k", "v"):
            fn = mmq.mmq_gemm_q4k if specs[k][0] == "q4_K" else mmq.mmq_gemm_q6k
            fn(c, ws[k], y, n, outs[k])
        mmq.mmq_gemm_q4k(c, ws["o"], a, n, outs["o"])
        st = mmq.mmq_stats(c)
        assert (st["cache_hits"], st["cache_misses"], st["launches_quant_rms"],
                st["launches_quant_f32"]) == (3, 1, 1, 1)
        py = export_plane(c, y, n, d)
        pa = export_plane(c, a, n, d)
        rng = np.random.default_rng(3)
        tok = np.unique(np.concatenate([[0, 127, 128, 3199, 3200, n - 1], rng.integers(0, n, 14)]))
        for k, (t, od) in specs.items():
            q, D, S = pa if k == "o" else py
            cols = np.unique(np.concatenate([[0, 127, 128, od - 1], rng.integers(0, od, 200)]))
            ref = gemm_ref(t, q, D, S, raws[k], od, d, tok=tok, outs=cols)
            assert_gemm_close(outs[k].cpu().numpy()[np.ix_(tok, cols)], ref, k)
        # the o input plane is exactly the oracle's quantisation of it
        assert_plane_equal(pa, oracle.quantize(ah), "o input")
        for wt in ws.values():
            mmq.mmq_weight_free(wt)
    finally:
        mmq.mmq_destroy(c)


def test_dead_write_refusal_launches_nothing():
    c = mmq.mmq_create(0, 0)
    try:
        n, d = 40, 512
        raw = synth.q4k_weights(synth.rng_for("dead", 0, "w"), 128, d)
        w = mmq.mmq_register_weight(c, 12, 128, d, raw, 1)
        x = dev_tensor(synth.activations(synth.rng_for("dead", 0, "x"), n, d))
        wn = dev_tensor(synth.rms_weight(synth.rng_for("dead", 0, "n"), d))
        y = torch.empty((n, d), dtype=torch.float32, device="cuda")
        out = torch.empty((n, 128), dtype=torch.float32, device="cuda")
        mmq.mmq_quant_rms(c, x, wn, y, n, d, EPS, 0)
        before = mmq.mmq_stats(c)
        with pytest.raises(mmq.MmqError) as e1:
            mmq.mmq_quant_f32(c, y, n, d)
        with pytest.raises(mmq.MmqError) as e2:
            mmq.mmq_gemm_q4k(c, w, y, n - 1, out)      # different n: a miss on a dead buffer
        assert e1.value.status == mmq.MMQ_E_DEAD_WRITE == e2.value.status
        after = mmq.mmq_stats(c)
        assert after["cache_refusals"] == before["cache_refusals"] + 2
        for k in ("launches_quant_f32", "launches_gemm_q4k", "launches_quant_rms"):
            assert after[k] == before[k]
        mmq.mmq_gemm_q4k(c, w, y, n, out)             # the recorded plane still serves
        mmq.mmq_cache_clear(c)                        # window boundary: y is no longer dead
        y.zero_()
        mmq.mmq_quant_f32(c, y, n, d)
        mmq.mmq_weight_free(w)
    finally:
        mmq.mmq_destroy(c)


# ------------------------------------------------------------------ degradation ladder on the device
def test_degraded_skip_write_writes_y_and_the_same_plane():
    """After a foreign consumer is declared, write_y=0 writes y and records a
    live plane that is byte-identical to the write_y=1 plane."""
    n, d = 37, 3584
    xh = synth.activations(synth.rng_for("ladder", n, "x"), n, d)
    wn = synth.rms_weight(synth.rng_for("ladder", n, "w"), d)
    ref_c = mmq.mmq_create(0, 0)
    deg_c = mmq.mmq_create(0, 0)
    try:
        x, w = dev_tensor(xh), dev_tensor(wn)
        y1 = torch.full((n, d), float("nan"), dtype=torch.float32, device="cuda")
        y0 = torch.full((n, d), float("nan"), dtype=torch.float32, device="cuda")
        mmq.mmq_quant_rms(ref_c, x, w, y1, n, d, EPS, 1)
        mmq.mmq_register_foreign_consumer(deg_c, mmq.MMQ_FOREIGN_QUANT)
        mmq.mmq_quant_rms(deg_c, x, w, y0, n, d, EPS, 0)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)
        for a, b in zip(export_plane(deg_c, y0, n, d), export_plane(ref_c, y1, n, d)):
            assert np.array_equal(a, b)
        assert mmq.mmq_stats(deg_c)["degraded_writes"] == 1
        mmq.mmq_quant_f32(deg_c, y0, n, d)      # live: re-quantising is allowed
    finally:
        mmq.mmq_destroy(ref_c)
        mmq.mmq_destroy(deg_c)


@pytest.mark.parametrize("kind", ["rms", "swiglu"])
def test_auto_without_plane_memory_writes_y_only(kind):
    """MMQ_WRITE_AUTO with no plane memory allowed: the unfused tier writes y
    (checked against the oracle's f32 producer) and records no plane."""
    n, d = 40, 2560
    c = mmq.mmq_create(0, 0)
    try:
        mmq.mmq_set_scratch_cap(c, 0)
        y = torch.full((n, d), float("nan"), dtype=torch.float32, device="cuda")
        if kind == "rms":
            xh = synth.activations(synth.rng_for("unfused", n, "x"), n, d)
            wn = synth.rms_weight(synth.rng_for("unfused", n, "w"), d)
            mmq.mmq_quant_rms(c, dev_tensor(xh), dev_tensor(wn), y, n, d, EPS, mmq.MMQ_WRITE_AUTO)
            ref = oracle.rmsnorm(xh, wn, EPS)
        else:
            gh = synth.activations(synth.rng_for("unfused", n, "g"), n, d)
            uh = synth.activations(synth.rng_for("unfused", n, "u"), n, d)
            mmq.mmq_quant_swiglu(c, dev_tensor(gh), dev_tensor(uh), y, n, d, mmq.MMQ_WRITE_AUTO)
            ref = oracle.swiglu(gh, uh)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        # same expressions as the oracle; only the f64 sum order (rms) or the
        # device expf (swiglu) may move a value by a few ulp
        np.testing.assert_allclose(got, ref, rtol=4e-7, atol=1e-30)
        st = mmq.mmq_stats(c)
        assert st["unfused_fallbacks"] == 1 and st["cache_entries"] == 0 and st["plane_bytes"] == 0
    finally:
        mmq.mmq_destroy(c)


def test_side_stream_matches_default_stream(ctx):
    """Every launch goes on the caller's stream: a producer -> matmul chain
    (with a K split and the GEMV path) run on a side stream, with its inputs
    written on that stream just before, equals the same chain on the default
    stream bit for bit."""
    n, d, od = 70, 1024, 512
    xh = synth.activations(synth.rng_for("test", n, "side_x"), n, d)
    wn = synth.rms_weight(synth.rng_for("test", n, "side_w"), d)
    raw4 = synth.weights("q4_K", synth.rng_for("test", od, "side4"), od, d)
    raw6 = synth.weights("q6_K", synth.rng_for("test", od, "side6"), od, d)
    w4 = mmq.mmq_register_weight(ctx, WT["q4_K"], od, d, raw4, mmq.MMQ_USE_GEMM | mmq.MMQ_USE_GEMV)
    w6 = mmq.mmq_register_weight(ctx, WT["q6_K"], od, d, raw6, mmq.MMQ_USE_GEMM | mmq.MMQ_USE_GEMV)
    xs = torch.from_numpy(xh).cuda()
    wt = torch.from_numpy(wn).cuda()

    def chain(x):
        y = torch.empty((n, d), dtype=torch.float32, device="cuda")
        o4 = torch.empty((n, od), dtype=torch.float32, device="cuda")
        o6 = torch.empty((n, od), dtype=torch.float32, device="cuda")
        o1 = torch.empty((1, od), dtype=torch.float32, device="cuda")
        mmq.mmq_quant_rms(ctx, x, wt, y, n, d, 1e-6, 0)
        mmq.mmq_gemm_q4k(ctx, w4, y, n, o4)
        mmq.mmq_gemm_q6k(ctx, w6, y, n, o6)
        mmq.mmq_gemm_q6k(ctx, w6, x[:1], 1, o1)       # one token: the GEMV path
        return o4, o6, o1

    ref = [t.clone() for t in chain(xs)]
    torch.cuda.synchronize()
    mmq.mmq_cache_clear(ctx)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        x2 = torch.empty_like(xs)
        x2.copy_(xs)                                   # written on the side stream
        got = chain(x2)
    side.synchronize()
    mmq.mmq_cache_clear(ctx)
    for r, g_ in zip(ref, got):
        assert torch.equal(r, g_)
    mmq.mmq_weight_free(w4)
    mmq.mmq_weight_free(w6)
