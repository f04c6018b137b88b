"""Seeded random shapes through the C ABI, against the CPU oracle.

The hand-picked shapes of the other parity tests sit on the edges the kernels
were written for.  These cases draw token counts, output rows, widths and
registration uses from a fixed seed, so that routing (one-token GEMV, the
few-token band in one or two passes, the matmul with or without a K split
and a tail split) and tile edges meet in combinations nobody chose.  Every
output is compared: the matmuls on the exported plane at the matmul bar, the
producers' planes bit-exact (standalone quantise) or at the fused bar.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_rmsnorm_amd as mmq
import synth
from tests.gpu_util import (assert_fused_close, assert_gemm_close, assert_plane_equal, dev_tensor,
                            export_plane, gemm_ref)

pytestmark = pytest.mark.gpu

WT = {"q4_K": mmq.MMQ_Q4_K, "q6_K": mmq.MMQ_Q6_K}
NS = [1, 2, 3, 5, 8, 9, 12, 16, 17, 31, 33, 100, 129, 257]


def _gemm_cases(count=48, budget=400_000_000):
    """(wtype, n, od, id, registered for the GEMV too, packed q4_K tiles);
    n * od * id within the oracle's budget, a third of the cases with
    n >= 100 (several 128-token tiles and a ragged tail), every other q4_K
    case on the packed 4-bit matmul tiles."""
    rng = np.random.default_rng(20261203)
    cases = []
    while len(cases) < count:
        wtype = ("q4_K", "q6_K")[len(cases) % 2]
        n = int(rng.choice(NS)) if len(cases) % 3 else int(rng.integers(100, 420))
        od = int(rng.integers(1, 1600))
        id_ = 256 * int(rng.integers(1, 25))
        both = bool(rng.integers(0, 2))
        if n * od * id_ <= budget:
            packed = wtype == "q4_K" and (len(cases) // 2) % 2 == 1
            cases.append((wtype, n, od, id_, both, packed))
    return cases


def _producer_cases(count=24):
    rng = np.random.default_rng(31337)
    kinds = ("rms", "swiglu", "f32")
    return [(kinds[i % 3], int(rng.integers(1, 71)), 256 * int(rng.integers(1, 81)))
            for i in range(count)]


@pytest.fixture(scope="module")
def _module_ctx():
    c = mmq.mmq_create(0, 0)
    yield c
    mmq.mmq_destroy(c)


@pytest.fixture
def ctx(_module_ctx):
    mmq.mmq_cache_clear(_module_ctx)
    return _module_ctx


@pytest.mark.parametrize("wtype,n,od,id_,both,packed", _gemm_cases())
def test_random_matmul_shape(ctx, wtype, n, od, id_, both, packed):
    tag = f"rand{wtype}{n}x{od}x{id_}"
    raw = synth.weights(wtype, synth.rng_for("random", n, tag), od, id_)
    uses = (mmq.MMQ_USE_GEMM | (mmq.MMQ_USE_GEMV if both else 0) |
            (mmq.MMQ_USE_GEMM_PACKED if packed else 0))
    w = mmq.mmq_register_weight(ctx, WT[wtype], od, id_, raw, uses)
    try:
        rng = synth.rng_for("random", n, tag + "a")
        ah = synth.activations(rng, n, id_) * rng.uniform(0.1, 10.0, (n, 1)).astype(np.float32)
        ah = np.ascontiguousarray(ah, np.float32)
        a = dev_tensor(ah)
        out = torch.full((n, od), float("nan"), dtype=torch.float32, device="cuda")
        (mmq.mmq_gemm_q4k if wtype == "q4_K" else mmq.mmq_gemm_q6k)(ctx, w, a, n, out)
        torch.cuda.synchronize()
        q, D, S = export_plane(ctx, a, n, id_)
        assert_plane_equal((q, D, S), oracle.quantize(ah), f"{tag} plane")
        ref = gemm_ref(wtype, q, D, S, raw, od, id_)
        assert_gemm_close(out.cpu().numpy(), ref, f"{tag} uses={uses}")
    finally:
        mmq.mmq_weight_free(w)


@pytest.mark.parametrize("kind,n,d", _producer_cases())
def test_random_producer_shape(ctx, kind, n, d):
    rng = synth.rng_for("random", n, f"prod{kind}{d}")
    x = synth.activations(rng, n, d)
    y = torch.empty((n, d), dtype=torch.float32, device="cuda")
    if kind == "f32":
        xd = dev_tensor(x)
        mmq.mmq_quant_f32(ctx, xd, n, d)
        assert_plane_equal(export_plane(ctx, xd, n, d), oracle.quantize(x), f"f32 {n}x{d}")
        return
    if kind == "rms":
        wn = synth.rms_weight(rng, d)
        mmq.mmq_quant_rms(ctx, dev_tensor(x), dev_tensor(wn), y, n, d, synth.EPS, 1)
        y_ref = oracle.rmsnorm(x, wn, synth.EPS)
    else:
        u = synth.activations(rng, n, d)
        mmq.mmq_quant_swiglu(ctx, dev_tensor(x), dev_tensor(u), y, n, d, 1)
        y_ref = oracle.swiglu(x, u)
    torch.cuda.synchronize()
    plane = export_plane(ctx, y, n, d)
    y_gpu = y.cpu().numpy()
    assert_plane_equal(oracle.quantize(y_gpu), plane, f"{kind} {n}x{d}: oracle quantiser on the GPU's y")
    assert_fused_close(plane, oracle.quantize(y_ref), y_gpu, y_ref, f"{kind} {n}x{d}")
