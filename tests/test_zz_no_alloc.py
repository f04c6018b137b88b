"""The allocation-free one-token q6_K GEMV (mmvq_q6k_noalloc) through the C ABI.

Two calls in a row, the second with a smaller input, then the same inputs
through mmvq_q6k (the entry point it is a variant of): the outputs are equal
bit for bit (the same quantise and GEMV kernels on the same plane bytes) and
within the matmul bar of the oracle on the exported plane.  The calls
allocate nothing (the context's plane bytes do not move) and record nothing;
a recorded plane is served on a hit; columns beyond the static plane are
refused before any launch.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_rmsnorm_amd as mmq
import synth
from tests.gpu_util import assert_gemm_close, assert_plane_equal, dev_tensor, export_plane, gemm_ref

pytestmark = pytest.mark.gpu


def test_noalloc_gemv_matches_mmvq_q6k():
    ctx = mmq.mmq_create(0, 0)
    ws = []
    try:
        cases = []
        for step, (od, id_) in enumerate([(1024, 5120), (300, 2048)]):   # the second is smaller
            raw = synth.q6k_weights(synth.rng_for("noalloc", step, "w"), od, id_)
            w = mmq.mmq_register_weight(ctx, mmq.MMQ_Q6_K, od, id_, raw, mmq.MMQ_USE_GEMV)
            ws.append(w)
            xh = synth.activations(synth.rng_for("noalloc", step, "x"), 1, id_)
            cases.append((od, id_, raw, w, xh, dev_tensor(xh)))
        torch.cuda.synchronize()
        before = mmq.mmq_stats(ctx)
        got = []
        for od, id_, raw, w, xh, x in cases:                              # two calls in a row
            out = torch.full((od,), float("nan"), dtype=torch.float32, device="cuda")
            print(f"mmvq_q6k_noalloc {od}x{id_}", flush=True)
            mmq.mmvq_q6k_noalloc(ctx, w, x, out)
            got.append(out)
        torch.cuda.synchronize()
        after = mmq.mmq_stats(ctx)
        assert after["plane_bytes"] == before["plane_bytes"] == 0      # nothing allocated
        assert after["cache_entries"] == before["cache_entries"]        # nothing recorded
        assert after["cache_misses"] - before["cache_misses"] == 2
        for (od, id_, raw, w, xh, x), out in zip(cases, got):
            ref_out = torch.full((od,), float("nan"), dtype=torch.float32, device="cuda")
            mmq.mmvq_q6k(ctx, w, x, ref_out)                              # allocates and records
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out), f"{od}x{id_}"
            q, D, S = export_plane(ctx, x, 1, id_)
            assert_plane_equal((q, D, S), oracle.quantize(xh), f"plane {od}x{id_}")
            assert_gemm_close(out.cpu().numpy(), gemm_ref("q6_K", q, D, S, raw, od, id_)[0],
                              f"noalloc {od}x{id_}")
            # a hit: the recorded plane serves, and the output is the same again
            again = torch.full((od,), float("nan"), dtype=torch.float32, device="cuda")
            h0 = mmq.mmq_stats(ctx)["cache_hits"]
            mmq.mmvq_q6k_noalloc(ctx, w, x, again)
            torch.cuda.synchronize()
            assert mmq.mmq_stats(ctx)["cache_hits"] == h0 + 1
            assert torch.equal(again, out)
        # beyond the static plane: refused before any launch
        wide_cols = mmq.MMQ_NOALLOC_MAX_COLS + 256
        wide = mmq.mmq_register_weight(ctx, mmq.MMQ_Q6_K, 4, wide_cols,
                                       synth.q6k_weights(synth.rng_for("noalloc", 9, "w"), 4, wide_cols),
                                       mmq.MMQ_USE_GEMV)
        ws.append(wide)
        xw = torch.zeros(wide_cols, dtype=torch.float32, device="cuda")
        ow = torch.full((4,), 7.0, dtype=torch.float32, device="cuda")
        st0 = mmq.mmq_stats(ctx)
        with pytest.raises(mmq.MmqError) as e:
            mmq.mmvq_q6k_noalloc(ctx, wide, xw, ow)
        assert e.value.status == mmq.MMQ_E_SHAPE
        torch.cuda.synchronize()
        assert mmq.mmq_stats(ctx) == st0 and torch.all(ow == 7.0)
    finally:
        for w in ws:
            mmq.mmq_weight_free(w)
        mmq.mmq_destroy(ctx)
