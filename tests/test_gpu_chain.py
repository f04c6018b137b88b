"""Full-size parity of the timed prefill chain against the CPU oracle.

Layers 0 and 27 of the 28-layer 7B sweep (3314 tokens, hidden 3584, ffn 18944,
seeded by their layer index exactly as in the benchmark) are built and run by
bench.py's own Chain class: the same eleven calls per layer, the same shapes,
hence the same launch plans the benchmark times.  Layer 27 runs a second time
with its q4_K weights on packed 4-bit tiles, as the benchmark's packed chain.  After each layer, checked
against the oracle:
  * the attention output's standalone plane: bit-exact (q, D, S);
  * the two RMSNorm planes and the SwiGLU plane (whose inputs are the GPU's own
    gate/up outputs): at most 1e-4 of the codes differ, by one; S = sum q of
    the GPU's plane; D within a few ulp (the skip-write producers store no y,
    so the block amax itself is not available for a bit-level D check);
  * all seven matmuls on sampled tokens x outputs, the 128-tile edges
    included, against the oracle matmul on the exported plane:
    |got - ref| <= 1e-3 * (|ref| + 1) plus the f32 rescale's rounding budget
    (tests/gpu_util.py);
  * the layer's cache census: three producer planes and one standalone
    quantise, seven hits, no miss.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import quantized_matmul_rmsnorm_amd as mmq
import synth
from tests.gpu_util import (assert_fused_close, assert_gemm_close, assert_plane_equal,
                            export_plane, gemm_ref)

pytestmark = pytest.mark.gpu

N, HID, FFN = bench.TOKENS, bench.HIDDEN, bench.FFN


def _tok(rng):
    edges = [0, 1, 31, 32, 127, 128, 129, 255, 256, 1663, 3199, 3200, 3312, N - 1]
    return np.unique(np.concatenate([edges, rng.integers(0, N, 6)]))


def _outs(rng, od):
    edges = [0, 1, 31, 32, 127, 128, od - 129, od - 128, od - 1]
    return np.unique(np.concatenate([edges, rng.integers(0, od, 120)]))


def _d_close(gpu, ref, what):
    Dg, Dr = gpu[1].astype(np.float64), ref[1].astype(np.float64)
    zero = Dr == 0
    assert np.array_equal(Dg[zero], Dr[zero]), f"{what}: zero scales differ"
    rel = np.abs(Dg[~zero] - Dr[~zero]) / Dr[~zero]
    assert rel.max(initial=0.0) < 1e-5, f"{what}: D off by {rel.max()}"


@pytest.mark.parametrize("layer,packed", [(0, False), (27, False), (27, True)],
                         ids=["layer0", "layer27", "layer27_packed_q4k_tiles"])
def test_timed_chain_layer_against_oracle(layer, packed):
    ch = bench.Chain(mmq, torch, synth, bench.LAYERS, layer_ids=[layer], packed_q4k=packed)
    try:
        L = ch.layers[0]
        before = mmq.mmq_stats(ch.ctx)
        ch.run_layer(L)
        torch.cuda.synchronize()
        after = mmq.mmq_stats(ch.ctx)
        census = {k: after[k] - before[k] for k in
                  ("launches_quant_rms", "launches_quant_swiglu", "launches_quant_f32",
                   "launches_gemm_q4k", "launches_gemm_q6k", "cache_hits", "cache_misses")}
        assert census == {"launches_quant_rms": 2, "launches_quant_swiglu": 1,
                          "launches_quant_f32": 1, "launches_gemm_q4k": 5,
                          "launches_gemm_q6k": 2, "cache_hits": 7, "cache_misses": 0}, census

        # host copies of this layer's inputs, from the same seeds
        rf = lambda t: synth.rng_for("chain7b", layer, t)
        x_attn = synth.activations(rf("x_attn"), N, HID)
        attn_out = synth.activations(rf("attn_out"), N, HID)
        x_ffn = synth.activations(rf("x_ffn"), N, HID)
        n_attn, n_ffn = synth.rms_weight(rf("norm_attn"), HID), synth.rms_weight(rf("norm_ffn"), HID)
        assert np.array_equal(L["x_attn"].cpu().numpy(), x_attn)

        planes = {"attn_norm": export_plane(ch.ctx, ch.y_attn, N, HID),
                  "attn_out": export_plane(ch.ctx, L["attn_out"], N, HID),
                  "ffn_norm": export_plane(ch.ctx, ch.y_ffn, N, HID),
                  "swiglu": export_plane(ch.ctx, ch.y_sw, N, FFN)}
        assert_plane_equal(planes["attn_out"], oracle.quantize(attn_out), f"layer {layer} o input")
        ref_attn = oracle.quantize(oracle.rmsnorm(x_attn, n_attn, synth.EPS))
        ref_ffn = oracle.quantize(oracle.rmsnorm(x_ffn, n_ffn, synth.EPS))
        gate, up = ch.out["gate"].cpu().numpy(), ch.out["up"].cpu().numpy()
        ref_sw = oracle.quantize(oracle.swiglu(gate, up))
        del gate, up
        for key, ref in (("attn_norm", ref_attn), ("ffn_norm", ref_ffn), ("swiglu", ref_sw)):
            rate = assert_fused_close(planes[key], ref, what=f"layer {layer} {key} plane")
            _d_close(planes[key], ref, f"layer {layer} {key} plane")
            print(f"layer {layer} {key}: flip rate {rate:.2e}", flush=True)

        raws = {name: synth.weights(wt, rf(name), od, id_)
                for name, wt, od, id_, _ in bench.LAYER_GEMMS}
        rng = np.random.default_rng(1000 + layer)
        for name, wt, od, id_, src in bench.LAYER_GEMMS:
            q, D, S = planes[src]
            tok, outs = _tok(rng), _outs(rng, od)
            ref = gemm_ref(wt, q, D, S, raws[name], od, id_, tok=tok, outs=outs)
            got = ch.out[name].cpu().numpy()[np.ix_(tok, outs)]
            worst = assert_gemm_close(got, ref, f"layer {layer} {name} {od}x{id_}")
            print(f"layer {layer} {name}: worst err/(|ref|+1) {worst:.2e}", flush=True)
            assert np.isfinite(ch.out[name].cpu().numpy()).all()
    finally:
        ch.close()
