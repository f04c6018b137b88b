"""HIP-graph capture of the prefill chain through the C ABI.

The chain of two layers (RMSNorm -> plane -> q, k, v; standalone quantise ->
o; RMSNorm -> plane -> gate, up; SwiGLU -> plane -> down) is captured once and
replayed several times.  Between replays the inputs are rewritten in place and
the same chain is run eagerly; every replay must equal the eager run bit for
bit (same kernels, same inputs), and the last replay's final layer is checked
against the CPU oracle: the o projection on the oracle's own quantisation of
its input, every matmul on the exported plane, and the SwiGLU plane against
the oracle's SwiGLU of the replayed gate/up outputs.  The chain runs once with
the q4_K weights on f16 tiles and once on packed 4-bit tiles.  The launch
census of the capture comes from mmq_stats.  Capture rules tested: nothing is allocated
during a capture (a plane that would need a bigger slot is refused before
anything is recorded).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_matmul_rmsnorm_amd as mmq
import synth
from tests.gpu_util import assert_fused_close, assert_gemm_close, export_plane, gemm_ref

pytestmark = pytest.mark.gpu

N, HID, KV, FFN, LAYERS = 70, 512, 256, 1024, 2
GEMMS = [("q", "q4_K", HID, HID), ("k", "q4_K", KV, HID), ("v", "q6_K", KV, HID),
         ("o", "q4_K", HID, HID), ("gate", "q4_K", FFN, HID), ("up", "q4_K", FFN, HID),
         ("down", "q6_K", HID, FFN)]


class Chain:
    def __init__(self, mmq, packed=False):
        self.m = mmq
        self.ctx = mmq.mmq_create(0, 0)
        dev = "cuda"
        self.layers = []
        for l in range(LAYERS):
            L = {}
            for name, wt, od, id_ in GEMMS:
                raw = synth.weights(wt, synth.rng_for("graph", l, name), od, id_)
                code = mmq.MMQ_Q4_K if wt == "q4_K" else mmq.MMQ_Q6_K
                uses = mmq.MMQ_USE_GEMM | (mmq.MMQ_USE_GEMM_PACKED if packed and wt == "q4_K" else 0)
                L[name] = mmq.mmq_register_weight(self.ctx, code, od, id_, raw, uses)
            for t in ("x_attn", "attn_out", "x_ffn"):
                L[t] = torch.empty((N, HID), dtype=torch.float32, device=dev)
            for t in ("norm_attn", "norm_ffn"):
                L[t] = torch.from_numpy(synth.rms_weight(synth.rng_for("graph", l, t), HID)).to(dev)
            self.layers.append(L)
        e = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
        self.y_attn, self.y_ffn, self.y_sw = e(N, HID), e(N, HID), e(N, FFN)
        self.out = [{name: e(N, od) for name, _, od, _ in GEMMS} for _ in range(LAYERS)]

    def set_inputs(self, seed):
        self.host = []
        for l, L in enumerate(self.layers):
            h = {}
            for t in ("x_attn", "attn_out", "x_ffn"):
                h[t] = synth.activations(synth.rng_for(f"graph{seed}", l, t), N, HID)
                L[t].copy_(torch.from_numpy(h[t]))
            self.host.append(h)
        torch.cuda.synchronize()

    def step(self):
        m, c = self.m, self.ctx
        for l, L in enumerate(self.layers):
            o = self.out[l]
            m.mmq_quant_rms(c, L["x_attn"], L["norm_attn"], self.y_attn, N, HID, 1e-6, 0)
            m.mmq_gemm_q4k(c, L["q"], self.y_attn, N, o["q"])
            m.mmq_gemm_q4k(c, L["k"], self.y_attn, N, o["k"])
            m.mmq_gemm_q6k(c, L["v"], self.y_attn, N, o["v"])
            m.mmq_quant_f32(c, L["attn_out"], N, HID)
            m.mmq_gemm_q4k(c, L["o"], L["attn_out"], N, o["o"])
            m.mmq_quant_rms(c, L["x_ffn"], L["norm_ffn"], self.y_ffn, N, HID, 1e-6, 0)
            m.mmq_gemm_q4k(c, L["gate"], self.y_ffn, N, o["gate"])
            m.mmq_gemm_q4k(c, L["up"], self.y_ffn, N, o["up"])
            m.mmq_quant_swiglu(c, o["gate"], o["up"], self.y_sw, N, FFN, 0)
            m.mmq_gemm_q6k(c, L["down"], self.y_sw, N, o["down"])

    def outputs(self):
        return [{k: v.clone() for k, v in o.items()} for o in self.out]

    def close(self):
        for L in self.layers:
            for name, _, _, _ in GEMMS:
                self.m.mmq_weight_free(L[name])
        self.m.mmq_destroy(self.ctx)


@pytest.mark.parametrize("packed", [False, True], ids=["f16_tiles", "packed_q4k_tiles"])
def test_chain_graph_replays_equal_eager(packed):
    ch = Chain(mmq, packed)
    try:
        ch.set_inputs(0)
        ch.step()                      # eager: sizes every plane slot
        torch.cuda.synchronize()
        mmq.mmq_cache_clear(ch.ctx)
        st0 = mmq.mmq_stats(ch.ctx)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ch.step()
        st1 = mmq.mmq_stats(ch.ctx)
        mmq.mmq_cache_clear(ch.ctx)
        census = {k: st1[k] - st0[k] for k in st1 if k.startswith("launches_")}
        expect = {"launches_quant_rms": 2 * LAYERS, "launches_quant_swiglu": LAYERS,
                  "launches_quant_f32": LAYERS, "launches_gemm_q4k": 5 * LAYERS,
                  "launches_gemm_q6k": 2 * LAYERS}
        # every other launch counter (the GEMVs) stays at zero
        assert census == {k: expect.get(k, 0) for k in census}, census
        assert st1["cache_hits"] - st0["cache_hits"] == 7 * LAYERS
        assert st1["cache_misses"] - st0["cache_misses"] == 0
        for rep in range(1, 4):
            ch.set_inputs(rep)         # eager work between replays
            g.replay()
            torch.cuda.synchronize()
            got = ch.outputs()
            ch.step()                  # eager reference on the same inputs
            torch.cuda.synchronize()
            mmq.mmq_cache_clear(ch.ctx)
            ref = ch.outputs()
            for l in range(LAYERS):
                for name in ref[l]:
                    assert torch.equal(got[l][name], ref[l][name]), (rep, l, name)
                    assert torch.isfinite(ref[l][name]).all()
            # the inputs changed, so the outputs must have too
            assert not torch.equal(got[0]["q"], ch.out[0]["q"].new_zeros(ch.out[0]["q"].shape))
        # the last replay's final layer against the oracle; its planes come from
        # one more eager run on the same inputs (the outputs were just found
        # equal bit for bit), left in the cache for the export
        ch.step()
        torch.cuda.synchronize()
        l = LAYERS - 1
        rep_out = {k: v.cpu().numpy() for k, v in got[l].items()}
        raws = {name: synth.weights(wt, synth.rng_for("graph", l, name), od, id_)
                for name, wt, od, id_ in GEMMS}
        planes = {"attn": export_plane(ch.ctx, ch.y_attn, N, HID),
                  "o": export_plane(ch.ctx, ch.layers[l]["attn_out"], N, HID),
                  "ffn": export_plane(ch.ctx, ch.y_ffn, N, HID),
                  "sw": export_plane(ch.ctx, ch.y_sw, N, FFN)}
        src = {"q": "attn", "k": "attn", "v": "attn", "o": "o", "gate": "ffn", "up": "ffn",
               "down": "sw"}
        for name, wt, od, id_ in GEMMS:
            ref = gemm_ref(wt, *planes[src[name]], raws[name], od, id_)
            assert_gemm_close(rep_out[name], ref, f"replayed {name}")
        own = oracle.quantize(ch.host[l]["attn_out"])    # no GPU plane involved
        assert_gemm_close(rep_out["o"], gemm_ref("q4_K", *own, raws["o"], HID, HID),
                          "replayed o on the oracle plane")
        assert_fused_close(planes["sw"], oracle.quantize(oracle.swiglu(rep_out["gate"], rep_out["up"])),
                           what="replayed swiglu plane")
        del g
    finally:
        ch.close()


def test_capture_refuses_slot_growth():
    ctx = mmq.mmq_create(0, 0)
    try:
        x = torch.from_numpy(synth.activations(synth.rng_for("graphgrow", 0, "x"), 8, 256)).cuda()
        big = torch.from_numpy(synth.activations(synth.rng_for("graphgrow", 0, "b"), 64, 2048)).cuda()
        mmq.mmq_quant_f32(ctx, x, 8, 256)      # one small slot exists
        torch.cuda.synchronize()
        mmq.mmq_cache_clear(ctx)
        before = mmq.mmq_stats(ctx)
        g = torch.cuda.CUDAGraph()
        err = None
        with torch.cuda.graph(g):
            mmq.mmq_quant_f32(ctx, x, 8, 256)  # fits the existing slot: recorded
            try:
                mmq.mmq_quant_f32(ctx, big, 64, 2048)   # needs a new allocation
            except mmq.MmqError as e:
                err = e
        assert err is not None and err.status == mmq.MMQ_E_ARG
        assert "capture" in str(err)
        after = mmq.mmq_stats(ctx)
        assert after["launches_quant_f32"] - before["launches_quant_f32"] == 1
        mmq.mmq_cache_clear(ctx)
        g.replay()
        torch.cuda.synchronize()
        del g
    finally:
        mmq.mmq_destroy(ctx)
