"""Benchmark: the 7B prefill matmul chain (one step = all 28 layers) on one MI355X.

One step runs, for each of 28 layers at 3314 tokens (hidden 3584, ffn 18944):
  RMSNorm -> q8 plane (skip-write) -> q (q4_K 3584x3584), k (q4_K 512x3584),
  v (q6_K 512x3584), all three reading the one cached plane;
  standalone quantise of the attention output -> o (q4_K 3584x3584);
  RMSNorm -> plane (skip-write) -> gate, up (q4_K 18944x3584);
  SwiGLU(gate, up) -> plane (skip-write) -> down (q6_K 3584x18944);
then one cache clear (the execution-window boundary).  Every layer has its own
seeded synthetic weights and N(0,1) inputs, resident in HBM before timing.

Printed (one JSON line): MMQ chain TOPS (value), tok/s-equivalent, per-kernel-
class times from HIP events over the timed region, the roofline of the
dominant kernel (the q4_K matmul), the one-token q6_K GEMV bandwidth at the
14B decode shapes (weights rotated so they stream from HBM, not the 256 MB
last-level cache), and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HIDDEN, FFN, KV, TOKENS, LAYERS = 3584, 18944, 512, 3314, 28
PEAK_INT8_TOPS = 5000.0          # MI355X dense int8 MFMA
PEAK_F16_TOPS = 2500.0           # MI355X dense f16 MFMA (the instruction the matmul issues)
PEAK_HBM_GBS = 8000.0

# (name, weight type, od, id, input) per layer, in chain order
LAYER_GEMMS = [("q", "q4_K", HIDDEN, HIDDEN, "attn_norm"), ("k", "q4_K", KV, HIDDEN, "attn_norm"),
               ("v", "q6_K", KV, HIDDEN, "attn_norm"), ("o", "q4_K", HIDDEN, HIDDEN, "attn_out"),
               ("gate", "q4_K", FFN, HIDDEN, "ffn_norm"), ("up", "q4_K", FFN, HIDDEN, "ffn_norm"),
               ("down", "q6_K", HIDDEN, FFN, "swiglu")]


def chain_ops(tokens=TOKENS, layers=LAYERS):
    return 2 * tokens * layers * sum(od * id_ for _, _, od, id_, _ in LAYER_GEMMS)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--layers", type=int, default=LAYERS, help=argparse.SUPPRESS)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-packed", action="store_true",
                   help="skip the packed q4_K tiles leg (both tile forms timed per call)")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--small-n", action="store_true", help="add the small-n band sweep (us per call)")
    p.add_argument("--power", action="store_true",
                   help="add socket power and clocks (amd-smi) under the matmuls, probes and read stream")
    p.add_argument("--decode-crossover", action="store_true",
                   help="add the q6_K decode arm's path sweep over od x id (us per call)")
    p.add_argument("--f16-reference", action="store_true",
                   help="add a dense f16 GEMM of the gate shape through torch.matmul (context)")
    # one untimed device copy of this many MiB before the chain: the plain copy
    # kernel of known size that scales the HBM byte counters of a --pmc run
    p.add_argument("--copy-calibration", type=int, default=0, help=argparse.SUPPRESS)
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Chain:
    """The 7B chain on one context: per layer its registered weights, inputs
    and RMSNorm weights (seeded by the layer index), shared producer output
    buffers (the plane keys) and matmul outputs.  `layer_ids` picks which
    layers of the 28 are built (all of them for the timed step)."""

    def __init__(self, mmq, torch, synth, layers, layer_ids=None, packed_q4k=False):
        self.mmq, self.torch = mmq, torch
        self.ctx = mmq.mmq_create(0, 0)
        self.layers = []
        dev = "cuda"
        self.layer_ids = list(range(layers)) if layer_ids is None else list(layer_ids)
        for l in self.layer_ids:
            L = {}
            for name, wt, od, id_, _ in LAYER_GEMMS:
                raw = synth.weights(wt, synth.rng_for("chain7b", l, name), od, id_)
                code = mmq.MMQ_Q4_K if wt == "q4_K" else mmq.MMQ_Q6_K
                uses = mmq.MMQ_USE_GEMM | (mmq.MMQ_USE_GEMM_PACKED if packed_q4k and wt == "q4_K" else 0)
                L[name] = mmq.mmq_register_weight(self.ctx, code, od, id_, raw, uses)
                del raw
            for t in ("x_attn", "attn_out", "x_ffn"):
                L[t] = torch.from_numpy(synth.activations(synth.rng_for("chain7b", l, t), TOKENS,
                                                          HIDDEN)).to(dev)
            for t in ("norm_attn", "norm_ffn"):
                L[t] = torch.from_numpy(synth.rms_weight(synth.rng_for("chain7b", l, t), HIDDEN)).to(dev)
            self.layers.append(L)
            if len(self.layers) % 7 == 0:
                log(f"registered {len(self.layers)}/{len(self.layer_ids)} layers")
        e = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
        # producer output buffers: allocated (they are the plane keys) but never written
        self.y_attn, self.y_ffn, self.y_sw = e(TOKENS, HIDDEN), e(TOKENS, HIDDEN), e(TOKENS, FFN)
        self.out = {name: e(TOKENS, od) for name, _, od, _, _ in LAYER_GEMMS}
        self.events = None

    def _ev(self, cls):
        if self.events is None:
            return None
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record()
        self.events.setdefault(cls, []).append((a, b))
        return b

    def _run(self, cls, fn, *args):
        end = self._ev(cls)
        fn(*args)
        if end is not None:
            end.record()

    def step(self):
        for L in self.layers:
            self.run_layer(L)
        self.mmq.mmq_cache_clear(self.ctx)

    def run_layer(self, L):
        """One layer's eleven calls, in chain order, on the current stream."""
        m, c, n = self.mmq, self.ctx, TOKENS
        self._run("quant_rms", m.mmq_quant_rms, c, L["x_attn"], L["norm_attn"], self.y_attn, n,
                  HIDDEN, 1e-6, 0)
        self._run("gemm_q4k", m.mmq_gemm_q4k, c, L["q"], self.y_attn, n, self.out["q"])
        self._run("gemm_q4k", m.mmq_gemm_q4k, c, L["k"], self.y_attn, n, self.out["k"])
        self._run("gemm_q6k", m.mmq_gemm_q6k, c, L["v"], self.y_attn, n, self.out["v"])
        self._run("quant_f32", m.mmq_quant_f32, c, L["attn_out"], n, HIDDEN)
        self._run("gemm_q4k", m.mmq_gemm_q4k, c, L["o"], L["attn_out"], n, self.out["o"])
        self._run("quant_rms", m.mmq_quant_rms, c, L["x_ffn"], L["norm_ffn"], self.y_ffn, n,
                  HIDDEN, 1e-6, 0)
        self._run("gemm_q4k", m.mmq_gemm_q4k, c, L["gate"], self.y_ffn, n, self.out["gate"])
        self._run("gemm_q4k", m.mmq_gemm_q4k, c, L["up"], self.y_ffn, n, self.out["up"])
        self._run("quant_swiglu", m.mmq_quant_swiglu, c, self.out["gate"], self.out["up"],
                  self.y_sw, n, FFN, 0)
        self._run("gemm_q6k", m.mmq_gemm_q6k, c, L["down"], self.y_sw, n, self.out["down"])

    def close(self):
        for L in self.layers:
            for name, _, _, _, _ in LAYER_GEMMS:
                self.mmq.mmq_weight_free(L[name])
        self.mmq.mmq_destroy(self.ctx)

    def class_times_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) for k, v in self.events.items()}, \
               {k: len(v) for k, v in self.events.items()}


def _graph_time_us(torch, fn, reps):
    """Average time of one fn() launch: `reps` launches captured in one HIP
    graph, the graph replayed three times between HIP events (launch gaps
    inside a graph are included; host call overhead is not)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / (3 * reps)


def decode_gemv(mmq, torch, synth):
    """One-token q6_K GEMV at the 14B decode shapes, weights streamed cold
    (copies rotated so the set exceeds the 256 MB last-level cache), and the
    n = 1 producers that feed them; each timed as a captured HIP graph."""
    ctx = mmq.mmq_create(0, 0)
    shapes = {"attn_v": (1024, 5120, 64), "ffn_down": (5120, 13824, 8), "lm_head": (152064, 5120, 2)}
    res = {}
    try:
        y5 = torch.empty((1, 5120), dtype=torch.float32, device="cuda")
        y13 = torch.empty((1, 13824), dtype=torch.float32, device="cuda")
        x = torch.from_numpy(synth.activations(synth.rng_for("decode14b", 0, "x"), 1, 5120)).cuda()
        wn = torch.from_numpy(synth.rms_weight(synth.rng_for("decode14b", 0, "norm"), 5120)).cuda()
        g = torch.from_numpy(synth.activations(synth.rng_for("decode14b", 0, "gate"), 1, 13824)).cuda()
        u = torch.from_numpy(synth.activations(synth.rng_for("decode14b", 0, "up"), 1, 13824)).cuda()
        tot_b, tot_t = 0.0, 0.0
        for name, (od, id_, copies) in shapes.items():
            raw = synth.q6k_weights(synth.rng_for("decode14b", 0, name), od, id_)
            ws = [mmq.mmq_register_weight(ctx, mmq.MMQ_Q6_K, od, id_, raw, mmq.MMQ_USE_GEMV)
                  for _ in range(copies)]
            del raw
            out = torch.empty((od,), dtype=torch.float32, device="cuda")
            key = y5 if id_ == 5120 else y13
            if id_ == 5120:
                mmq.mmq_quant_rms(ctx, x, wn, y5, 1, 5120, 1e-6, 0)
            else:
                mmq.mmq_quant_swiglu(ctx, g, u, y13, 1, 13824, 0)
            mmq.mmvq_q6k(ctx, ws[0], key, out)
            torch.cuda.synchronize()
            ref = out.clone()
            reps = max(2 * copies, 32)
            t_us = _graph_time_us(torch, lambda i: mmq.mmvq_q6k(ctx, ws[i % copies], key, out), reps)
            if not torch.equal(out, ref):       # every copy holds the same weights
                raise RuntimeError(f"{name}: graph replay output differs from the eager launch")
            nbytes = od * id_ / 256 * 210 + id_ * 1.25 + od * 4
            res[name] = {"od": od, "id": id_, "us": round(t_us, 3),
                         "GB_s": round(nbytes / (t_us * 1e-6) / 1e9, 1)}
            tot_b += nbytes; tot_t += t_us
            for w in ws:
                mmq.mmq_weight_free(w)
        res["aggregate_GB_s"] = round(tot_b / (tot_t * 1e-6) / 1e9, 1)
        res["aggregate_frac_hbm"] = round(res["aggregate_GB_s"] / PEAK_HBM_GBS, 4)
        # q4_K and q5_K one-token GEMVs at the 14B shapes (ffn gate/up, attention q/output)
        arms = {"q4_K": (mmq.MMQ_Q4_K, synth.q4k_weights, mmq.mmvq_q4k, 144),
                "q5_K": (mmq.MMQ_Q5_K, synth.q5k_weights, mmq.mmvq_q5k, 176)}
        for wt, (code, gen, fn, bpb) in arms.items():
            arm = {}
            for name, (od, id_, copies) in {"ffn_gate": (13824, 5120, 8),
                                            "attn_q": (5120, 5120, 16)}.items():
                raw = gen(synth.rng_for("decode14b", 0, f"{name}/{wt}"), od, id_)
                ws = [mmq.mmq_register_weight(ctx, code, od, id_, raw, mmq.MMQ_USE_GEMV)
                      for _ in range(copies)]
                del raw
                out = torch.empty((od,), dtype=torch.float32, device="cuda")
                mmq.mmq_quant_rms(ctx, x, wn, y5, 1, 5120, 1e-6, 0)
                fn(ctx, ws[0], y5, out)
                torch.cuda.synchronize()
                ref = out.clone()
                reps = max(2 * copies, 32)
                t_us = _graph_time_us(torch, lambda i: fn(ctx, ws[i % copies], y5, out), reps)
                if not torch.equal(out, ref):
                    raise RuntimeError(f"{wt} {name}: graph replay output differs from the eager launch")
                nbytes = od * id_ / 256 * bpb + id_ * 1.25 + od * 4
                arm[name] = {"od": od, "id": id_, "us": round(t_us, 3),
                             "GB_s": round(nbytes / (t_us * 1e-6) / 1e9, 1)}
                for w in ws:
                    mmq.mmq_weight_free(w)
            res[wt] = arm
        # decode producers (rms 5120, swiglu 13824) at n = 1
        for name, fn in (("rms_5120", lambda i: mmq.mmq_quant_rms(ctx, x, wn, y5, 1, 5120, 1e-6, 0)),
                         ("swiglu_13824", lambda i: mmq.mmq_quant_swiglu(ctx, g, u, y13, 1, 13824, 0))):
            res[name] = {"us": round(_graph_time_us(torch, fn, 50), 3)}
    finally:
        mmq.mmq_cache_clear(ctx)
        mmq.mmq_destroy(ctx)
    return res


def packed_q4k(mmq, torch, synth, chain, rounds=3, reps=10):
    """Layer 0's q4_K matmuls with their weights registered a second time as
    packed 4-bit tiles (MMQ_USE_GEMM_PACKED): per-call time of both forms on
    the same recorded plane (alternating rounds, best round), whether the two
    outputs are the same bits, and the device bytes of each form.  (main()
    adds the whole chain on packed tiles under "chain".)"""
    L, c, n = chain.layers[0], chain.ctx, TOKENS
    a = L["attn_out"]
    shapes, f16_b, packed_b = {}, 0, 0
    for name, wt, od, id_, _ in LAYER_GEMMS:
        if wt != "q4_K":
            continue
        raw = synth.weights(wt, synth.rng_for("chain7b", chain.layer_ids[0], name), od, id_)
        wp = mmq.mmq_register_weight(c, mmq.MMQ_Q4_K, od, id_, raw,
                                     mmq.MMQ_USE_GEMM | mmq.MMQ_USE_GEMM_PACKED)
        del raw
        out_f = chain.out[name]
        out_p = torch.empty_like(out_f)
        mmq.mmq_gemm_q4k(c, L[name], a, n, out_f)
        mmq.mmq_gemm_q4k(c, wp, a, n, out_p)
        torch.cuda.synchronize()
        same = bool(torch.equal(out_f, out_p))
        best = {"f16": float("inf"), "packed": float("inf")}
        for _ in range(rounds):
            for form, w, o in (("f16", L[name], out_f), ("packed", wp, out_p)):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    mmq.mmq_gemm_q4k(c, w, a, n, o)
                e1.record()
                torch.cuda.synchronize()
                best[form] = min(best[form], e0.elapsed_time(e1) * 1e3 / reps)
        bf, bp = mmq.mmq_weight_bytes(L[name]), mmq.mmq_weight_bytes(wp)
        f16_b += bf
        packed_b += bp
        shapes[name] = {"od": od, "id": id_, "f16_us": round(best["f16"], 2),
                        "packed_us": round(best["packed"], 2),
                        "packed_over_f16": round(best["packed"] / best["f16"], 4),
                        "bit_identical": same,
                        "f16_bytes_per_weight": round(bf / (od * id_), 4),
                        "packed_bytes_per_weight": round(bp / (od * id_), 4)}
        mmq.mmq_weight_free(wp)
    mmq.mmq_cache_clear(c)
    mean = lambda k: sum(v[k] for v in shapes.values()) / len(shapes)
    q6_b = sum(mmq.mmq_weight_bytes(L[name]) for name, wt, _, _, _ in LAYER_GEMMS if wt == "q6_K")
    raw_b = sum(od * id_ // 256 * (144 if wt == "q4_K" else 210) for _, wt, od, id_, _ in LAYER_GEMMS)
    rec = {"shapes": shapes, "tokens": n,
           "mean_call_f16_us": round(mean("f16_us"), 2), "mean_call_packed_us": round(mean("packed_us"), 2),
           "mean_packed_over_f16": round(mean("packed_us") / mean("f16_us"), 4),
           "all_bit_identical": all(v["bit_identical"] for v in shapes.values()),
           "chain_registered_bytes_f16": len(chain.layers) * (f16_b + q6_b),
           "chain_registered_bytes_packed_q4k": len(chain.layers) * (packed_b + q6_b),
           "chain_raw_bytes": len(chain.layers) * raw_b}
    log(f"packed q4_K tiles: {rec['mean_call_packed_us']} us per call against "
        f"{rec['mean_call_f16_us']} (f16 tiles), bit-identical {rec['all_bit_identical']}; "
        f"chain weights {rec['chain_registered_bytes_packed_q4k'] / 1e9:.2f} GB against "
        f"{rec['chain_registered_bytes_f16'] / 1e9:.2f} GB (raw {rec['chain_raw_bytes'] / 1e9:.2f})")
    return rec


def packed_chain(mmq, torch, synth, args, ops):
    """The same chain with every q4_K weight registered on packed 4-bit tiles
    (q6_K as before): K steps with events only at the step boundaries, after
    the warm-up steps, and the library's registered bytes."""
    ch = Chain(mmq, torch, synth, args.layers, packed_q4k=True)
    try:
        for _ in range(args.warmup):
            ch.step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            ch.step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        wb = mmq.mmq_stats(ch.ctx)["weight_bytes"]
    finally:
        ch.close()
    log(f"chain on packed q4_K tiles: {ms:.2f} ms/step, {ops / (ms * 1e-3) / 1e12:.1f} TOPS, "
        f"{wb / 1e9:.2f} GB of registered weights")
    return {"ms_per_step": round(ms, 3), "tops": round(ops / (ms * 1e-3) / 1e12, 2),
            "registered_weight_bytes": wb}


def small_n_sweep(mmq, torch, synth):
    """The small-n band: matmul-call time for n = 1..128 tokens at the 7B/14B
    shapes, weights registered for both paths (few tokens take the GEMV path in
    one or two passes, as the library routes them; larger n the matmul tiles
    with a K split).  Each point is a captured-graph replay over rotated
    weight copies."""
    ctx = mmq.mmq_create(0, 0)
    res = {}
    try:
        for wt, od, id_ in (("q4_K", 18944, 3584), ("q4_K", 3584, 3584), ("q6_K", 3584, 18944),
                            ("q6_K", 512, 3584), ("q4_K", 13824, 5120), ("q6_K", 5120, 13824)):
            raw = synth.weights(wt, synth.rng_for("smalln", 0, wt), od, id_)
            code = mmq.MMQ_Q4_K if wt == "q4_K" else mmq.MMQ_Q6_K
            copies = max(2, int(600e6 // (od * id_ * 2)))
            ws = [mmq.mmq_register_weight(ctx, code, od, id_, raw, mmq.MMQ_USE_GEMM | mmq.MMQ_USE_GEMV)
                  for _ in range(copies)]
            fn = mmq.mmq_gemm_q4k if wt == "q4_K" else mmq.mmq_gemm_q6k
            row = {}
            for n in (1, 2, 4, 8, 16, 32, 128):
                a = torch.from_numpy(synth.activations(synth.rng_for("smalln", n, "a"), n, id_)).cuda()
                out = torch.empty((n, od), dtype=torch.float32, device="cuda")
                fn(ctx, ws[0], a, n, out)
                torch.cuda.synchronize()
                row[n] = round(_graph_time_us(torch, lambda i: fn(ctx, ws[i % copies], a, n, out),
                                              2 * copies), 2)
                mmq.mmq_cache_clear(ctx)
            res[f"{wt} {od}x{id_}"] = row
            for w in ws:
                mmq.mmq_weight_free(w)
    finally:
        mmq.mmq_destroy(ctx)
    return res


def decode_crossover_sweep(mmq, torch, synth):
    """The q6_K decode arm's two paths across od x id at one token: the
    quantised GEMV from a written activation with no plane yet (standalone
    quantise + GEMV, as the routed arm would run it), the same GEMV with the
    plane already recorded, and the f32-activation GEMV (one launch, no
    quantise).  us per call, captured-graph replays over rotated weight
    copies; the f32 gate is the smallest od*id where the quantised route is
    no slower."""
    ctx = mmq.mmq_create(0, 0)
    res = {}
    try:
        for id_ in (3584, 5120):
            x = torch.from_numpy(synth.activations(synth.rng_for("crossover", id_, "x"), 1, id_)[0]).cuda()
            for od in (256, 512, 1024, 2048, 4096, 8192, 16384):
                raw = synth.q6k_weights(synth.rng_for("crossover", od, str(id_)), od, id_)
                copies = max(2, min(128, int(400e6 // (od * id_ * 0.83))))
                ws = [mmq.mmq_register_weight(ctx, mmq.MMQ_Q6_K, od, id_, raw, mmq.MMQ_USE_GEMV)
                      for _ in range(copies)]
                out = torch.empty((od,), dtype=torch.float32, device="cuda")
                reps = 2 * copies

                def miss(i):
                    mmq.mmq_cache_clear(ctx)   # host bookkeeping only: every call quantises x
                    mmq.mmvq_q6k(ctx, ws[i % copies], x, out)

                miss(0)
                torch.cuda.synchronize()
                t_miss = _graph_time_us(torch, miss, reps)
                mmq.mmq_cache_clear(ctx)
                mmq.mmq_quant_f32(ctx, x, 1, id_)
                t_hit = _graph_time_us(torch, lambda i: mmq.mmvq_q6k(ctx, ws[i % copies], x, out), reps)
                mmq.mmq_cache_clear(ctx)
                mmq.mmq_gemv_q6k_f32(ctx, ws[0], x, out)
                torch.cuda.synchronize()
                t_f32 = _graph_time_us(torch, lambda i: mmq.mmq_gemv_q6k_f32(ctx, ws[i % copies], x, out),
                                       reps)
                res[f"{od}x{id_}"] = {"od_id": od * id_, "quantise+gemv": round(t_miss, 2),
                                      "gemv_on_plane": round(t_hit, 2), "f32_gemv": round(t_f32, 2)}
                for w in ws:
                    mmq.mmq_weight_free(w)
    finally:
        mmq.mmq_cache_clear(ctx)
        mmq.mmq_destroy(ctx)
    return res


def f16_reference(torch):
    """Context for the matmul roofline: a plain dense f16 GEMM of the gate
    shape (3314 x 3584 times 3584 x 18944, f32 accumulation inside the vendor
    library that torch.matmul calls), random operands, timed like the chain."""
    a = torch.randn((TOKENS, HIDDEN), dtype=torch.float16, device="cuda")
    b = torch.randn((HIDDEN, FFN), dtype=torch.float16, device="cuda")
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / 20
    del a, b, c
    return {"shape": f"{TOKENS}x{HIDDEN} @ {HIDDEN}x{FFN}", "us": round(us, 2),
            "TFLOP_s": round(2 * TOKENS * HIDDEN * FFN / (us * 1e-6) / 1e12, 1)}


_LAYER0 = []


def _layer0_inputs():
    """Layer 0's weights and activations of the chain, generated once."""
    if not _LAYER0:
        import synth
        raws = {name: synth.weights(wt, synth.rng_for("chain7b", 0, name), od, id_)
                for name, wt, od, id_, _ in LAYER_GEMMS}
        _LAYER0.extend([
            raws,
            synth.activations(synth.rng_for("chain7b", 0, "x_attn"), TOKENS, HIDDEN),
            synth.activations(synth.rng_for("chain7b", 0, "attn_out"), TOKENS, HIDDEN),
            synth.activations(synth.rng_for("chain7b", 0, "x_ffn"), TOKENS, HIDDEN),
            synth.rms_weight(synth.rng_for("chain7b", 0, "norm_attn"), HIDDEN),
            synth.rms_weight(synth.rng_for("chain7b", 0, "norm_ffn"), HIDDEN)])
    return _LAYER0


def _oracle_layer_sample(seconds: float):
    """The CPU oracle on layer 0 of the chain (both RMSNorm producers, the
    standalone quantise, SwiGLU and all seven matmuls) for a growing number
    of tokens until about `seconds`; returns (TOPS, tokens, seconds)."""
    import oracle
    t_used = 0.0
    tok_done = 0
    raws, x, a, h, n1, n2 = _layer0_inputs()
    chunk = 4
    while t_used < seconds and tok_done + chunk <= TOKENS:
        sl = slice(tok_done, tok_done + chunk)
        t0 = time.perf_counter()
        pa = oracle.quantize(oracle.rmsnorm(x[sl], n1, 1e-6))
        po = oracle.quantize(a[sl])
        pf = oracle.quantize(oracle.rmsnorm(h[sl], n2, 1e-6))
        outs = {}
        for name, wt, od, id_, src in LAYER_GEMMS:
            if src == "swiglu":
                continue
            q, D, S = {"attn_norm": pa, "attn_out": po, "ffn_norm": pf}[src]
            outs[name] = oracle.gemm(wt, q, D, S, raws[name], od, id_)
        ps = oracle.quantize(oracle.swiglu(outs["gate"], outs["up"]))
        oracle.gemm("q6_K", *ps, raws["down"], HIDDEN, FFN)
        t_used += time.perf_counter() - t0
        tok_done += chunk
    ops = 2 * tok_done * sum(od * id_ for _, _, od, id_, _ in LAYER_GEMMS)
    return ops / t_used / 1e12, tok_done, t_used


def _oracle_decode_full():
    """The CPU oracle on the whole 14B decode step of the GEMV leg: RMSNorm and
    SwiGLU producers at one token, then the attn_v, ffn_down and lm_head q6_K
    GEMVs in full; returns (GB/s over the GEMVs' algorithmic bytes, seconds)."""
    import oracle
    import synth
    x = synth.activations(synth.rng_for("decode14b", 0, "x"), 1, 5120)
    wn = synth.rms_weight(synth.rng_for("decode14b", 0, "norm"), 5120)
    g = synth.activations(synth.rng_for("decode14b", 0, "gate"), 1, 13824)
    u = synth.activations(synth.rng_for("decode14b", 0, "up"), 1, 13824)
    shapes = {"attn_v": (1024, 5120), "ffn_down": (5120, 13824), "lm_head": (152064, 5120)}
    raws = {k: synth.q6k_weights(synth.rng_for("decode14b", 0, k), od, id_) for k, (od, id_) in shapes.items()}
    t0 = time.perf_counter()
    p5 = oracle.quantize(oracle.rmsnorm(x, wn, 1e-6))
    p13 = oracle.quantize(oracle.swiglu(g, u))
    byts = 0.0
    for k, (od, id_) in shapes.items():
        oracle.gemm("q6_K", *(p5 if id_ == 5120 else p13), raws[k], od, id_)
        byts += od * id_ / 256 * 210 + id_ * 1.25 + od * 4
    dt = time.perf_counter() - t0
    return byts / dt / 1e9, dt


def _oracle_tiny_full():
    """The CPU oracle on the tiny workload in full: RMSNorm of 32 x 256, its
    plane, and the q4_K 512 x 256 matmul; returns (TOPS, seconds)."""
    import oracle
    import synth
    x = synth.activations(synth.rng_for("tiny", 0, "x"), 32, 256)
    wn = synth.rms_weight(synth.rng_for("tiny", 0, "norm"), 256)
    raw = synth.q4k_weights(synth.rng_for("tiny", 0, "w"), 512, 256)
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.gemm("q4_K", *oracle.quantize(oracle.rmsnorm(x, wn, 1e-6)), raw, 512, 256)
        reps += 1
        dt = time.perf_counter() - t0
        if dt > 0.5:
            break
    return 2 * 32 * 512 * 256 * reps / dt / 1e12, dt / reps


def _oracle_producers_full():
    """The CPU oracle's producers on the 7B chain's full shapes (RMSNorm then
    quantise of 3314 x 3584, standalone quantise of 3314 x 3584, SwiGLU then
    quantise of 3314 x 18944); returns {name: (GB/s of algorithmic bytes, s)}."""
    import oracle
    _, x, a, _, n1, _ = _layer0_inputs()
    import synth
    g = synth.activations(synth.rng_for("chain7b", 0, "gate_cpu"), TOKENS, FFN)
    u = synth.activations(synth.rng_for("chain7b", 0, "up_cpu"), TOKENS, FFN)
    res = {}
    for name, fn, nbytes in (
            ("quant_rms", lambda: oracle.quantize(oracle.rmsnorm(x, n1, 1e-6)), TOKENS * HIDDEN * 5.25),
            ("quant_f32", lambda: oracle.quantize(a), TOKENS * HIDDEN * 5.25),
            ("quant_swiglu", lambda: oracle.quantize(oracle.swiglu(g, u)), TOKENS * FFN * 9.25)):
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
        res[name] = {"GB_s": round(nbytes / dt / 1e9, 3), "seconds": round(dt, 3)}
    return res


def cpu_baseline(seconds: float):
    """The CPU oracle (as it is) on a bounded sample of one layer of the chain,
    reported in the chain's unit (TOPS) on all the threads it uses; beside it,
    the same sample on one thread (a shorter one), the tiny workload, the
    producers at the 7B shapes and the 14B decode GEMV step, each in full."""
    import oracle
    tops, tok_done, t_used = _oracle_layer_sample(seconds)
    n_all = oracle.threads()
    oracle.set_threads(1)
    try:
        tops1, tok1, t1 = _oracle_layer_sample(max(1.0, seconds / 4))
    finally:
        oracle.set_threads(n_all)
    dec_gbs, dec_s = _oracle_decode_full()
    tiny_tops, tiny_s = _oracle_tiny_full()
    prod = _oracle_producers_full()
    return {"value": round(tops, 6), "unit": "TOPS", "cores": n_all,
            "host_cpus_available": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"layer 0 of the chain (both RMSNorm producers, the standalone quantise, "
                      f"SwiGLU and all 7 matmuls) for {tok_done} of {TOKENS} tokens, "
                      f"{t_used:.1f} s; the work is linear in tokens",
            "cpu_model": _cpu_model(), "seconds": round(t_used, 2),
            "one_thread": {"value": round(tops1, 6), "unit": "TOPS", "tokens": tok1,
                           "seconds": round(t1, 2)},
            "decode_gemv_full": {"value": round(dec_gbs, 3), "unit": "GB/s", "seconds": round(dec_s, 2),
                                 "sample": "14B decode step in full: RMSNorm 5120 and SwiGLU 13824 "
                                           "producers, attn_v, ffn_down and lm_head q6_K GEMVs"},
            "tiny_full": {"value": round(tiny_tops, 6), "unit": "TOPS", "seconds_per_pass": round(tiny_s, 6),
                          "sample": "32 x 256 RMSNorm -> plane -> q4_K 512 x 256 matmul, in full"},
            "producers_full": prod}


def _smi_sample():
    """One amd-smi reading: socket power (W) and the per-XCD shader clocks
    (MHz), or None where the tool is missing or prints neither."""
    import re
    import subprocess
    try:
        txt = subprocess.run(["amd-smi", "metric", "--power", "--clock"], capture_output=True,
                             text=True, timeout=30).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", txt)
    clk = []
    for blk in re.split(r"\n\s*GFX_\d+:", txt)[1:]:
        m = re.search(r"CLK:\s*([0-9.]+)\s*MHz", blk)
        if m:
            clk.append(float(m.group(1)))
    if pw is None and not clk:
        return None
    return {"socket_W": float(pw.group(1)) if pw else None, "gfx_clk_MHz": clk}


def power_sweep(mmq, torch, synth, seconds=10.0):
    """Socket power and shader clocks while one kernel runs back to back:
    the q4_K gate and q6_K down matmuls at 3314 tokens (also on all-zero
    activations), the matmul's MFMA +
    rescale probes without memory traffic (MFMAs alone, FMAs alone, both in
    the matmul's flow; on small constant operands, w2_, and on random ones
    that change every block, r2_) and the read stream.  Each runs for
    `seconds`; amd-smi is sampled once, after the first third."""
    import ctypes
    import time
    from quantized_matmul_rmsnorm_amd import build as _b
    peak = ctypes.CDLL(_b.LIB_PEAK)
    peak.mmq_peak_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    peak.mmq_peak_probe.restype = ctypes.c_int
    peak.mmq_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p]
    peak.mmq_peak_read.restype = ctypes.c_int
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    ctx = mmq.mmq_create(0, 0)
    res, work, weights = {}, {}, []
    try:
        for name, wt, od, id_ in (("gate_q4k_18944x3584", "q4_K", 18944, 3584),
                                  ("down_q6k_3584x18944", "q6_K", 3584, 18944)):
            raw = synth.weights(wt, synth.rng_for("power", 0, name), od, id_)
            code = mmq.MMQ_Q4_K if wt == "q4_K" else mmq.MMQ_Q6_K
            w = mmq.mmq_register_weight(ctx, code, od, id_, raw, mmq.MMQ_USE_GEMM)
            weights.append(w)
            a = torch.from_numpy(synth.activations(synth.rng_for("power", 0, name + "a"), TOKENS, id_)).cuda()
            o = torch.empty((TOKENS, od), dtype=torch.float32, device="cuda")
            mmq.mmq_quant_f32(ctx, a, TOKENS, id_)
            g = mmq.mmq_gemm_q4k if wt == "q4_K" else mmq.mmq_gemm_q6k
            work[name] = lambda g=g, w=w, a=a, o=o: g(ctx, w, a, TOKENS, o)
            # the same call on all-zero activations: the same instructions with
            # the matrix datapath's operands still
            z = torch.zeros((TOKENS, id_), dtype=torch.float32, device="cuda")
            mmq.mmq_quant_f32(ctx, z, TOKENS, id_)
            work[name + "_zero_activations"] = lambda g=g, w=w, z=z, o=o: g(ctx, w, z, TOKENS, o)
        pout = torch.empty(n_cu * 1024, dtype=torch.float32, device="cuda")
        peak.mmq_peak_probe_info.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                             ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                             ctypes.POINTER(ctypes.c_int)]
        probe_index = {}
        for i in range(peak.mmq_peak_probe_count()):
            nm, th, ti, mw = ctypes.c_char_p(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
            peak.mmq_peak_probe_info(i, ctypes.byref(nm), ctypes.byref(th), ctypes.byref(ti),
                                     ctypes.byref(mw))
            probe_index[nm.value.decode()] = i
        for pname in ("w2_t2_mfma_only", "w2_t2_fma_only", "w2_t2_both_matmul_flow",
                      "r2_t2_mfma_only", "r2_t2_fma_only", "r2_t2_both_matmul_flow"):
            i = probe_index[pname]
            work["probe_" + pname] = lambda i=i: peak.mmq_peak_probe(i, pout.data_ptr(), n_cu, 4096,
                                                                    stream.cuda_stream)
        rbytes = 4 << 30
        rbuf = torch.ones(rbytes // 4, dtype=torch.float32, device="cuda")
        rout = torch.empty(32 * n_cu * 256, dtype=torch.int32, device="cuda")
        work["read_stream_4GiB"] = lambda: peak.mmq_peak_read(rbuf.data_ptr(), rbytes, rout.data_ptr(),
                                                             32 * n_cu, 16, stream.cuda_stream)
        for name, fn in work.items():
            torch.cuda.synchronize()
            t0 = time.time()
            sample, calls = None, 0
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            while time.time() - t0 < seconds:
                e0.record()
                for _ in range(10):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                calls += 10
                if sample is None and time.time() - t0 > seconds / 3:
                    sample = _smi_sample() or {}
            rec = {"us_per_call": round(e0.elapsed_time(e1) * 100.0, 2), "calls": calls}
            rec.update(sample or {})
            res[name] = rec
            log(f"power {name}: {rec}")
        del rbuf, rout, pout
    finally:
        work.clear()
        for w in weights:
            mmq.mmq_weight_free(w)
        mmq.mmq_destroy(ctx)
    return res


def measured_peaks(torch):
    """Ceilings measured on this device, beside the published peaks: the
    matrix pipe's rate for the f16 and int8 32x32 MFMA instructions (a
    benchmark kernel of independent MFMA chains, libmmq_peak.so); the
    matmul's per-block MFMA + rescale-FMA mix with no memory traffic (MFMAs
    alone, FMAs alone and both; hidden_frac is the share of the shorter of
    the two that running both together hides); the overlap probes; a
    read-only stream over 4 GiB, the best of nine launch shapes (the same
    library); and the device-to-device copy rate of a 1 GiB buffer (read +
    write bytes)."""
    import ctypes
    from quantized_matmul_rmsnorm_amd import build as _b
    lib = ctypes.CDLL(_b.LIB_PEAK)
    for fn in (lib.mmq_peak_mfma_f16, lib.mmq_peak_mfma_i8):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    chains = lib.mmq_peak_chains()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * n_cu, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = {}
    for name, fn, ops_per_mfma in (("mfma_f16_32x32x16_TFLOPs", lib.mmq_peak_mfma_f16, 2 * 32 * 32 * 16),
                                   ("mfma_i8_32x32x32_TOPs", lib.mmq_peak_mfma_i8, 2 * 32 * 32 * 32)):
        if fn(out.data_ptr(), blocks, iters, stream.cuda_stream) != 0:
            raise RuntimeError(f"{name}: launch failed")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            if fn(out.data_ptr(), blocks, iters, stream.cuda_stream) != 0:
                raise RuntimeError(f"{name}: launch failed")
        e1.record()
        torch.cuda.synchronize()
        ops = 3 * blocks * 4 * iters * chains * ops_per_mfma
        res[name] = round(ops / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    # the matmul's per-block mix (4 MFMAs + 32 rescale FMAs per wave, 2 waves
    # per SIMD) without memory: MFMAs alone, FMAs alone, both
    lib.mmq_peak_mix.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p]
    lib.mmq_peak_mix.restype = ctypes.c_int
    mblocks, miters = n_cu, 2048
    mout = torch.empty(mblocks * 512, dtype=torch.float32, device="cuda")
    mix_ms = []
    for mode in (0, 1, 2, 3):
        if lib.mmq_peak_mix(mout.data_ptr(), mblocks, miters, mode, stream.cuda_stream) != 0:
            raise RuntimeError("instruction mix: launch failed")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            if lib.mmq_peak_mix(mout.data_ptr(), mblocks, miters, mode, stream.cuda_stream) != 0:
                raise RuntimeError("instruction mix: launch failed")
        e1.record()
        torch.cuda.synchronize()
        mix_ms.append(e0.elapsed_time(e1) / 3)
    mix_ops = mblocks * 8 * miters * 8 * (2 * 32 * 32 * 16)
    t_m, t_v, t_b, t_i8 = mix_ms
    res["matmul_mix"] = {"mfma_only_ms": round(t_m, 4), "fma_only_ms": round(t_v, 4),
                         "both_ms": round(t_b, 4),
                         "both_TFLOPs": round(mix_ops / (t_b * 1e-3) / 1e12, 1),
                         "both_frac_of_f16_peak": round(mix_ops / (t_b * 1e-3) / 1e12 / PEAK_F16_TOPS, 4),
                         "hidden_frac": round((t_m + t_v - t_b) / min(t_m, t_v), 3),
                         "int8_mfma_with_rescale_ms": round(t_i8, 4),
                         "int8_mfma_with_rescale_TOPs": round(mix_ops / (t_i8 * 1e-3) / 1e12, 1)}
    del mout
    res["overlap_probes"] = overlap_probes(torch, lib, n_cu, stream)
    lib.mmq_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p]
    lib.mmq_peak_read.restype = ctypes.c_int
    # the best of a few launch shapes over 4 GiB (well past the 256 MB MALL)
    rbytes = 4 << 30
    rbuf = torch.ones(rbytes // 4, dtype=torch.float32, device="cuda")
    rout = torch.empty(32 * n_cu * 256, dtype=torch.int32, device="cuda")
    best, shapes = None, {}
    for per_cu in (8, 16, 32):
        for unroll in (4, 8, 16):
            blocks = per_cu * n_cu
            for rep in range(4):    # one warm-up, three timed
                if rep == 1:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                if lib.mmq_peak_read(rbuf.data_ptr(), rbytes, rout.data_ptr(), blocks, unroll,
                                     stream.cuda_stream) != 0:
                    raise RuntimeError("read stream: launch failed")
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record()
            torch.cuda.synchronize()
            gbs = round(3 * rbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
            shapes[f"{per_cu}x{unroll}"] = gbs
            if best is None or gbs > best[0]:
                best = (gbs, per_cu, unroll)
    res["hbm_read_GB_s"] = best[0]
    res["hbm_read_shape"] = {"workgroups_per_cu": best[1], "loads_in_flight": best[2],
                             "GB_s_by_wg_per_cu_x_loads": shapes}
    del rbuf, rout
    nel = (1 << 30) // 4
    src = torch.ones(nel, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    res["hbm_copy_GB_s"] = round(5 * 2 * nel * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst, out
    return res


def overlap_probes(torch, lib, n_cu, stream, iters=4096):
    """How far the matrix pipe and the VALU overlap, by variant (libmmq_peak's
    probe table): per 32-block and wave, 2 f16 32x32x16 MFMAs and 16 rescale
    FMAs per output tile, one workgroup per CU with 1, 2 or 4 waves per SIMD;
    the FMAs reading the previous block's MFMA results (the matmul's flow) or
    registers no MFMA writes (independent); both from one wave, or split so
    that one wave of each SIMD pair issues only MFMAs and the other only FMAs.
    hidden_frac = (t_mfma_only + t_fma_only - t_both) / min(t_mfma_only,
    t_fma_only): 0 when the two run one after the other, 1 when the shorter
    one is hidden completely.  A split variant is set against half of the
    one-pipe times of its own wave count (half the waves issue each kind).
    The r2_ and r4_ probes repeat the 2- and 4-waves-per-SIMD ones on random
    operands that change from block to block: the matrix datapath then
    switches as on real data, which pulls the shader clock down."""
    import ctypes
    lib.mmq_peak_probe_count.restype = ctypes.c_int
    lib.mmq_peak_probe_info.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                        ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(ctypes.c_int)]
    lib.mmq_peak_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.mmq_peak_probe.restype = ctypes.c_int
    out = torch.empty(n_cu * 1024, dtype=torch.float32, device="cuda")
    times, info = {}, {}
    for i in range(lib.mmq_peak_probe_count()):
        nm, th, ti, mw = ctypes.c_char_p(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        if lib.mmq_peak_probe_info(i, ctypes.byref(nm), ctypes.byref(th), ctypes.byref(ti),
                                   ctypes.byref(mw)) != 0:
            raise RuntimeError("probe info")
        name = nm.value.decode()
        # random-operand probes pull the clock down as a matmul on real data
        # does, so they run long enough (about 0.2 s) for the clock to settle
        warm, reps = (64, 64) if name.startswith(("r2_", "r4_")) else (1, 3)
        for _ in range(warm):
            if lib.mmq_peak_probe(i, out.data_ptr(), n_cu, iters, stream.cuda_stream) != 0:
                raise RuntimeError(f"probe {name}: launch failed")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            lib.mmq_peak_probe(i, out.data_ptr(), n_cu, iters, stream.cuda_stream)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        ops = n_cu * mw.value * iters * 2 * ti.value * 2 * (2 * 32 * 32 * 16)
        times[name] = ms
        info[name] = {"ms": round(ms, 4), "threads": th.value,
                      "mfma_TFLOPs": round(ops / (ms * 1e-3) / 1e12, 1) if ops else None}
    del out
    for name, rec in info.items():
        pre = name.split("_both")[0].split("_split")[0]
        tm, tv = times.get(pre + "_mfma_only"), times.get(pre + "_fma_only")
        if tm is None or tv is None or name.endswith("_only"):
            continue
        if "_split" in name:
            tm, tv = tm / 2, tv / 2
        rec["hidden_frac"] = round((tm + tv - times[name]) / min(tm, tv), 3)
    return info


ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(ROOT, "quantized_matmul_rmsnorm_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemm_da_q4k_traffic_7b_chain.txt")


def gemm_source_sha():
    import hashlib
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per q4_K matmul launch from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE runs, each scaled by the copy calibration), or
    None when the summary is missing or was taken from another gemm.hip."""
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("traffic_json:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("gemm_sha256") == gemm_source_sha():
                        return rec
    except (OSError, ValueError):
        pass
    return None


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path is data-parallel over tokens and needs no "
              f"collective; --gpus {args.gpus} is not supported (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    root = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, root)
    from quantized_matmul_rmsnorm_amd import build as _b
    if not (os.path.exists(_b.LIB) and os.path.exists(_b.LIB_PEAK)):
        _b.build()
    import quantized_matmul_rmsnorm_amd as mmq
    import synth

    if args.copy_calibration:
        nel = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {nel * 4} bytes read, {nel * 4} bytes written")
        del src, dst

    t_setup = time.perf_counter()
    chain = Chain(mmq, torch, synth, args.layers)
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s")
    for _ in range(args.warmup):
        chain.step()
    torch.cuda.synchronize()
    st0 = mmq.mmq_stats(chain.ctx)

    def timed_steps():
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        marks = [start]
        for _ in range(args.steps):
            chain.step()
            ev = torch.cuda.Event(enable_timing=True)
            ev.record()
            marks.append(ev)
        stop.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per_step = sorted(a.elapsed_time(b) for a, b in zip(marks[:-1], marks[1:]))
        return start.elapsed_time(stop) / args.steps, per_step[len(per_step) // 2], wall

    # The value: K steps with nothing recorded but the step boundaries.
    chain.events = None
    ms_step, ms_median, wall = timed_steps()
    # The per-kernel breakdown and the roofline: K more steps with HIP events
    # around every call on the launch stream (the events add GPU time, so this
    # pass is not the value).
    chain.events = {}
    ms_step_instr, _, _ = timed_steps()
    cls_ms, cls_n = chain.class_times_ms()
    chain.events = None
    st1 = mmq.mmq_stats(chain.ctx)
    # device memory both ways: what the library holds (registered tiles,
    # planes and split-K scratch) against the raw superblocks it was given
    raw_bytes = args.layers * sum(od * id_ // 256 * (144 if wt == "q4_K" else 210)
                                  for _, wt, od, id_, _ in LAYER_GEMMS)
    memory = {"raw_superblock_bytes": raw_bytes, "registered_weight_bytes": st1["weight_bytes"],
              "registered_over_raw": round(st1["weight_bytes"] / raw_bytes, 3),
              "plane_and_scratch_bytes": st1["plane_bytes"],
              "activation_and_output_bytes": sum(
                  t.numel() * 4 for L in chain.layers for k, t in L.items()
                  if k in ("x_attn", "attn_out", "x_ffn", "norm_attn", "norm_ffn")) +
                  sum(t.numel() * 4 for t in (chain.y_attn, chain.y_ffn, chain.y_sw)) +
                  sum(t.numel() * 4 for t in chain.out.values())}
    ops = chain_ops(TOKENS, args.layers)
    tops = ops / (ms_step * 1e-3) / 1e12
    log(f"{ms_step:.2f} ms/step ({wall / args.steps * 1e3:.2f} ms wall), {tops:.1f} TOPS")

    q4_ops_launch = 2 * TOKENS * sum(od * id_ for _, wt, od, id_, _ in LAYER_GEMMS if wt == "q4_K") / 5
    q4_avg_us = 1e3 * cls_ms["gemm_q4k"] / cls_n["gemm_q4k"]
    achieved = q4_ops_launch / (q4_avg_us * 1e-6) / 1e12
    q4_shapes = [(od, id_) for _, wt, od, id_, _ in LAYER_GEMMS if wt == "q4_K"]
    # the method's own data, each byte once: q4_K superblocks (144 B / 256
    # weights), the plane (1 + 4/32 + 4/32 B per value), f32 outputs
    q4_alg_bytes = sum(od * id_ * 144 / 256 + TOKENS * id_ * 1.25 + TOKENS * od * 4
                       for od, id_ in q4_shapes) / len(q4_shapes)
    q6_ops_launch = 2 * TOKENS * sum(od * id_ for _, wt, od, id_, _ in LAYER_GEMMS if wt == "q6_K") / 2
    q6_avg_us = 1e3 * cls_ms["gemm_q6k"] / cls_n["gemm_q6k"]

    kernels = {}
    for k in cls_ms:
        kernels[k] = {"launches": cls_n[k], "avg_us": round(1e3 * cls_ms[k] / cls_n[k], 2),
                      "share": round(cls_ms[k] / (ms_step_instr * args.steps), 4)}
    # producers are HBM-bound: algorithmic bytes per launch
    rms_b = TOKENS * HIDDEN * (4 + 1.25) + HIDDEN * 4
    sw_b = TOKENS * FFN * (8 + 1.25)
    qf_b = TOKENS * HIDDEN * (4 + 1.25)
    for k, b in (("quant_rms", rms_b), ("quant_swiglu", sw_b), ("quant_f32", qf_b)):
        kernels[k]["GB_s"] = round(b / (kernels[k]["avg_us"] * 1e-6) / 1e9, 1)
    kernels["gemm_q4k"]["TOPS"] = round(achieved, 1)
    kernels["gemm_q6k"]["TOPS"] = round(q6_ops_launch / (q6_avg_us * 1e-6) / 1e12, 1)

    # the same step captured once into a HIP graph and replayed (launch census
    # from the library's counters during the capture)
    st_a = mmq.mmq_stats(chain.ctx)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain.step()
    st_b = mmq.mmq_stats(chain.ctx)
    mmq.mmq_cache_clear(chain.ctx)
    graph.replay()
    torch.cuda.synchronize()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(args.steps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / args.steps
    del graph
    graph_rec = {"ms_per_step": round(graph_ms, 3), "tops": round(ops / (graph_ms * 1e-3) / 1e12, 2),
                 "launches_per_step": sum(st_b[k] - st_a[k] for k in st_b if k.startswith("launches_"))}
    log(f"graph replay: {graph_ms:.2f} ms/step")

    packed = None if args.no_packed else packed_q4k(mmq, torch, synth, chain)
    traffic = measured_traffic()
    peaks = measured_peaks(torch)
    log(f"measured: f16 MFMA {peaks['mfma_f16_32x32x16_TFLOPs']} TFLOP/s, int8 MFMA "
        f"{peaks['mfma_i8_32x32x32_TOPs']} TOP/s, read {peaks['hbm_read_GB_s']} GB/s, "
        f"copy {peaks['hbm_copy_GB_s']} GB/s")
    decode = None if args.no_decode else decode_gemv(mmq, torch, synth)
    if decode is not None:
        decode["aggregate_frac_measured_copy"] = round(decode["aggregate_GB_s"] / peaks["hbm_copy_GB_s"], 4)
        decode["aggregate_frac_measured_read"] = round(decode["aggregate_GB_s"] / peaks["hbm_read_GB_s"], 4)
    small = small_n_sweep(mmq, torch, synth) if args.small_n else None
    power = power_sweep(mmq, torch, synth) if args.power else None
    crossover = decode_crossover_sweep(mmq, torch, synth) if args.decode_crossover else None
    f16ref = f16_reference(torch) if args.f16_reference else None
    if packed is not None:
        packed["chain"] = packed_chain(mmq, torch, synth, args, ops)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)

    rec = {
        "metric": "MMQ chain TOPS + tok/s-equiv at 7B pp3314; q6_K decode GEMV GB/s",
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "mfma_instruction": "v_mfma_f32_32x32x16_f16 on exact integer operands (int8 codes, "
                            "integer weight values); integer block dots, f32 rescale",
        "data": "synthetic",
        "config": {"workload": "7B prefill matmul chain: 28 layers x (RMSNorm->q8 plane->q,k,v; "
                               "quantise->o; RMSNorm->gate,up; SwiGLU->down), skip-write planes",
                   "tokens": TOKENS, "hidden": HIDDEN, "ffn": FFN, "kv": KV, "layers": args.layers,
                   "weights": "q4_K (q,k,o,gate,up), q6_K (v,down)"},
        "tok_s_equiv": round(TOKENS / (ms_step * 1e-3), 1),
        "median_ms_per_step": round(ms_median, 3),
        "instrumented_ms_per_step": round(ms_step_instr, 3),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TOPS", "frac": round(achieved / PEAK_INT8_TOPS, 4),
                     "traffic": None if traffic is None else traffic["bytes_per_launch"],
                     "kernel": "k_gemm_da<true> (q4_K)",
                     "ops_per_launch": q4_ops_launch,
                     "algorithmic_bytes_per_launch": round(q4_alg_bytes), "avg_launch_us": round(q4_avg_us, 2),
                     "frac_of_f16_mfma_peak": round(achieved / PEAK_F16_TOPS, 4),
                     "frac_of_measured_f16_mfma": round(achieved / peaks["mfma_f16_32x32x16_TFLOPs"], 4),
                     "frac_of_measured_i8_mfma": round(achieved / peaks["mfma_i8_32x32x32_TOPs"], 4),
                     "frac_of_measured_matmul_mix": round(achieved / peaks["matmul_mix"]["both_TFLOPs"], 4),
                     "frac_of_measured_matmul_flow": round(
                         achieved / peaks["overlap_probes"]["w2_t2_both_matmul_flow"]["mfma_TFLOPs"], 4),
                     "frac_of_measured_matmul_flow_random": round(
                         achieved / peaks["overlap_probes"]["r2_t2_both_matmul_flow"]["mfma_TFLOPs"], 4)},
        "measured_peaks": peaks,
        "kernels": kernels,
        "graph": graph_rec,
        "cache": {k: st1[k] - st0[k] for k in ("cache_hits", "cache_misses", "cache_refusals")},
        "memory": memory,
        "packed_q4k_tiles": packed,
        "decode_gemv": decode,
        "small_n_us": small,
        "power": power,
        "decode_crossover_us": crossover,
        "f16_gemm_reference": f16ref,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
