"""Randomised check of the plane cache against a small Python model of its
contract (include/mmq.h): producers record planes under their output buffer
(dead when write_y == 0), consumers hit on (key, n, d) or quantise on a miss,
anything that would read bytes of a dead buffer (a quantise, a producer's
inputs) is refused, every library write to caller memory (a producer's y, a
consumer's out) drops the planes keyed in those bytes and revives them, eight
entries with least-recently-used reuse, and clear / invalidate (which drops
every piece of the dead range recorded for the key).  Runs on dry-run
contexts (host bookkeeping only).
"""
import random

import pytest

import quantized_matmul_rmsnorm_amd as mmq

SLOTS = 8


class Model:
    def __init__(self):
        self.entries = [None] * SLOTS          # dict(key, n, d, last)
        self.dead = []                         # [lo, hi, key of the recording producer]
        self.tick = 0
        self.st = dict(hits=0, misses=0, refusals=0, rms=0, swiglu=0, f32=0, gemm=0)

    def _overlaps_dead(self, lo, hi):
        return any(lo < h and l < hi for l, h, _ in self.dead)

    def _drop_overlapping(self, lo, hi):
        for i, e in enumerate(self.entries):
            if e and lo < e["key"] + e["n"] * e["d"] * 4 and e["key"] < hi:
                self.entries[i] = None

    def _revive(self, lo, hi):
        keep = []
        for l, h, k in self.dead:
            if hi <= l or h <= lo:
                keep.append((l, h, k))
                continue
            if l < lo:
                keep.append((l, lo, k))
            if hi < h:
                keep.append((hi, h, k))
        self.dead = keep

    def _written(self, lo, hi):
        self._drop_overlapping(lo, hi)
        self._revive(lo, hi)

    def _find(self, key, n, d):
        for i, e in enumerate(self.entries):
            if e and (e["key"], e["n"], e["d"]) == (key, n, d):
                return i
        return -1

    def _acquire(self, key, n, d):
        i = self._find(key, n, d)
        if i >= 0:
            return i
        for j, e in enumerate(self.entries):
            if e is None:
                return j
        return min(range(SLOTS), key=lambda j: self.entries[j]["last"])

    def _commit(self, i, key, n, d):
        self.tick += 1
        self.entries[i] = dict(key=key, n=n, d=d, last=self.tick)

    def produce(self, kind, a, y, n, d, write_y, b=None):
        bytes_ = n * d * 4
        b_bytes = d * 4 if kind == "rms" else bytes_
        if kind != "f32" and (self._overlaps_dead(a, a + bytes_) or
                              self._overlaps_dead(b, b + b_bytes)):
            self.st["refusals"] += 1
            return mmq.MMQ_E_DEAD_WRITE
        if kind == "f32":
            if self._overlaps_dead(a, a + bytes_):
                self.st["refusals"] += 1
                return mmq.MMQ_E_DEAD_WRITE
            self._drop_overlapping(a, a + bytes_)
            self._commit(self._acquire(a, n, d), a, n, d)
            self.st["f32"] += 1
            return mmq.MMQ_OK
        self._drop_overlapping(y, y + bytes_)
        i = self._acquire(y, n, d)
        if write_y:
            self._revive(y, y + bytes_)
        self._commit(i, y, n, d)
        if not write_y:
            self._revive(y, y + bytes_)
            self.dead.append((y, y + bytes_, y))
        self.st[kind] += 1
        return mmq.MMQ_OK

    def consume(self, a, n, d, out, od):
        i = self._find(a, n, d)
        if i >= 0:
            self.st["hits"] += 1
            self.tick += 1
            self.entries[i]["last"] = self.tick
            self.st["gemm"] += 1
            self._written(out, out + n * od * 4)
            return mmq.MMQ_OK
        if self._overlaps_dead(a, a + n * d * 4):
            self.st["refusals"] += 1
            return mmq.MMQ_E_DEAD_WRITE
        self.st["misses"] += 1
        rc = self.produce("f32", a, None, n, d, 0)
        if rc == mmq.MMQ_OK:
            self.st["gemm"] += 1
            self._written(out, out + n * od * 4)
        return rc

    def clear(self):
        self.entries = [None] * SLOTS
        self.dead = []

    def invalidate(self, key):
        for i, e in enumerate(self.entries):
            if e and e["key"] == key:
                self.entries[i] = None
        self.dead = [(l, h, k) for l, h, k in self.dead if k != key]


def _status(fn, *a):
    try:
        fn(*a)
    except mmq.MmqError as e:
        return e.status
    return mmq.MMQ_OK


@pytest.mark.parametrize("seed", range(6))
def test_cache_matches_model(seed):
    rng = random.Random(seed)
    ctx = mmq.mmq_create(0, mmq.MMQ_CTX_DRYRUN)
    model = Model()
    ws = {}
    try:
        for d in (256, 512):
            raw = bytes(64 * d // 256 * 144)
            ws[d] = mmq.mmq_register_weight(ctx, mmq.MMQ_Q4_K, 64, d, raw, mmq.MMQ_USE_GEMM)
        base = 0x10000000
        # buffers at 4 KiB steps in a 64 KiB window: 8 x 256 x 4 B = 8 KiB spans
        # make neighbouring keys overlap
        addrs = [base + 4096 * k for k in range(16)]
        W, O = 0x20000000, 0x30000000
        for step in range(400):
            op = rng.choices(["rms", "swiglu", "f32", "gemm", "clear", "invalidate"],
                             weights=[5, 3, 2, 8, 1, 1])[0]
            n = rng.choice((1, 2, 8))
            d = rng.choice((256, 512))
            a = rng.choice(addrs)
            if op in ("rms", "swiglu"):
                y = rng.choice(addrs)
                wy = rng.random() < 0.4
                # the second input: the RMSNorm weight (never a key), or the
                # SwiGLU up buffer, sometimes a key buffer
                b = W if (op == "rms" or rng.random() < 0.5) else rng.choice(addrs)
                if op == "rms":
                    got = _status(mmq.mmq_quant_rms, ctx, a, b, y, n, d, 1e-6, int(wy))
                else:
                    got = _status(mmq.mmq_quant_swiglu, ctx, a, b, y, n, d, int(wy))
                want = model.produce(op, a, y, n, d, wy, b)
            elif op == "f32":
                got = _status(mmq.mmq_quant_f32, ctx, a, n, d)
                want = model.produce("f32", a, None, n, d, 0)
            elif op == "gemm":
                # the output lands on a key buffer half of the time
                out = O if rng.random() < 0.5 else rng.choice(addrs)
                got = _status(mmq.mmq_gemm_q4k, ctx, ws[d], a, n, out)
                want = model.consume(a, n, d, out, 64)
            elif op == "clear":
                mmq.mmq_cache_clear(ctx)
                model.clear()
                got = want = mmq.MMQ_OK
            else:
                mmq.mmq_cache_invalidate(ctx, a)
                model.invalidate(a)
                got = want = mmq.MMQ_OK
            assert got == want, (seed, step, op)
            st = mmq.mmq_stats(ctx)
            assert st["cache_hits"] == model.st["hits"], (seed, step)
            assert st["cache_misses"] == model.st["misses"], (seed, step)
            assert st["cache_refusals"] == model.st["refusals"], (seed, step)
            assert st["launches_quant_rms"] == model.st["rms"]
            assert st["launches_quant_swiglu"] == model.st["swiglu"]
            assert st["launches_quant_f32"] == model.st["f32"]
            assert st["launches_gemm_q4k"] == model.st["gemm"]
            assert st["cache_entries"] == sum(e is not None for e in model.entries)
    finally:
        for w in ws.values():
            mmq.mmq_weight_free(w)
        mmq.mmq_destroy(ctx)
