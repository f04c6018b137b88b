"""The reading of the matmul tolerance, checked on the CPU.

The pages fix the matmul's arithmetic: an exact integer dot per 32-block,
rescaled in f32.  The acceptance bar 1e-3 * (|ref| + 1) is read per output,
plus the rounding budget of that f32 rescale, (24 + nsb) * 2^-24 *
sum_b |term_b| (tests/gpu_util.py, with the sum of |block term| from the
oracle).  This test pins both halves of that reading on outputs of the size
the 7B chain's down projection reaches (SwiGLU activations in the thousands,
q6_K weights of the synthetic recipe):
  * an f32 evaluation of the oracle's own block terms, in the matmul's order
    (per superblock a chain of eight fused multiply-adds of D and the block
    dot, then one fused multiply-add of d and that sum into the output), misses
    the bare bar on some outputs -- those whose sum cancels to far below its
    terms -- so no f32 rescale can meet it there;
  * the same evaluation stays within bar + budget on every output, as the
    first-order worst-case bound says it must.
"""
import numpy as np

import oracle
import synth
from tests.gpu_util import GEMM_TOL, gemm_bound, gemm_ref


def _f32(v):
    return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)


def _fma32(a, b, c):
    # the f64 product of two f32 values is exact; one rounding to f32 after the add
    return _f32(a * b + c)


def test_f32_rescale_needs_the_rounding_budget():
    n, od, id_ = 96, 512, 1024
    nsb = id_ // 256
    rng = synth.rng_for("tolerance", 0, "act")
    y = (synth.activations(rng, n, id_) * np.float32(3000.0)).astype(np.float32)
    raw = synth.q6k_weights(synth.rng_for("tolerance", 0, "w"), od, id_)
    q, D, S = oracle.quantize(y)
    ref = gemm_ref("q6_K", q, D, S, raw, od, id_)

    fields = [oracle.q6k_fields(raw.reshape(od, nsb, 210)[o, s]) for o in range(od) for s in range(nsb)]
    dd = np.array([f[0] for f in fields]).reshape(od, nsb)
    sc = np.array([f[1] for f in fields]).reshape(od, nsb, 16).astype(np.int64)
    qw = np.array([f[2] for f in fields]).reshape(od, nsb, 256).astype(np.int64) - 32
    qa = q.astype(np.int64).reshape(n, nsb, 8, 32)
    Dd = D.astype(np.float64)
    res = np.zeros((n, od))
    for s in range(nsb):
        acc = np.zeros((n, od))
        for j in range(8):
            w0 = qw[:, s, 32 * j:32 * j + 16] * sc[:, s, 2 * j:2 * j + 1]
            w1 = qw[:, s, 32 * j + 16:32 * j + 32] * sc[:, s, 2 * j + 1:2 * j + 2]
            X = (qa[:, s, j, :16] @ w0.T + qa[:, s, j, 16:] @ w1.T).astype(np.float64)  # exact
            acc = _fma32(Dd[:, s * 8 + j][:, None], X, acc)
        res = _fma32(dd[None, :, s], acc, res)

    r = ref.out.astype(np.float64)
    err = np.abs(res - r)
    bare = err > GEMM_TOL * (np.abs(r) + 1.0)
    assert np.abs(r).std() > 1e5                 # the scale the chain's down projection reaches
    assert bare.sum() >= 1, "expected near-zero sums of large terms to miss the bare bar"
    assert np.all(err <= gemm_bound(ref))
    # the budget is a small part of the bar for a typical output
    typical = np.median(gemm_bound(ref) / (GEMM_TOL * (np.abs(r) + 1.0)) - 1.0)
    assert typical < 0.2

