"""Helpers shared by the GPU tests: a context per test module, plane export into
numpy, and the parity predicates the acceptance rules fix.

Acceptance (as fixed for this path):
  * a standalone quantise of the oracle's f32 y is bit-exact (q, D, S);
  * a fused producer may differ from the oracle plane in at most 1e-4 of the
    codes, each by at most 1; S equals the sum of the GPU's own codes;
  * matmul / GEMV outputs satisfy |got - ref| <= 1e-3 * (|ref| + 1), with ref
    the oracle matmul run on the GPU's exported plane, plus the rounding budget
    of the f32 per-block rescale the method prescribes: (24 + nsb) * 2^-24 *
    sum_b |term_b|, with nsb the superblocks of the contraction and the sum of
    |block term| from the oracle.  Each output is a chain of at most 8 block
    FMAs per superblock sum, nsb superblock steps, the min-term MFMA's
    products and at most 8 split or reduction steps; every f32 step rounds
    once against a partial sum bounded by sum_b |term_b|, so this is the
    first-order worst-case error of that evaluation.  It only matters where
    an output cancels to far below its terms: there even an f32 evaluation of
    the oracle's own terms misses the bare 1e-3 * (|ref| + 1) (pinned on the
    CPU in tests/test_tolerance_reading.py).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import quantized_matmul_rmsnorm_amd as mmq

GEMM_TOL = 1e-3
FLIP_RATE = 1e-4
U = 2.0 ** -24


class GemmRef:
    """An oracle matmul result with, per element, the sum over blocks of
    |block term| and the superblock count of the contraction."""

    def __init__(self, out: np.ndarray, mag: np.ndarray, nsb: int):
        self.out, self.mag, self.nsb = out, mag, nsb

    def __getitem__(self, k):
        return GemmRef(self.out[k], self.mag[k], self.nsb)

    @property
    def shape(self):
        return self.out.shape


def gemm_ref(wtype, q, D, S, raw, od, id_, tok=None, outs=None) -> GemmRef:
    out, mag = oracle.gemm(wtype, q, D, S, raw, od, id_, tok=tok, outs=outs, with_mag=True)
    return GemmRef(out, mag, id_ // 256)


def gemm_bound(ref: GemmRef) -> np.ndarray:
    return GEMM_TOL * (np.abs(ref.out.astype(np.float64)) + 1.0) + (24 + ref.nsb) * U * ref.mag


def dev_tensor(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def export_plane(ctx, key: torch.Tensor, n: int, d: int, include_pad: bool = False):
    rows = mmq.mmq_plane_rows(n) if include_pad else n
    q = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    D = torch.empty((rows, d // 32), dtype=torch.float32, device="cuda")
    S = torch.empty((rows, d // 32), dtype=torch.int32, device="cuda")
    mmq.mmq_plane_export(ctx, key, n, d, int(include_pad), q, D, S)
    torch.cuda.synchronize()
    return q.cpu().numpy(), D.cpu().numpy(), S.cpu().numpy()


def assert_plane_equal(a, b, what=""):
    qa, Da, Sa = a
    qb, Db, Sb = b
    assert np.array_equal(qa, qb), f"{what}: codes differ at {np.argwhere(qa != qb)[:5]}"
    assert np.array_equal(Da.view(np.uint32), Db.view(np.uint32)), f"{what}: scales differ"
    assert np.array_equal(Sa, Sb), f"{what}: sums differ"


def assert_fused_close(gpu, ref, y_gpu=None, y_ref=None, what=""):
    qg, Dg, Sg = gpu
    qr, Dr, Sr = ref
    diff = np.abs(qg.astype(np.int32) - qr.astype(np.int32))
    assert diff.max(initial=0) <= 1, f"{what}: a code differs by {diff.max()}"
    rate = np.count_nonzero(diff) / diff.size
    assert rate <= FLIP_RATE, f"{what}: flip rate {rate:.3g} > {FLIP_RATE}"
    n, d = qg.shape
    assert np.array_equal(Sg, qg.reshape(n, d // 32, 32).astype(np.int32).sum(-1)), f"{what}: S != sum q"
    if y_gpu is not None:
        am_g = np.abs(y_gpu.reshape(n, -1, 32)).max(-1)
        am_r = np.abs(y_ref.reshape(n, -1, 32)).max(-1)
        same = am_g == am_r
        assert np.array_equal(Dg[same].view(np.uint32), Dr[same].view(np.uint32)), f"{what}: D differs"
        # elsewhere D follows the (few-ulp) amax difference
        rel = np.abs(Dg[~same].astype(np.float64) - Dr[~same]) / np.maximum(np.abs(Dr[~same]), 1e-30)
        assert rel.max(initial=0) < 1e-5, f"{what}: D off by {rel.max()}"
    return rate


def assert_gemm_close(got: np.ndarray, ref: GemmRef, what=""):
    """Every output within 1e-3 * (|ref| + 1) plus the f32 rescale's rounding
    budget; returns the worst err / (|ref| + 1) and prints how many outputs
    needed the budget."""
    assert isinstance(ref, GemmRef), "compare against gemm_ref(...), which carries the budget"
    r = ref.out.astype(np.float64)
    assert got.shape == r.shape, (got.shape, r.shape)
    err = np.abs(got.astype(np.float64) - r)
    bad = ~(err <= gemm_bound(ref))          # NaN in got fails too
    assert not bad.any(), (f"{what}: {bad.sum()} outputs outside 1e-3*(|ref|+1) + budget; worst err "
                           f"{np.nanmax(err):.4g} at {np.unravel_index(np.nanargmax(err), err.shape)}")
    over = int((err > GEMM_TOL * (np.abs(r) + 1.0)).sum())
    if over:
        print(f"{what}: {over} of {err.size} outputs within the rounding budget only "
              f"(near-zero sums of large terms)", flush=True)
    return float((err / (np.abs(r) + 1.0)).max(initial=0.0))
