"""Pins of the CPU oracle against facts fixed outside the oracle itself.

None of these re-run the oracle's own formula: they check it against the
binary16 definition (via numpy's independent float16), an independent field
encoder, brute-force f64 dequantised matmuls, exact integer matmuls in the
unit-scale special case, textbook constants, closed forms and invariants of
the quantiser.  Each is chosen so that a plausible slip (dropped term, wrong
sign, swapped nibble or half, transposed operand, divide-by-(d-1), a
reciprocal instead of a quotient) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle
from tests.kquant_encode import (f16_bits, q4k_encode, q5k_encode, q6k_encode, random_q4k,
                                 random_q5k, random_q6k)

U24 = 2.0 ** -24


# ---------------------------------------------------------------- binary16
def test_f16_all_values_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(b)) for b in bits], np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isnan(got[np.isnan(ref)]))
    assert np.array_equal(np.isinf(got), np.isinf(ref))


def test_f16_textbook_values():
    assert oracle.f16_to_f32(0x3C00) == 1.0
    assert oracle.f16_to_f32(0xC000) == -2.0
    assert oracle.f16_to_f32(0x7BFF) == 65504.0
    assert oracle.f16_to_f32(0x0001) == 2.0 ** -24
    assert oracle.f16_to_f32(0x0400) == 2.0 ** -14
    assert oracle.f16_to_f32(0x3555) == 0.333251953125


# ---------------------------------------------------------------- formats
def test_q4k_field_roundtrip_random():
    rng = np.random.default_rng(1)
    for _ in range(50):
        sc = rng.integers(0, 64, 8); mn = rng.integers(0, 64, 8); q = rng.integers(0, 16, 256)
        d = np.float16(rng.uniform(1e-3, 1e-2)); dm = np.float16(rng.uniform(1e-3, 1e-2))
        blk = q4k_encode(f16_bits(d), f16_bits(dm), sc, mn, q)
        gd, gdm, gsc, gmn, gq = oracle.q4k_fields(blk)
        assert gd == float(d) and gdm == float(dm)
        assert np.array_equal(gsc, sc) and np.array_equal(gmn, mn) and np.array_equal(gq, q)


def test_q5k_field_roundtrip_random():
    rng = np.random.default_rng(4)
    for _ in range(50):
        sc = rng.integers(0, 64, 8); mn = rng.integers(0, 64, 8); q = rng.integers(0, 32, 256)
        d = np.float16(rng.uniform(1e-3, 1e-2)); dm = np.float16(rng.uniform(1e-3, 1e-2))
        blk = q5k_encode(f16_bits(d), f16_bits(dm), sc, mn, q)
        gd, gdm, gsc, gmn, gq = oracle.q5k_fields(blk)
        assert gd == float(d) and gdm == float(dm)
        assert np.array_equal(gsc, sc) and np.array_equal(gmn, mn) and np.array_equal(gq, q)


def test_q6k_field_roundtrip_random():
    rng = np.random.default_rng(2)
    for _ in range(50):
        sc = rng.integers(-128, 128, 16); q = rng.integers(0, 64, 256)
        d = np.float16(rng.uniform(1e-3, 1e-2))
        blk = q6k_encode(f16_bits(d), sc, q)
        gd, gsc, gq = oracle.q6k_fields(blk)
        assert gd == float(d)
        assert np.array_equal(gsc, sc) and np.array_equal(gq, q)


def test_q4k_hand_worked_block():
    """A block written byte by byte, fields worked out by hand from the format."""
    blk = np.zeros(144, np.uint8)
    blk[0:2] = [0x00, 0x3C]          # d = 1.0
    blk[2:4] = [0x00, 0x38]          # dmin = 0.5
    blk[4] = 0xC3                    # sc0 = 0x03, top bits 11 -> high bits of sc4
    blk[8] = 0x45                    # m0 = 0x05, top bits 01 -> high bits of m4
    blk[12] = 0x5A                   # sc4 low nibble 0xA, m4 low nibble 0x5
    blk[16] = 0x72                   # element 0 -> 2, element 32 -> 7
    blk[16 + 32 * 3 + 31] = 0xF1     # element 223 -> 1, element 255 -> 15
    d, dm, sc, mn, q = oracle.q4k_fields(blk)
    assert (d, dm) == (1.0, 0.5)
    assert sc[0] == 3 and mn[0] == 5
    assert sc[4] == 0x3A and mn[4] == 0x15        # (11 << 4) | 0xA, (01 << 4) | 0x5
    assert q[0] == 2 and q[32] == 7 and q[223] == 1 and q[255] == 15
    assert q[1] == 0 and q[33] == 0
    w = oracle.dequant("q4_K", blk, 1, 256)
    assert w[0, 0] == 1.0 * 3 * 2 - 0.5 * 5          # sub-block 0
    assert w[0, 32] == 1.0 * sc[1] * 7 - 0.5 * mn[1]  # element 32 is sub-block 1
    assert w[0, 255] == 1.0 * sc[7] * 15 - 0.5 * mn[7]


def test_q5k_hand_worked_block():
    """A q5_K block written byte by byte: the header as in the q4_K block
    above, then high bits and low nibbles whose quants are worked out by hand."""
    blk = np.zeros(176, np.uint8)
    blk[0:2] = [0x00, 0x3C]          # d = 1.0
    blk[2:4] = [0x00, 0x38]          # dmin = 0.5
    blk[4] = 0xC3                    # sc0 = 3; top bits 11 -> high bits of sc4
    blk[8] = 0x45                    # m0 = 5; top bits 01 -> high bits of m4
    blk[12] = 0x5A                   # sc4 = 0x3A, m4 = 0x15
    blk[16] = 0b10000101             # byte 0: bit0 -> e0, bit2 -> e64, bit7 -> e224
    blk[16 + 31] = 0b00000010        # byte 31: bit1 -> e63
    blk[48] = 0x72                   # e0 low 2, e32 low 7
    blk[48 + 32] = 0x3C              # e64 low 0xC, e96 low 3
    blk[48 + 31] = 0x90              # e31 low 0, e63 low 9
    blk[48 + 96] = 0x0E              # e192 low 0xE, e224 low 0
    d, dm, sc, mn, q = oracle.q5k_fields(blk)
    assert (d, dm) == (1.0, 0.5)
    assert sc[0] == 3 and mn[0] == 5 and sc[4] == 0x3A and mn[4] == 0x15
    assert q[0] == 2 + 16 and q[32] == 7 and q[64] == 12 + 16 and q[96] == 3
    assert q[31] == 0 and q[63] == 9 + 16 and q[192] == 14 and q[224] == 16
    assert q[1] == 0 and q[65] == 0
    w = oracle.dequant("q5_K", blk, 1, 256)
    assert w[0, 0] == 1.0 * 3 * 18 - 0.5 * 5
    assert w[0, 224] == 1.0 * sc[7] * 16 - 0.5 * mn[7]


def test_q6k_hand_worked_block():
    blk = np.zeros(210, np.uint8)
    blk[208:210] = [0x00, 0x40]      # d = 2.0
    blk[192] = 0xFF                  # scale 0 = -1
    blk[193] = 0x05                  # scale 1 = 5
    blk[207] = 0x80                  # scale 15 = -128
    blk[0] = 0x9F                    # element 0 low 0xF, element 64 low 0x9
    blk[128] = 0b11100100            # element 0 hi 0, element 32 hi 1, 64 hi 2, 96 hi 3
    blk[64 + 31 + 32] = 0xA0         # element 128+64+32+31 = 255 low nibble 0xA
    blk[128 + 32 + 31] = 0b11000000  # element 255 hi 3
    d, sc, q = oracle.q6k_fields(blk)
    assert d == 2.0 and sc[0] == -1 and sc[1] == 5 and sc[15] == -128
    assert q[0] == 15 and q[32] == 16 and q[64] == 9 + 32 and q[96] == 48
    assert q[255] == 10 + 48
    w = oracle.dequant("q6_K", blk, 1, 256)
    assert w[0, 0] == 2.0 * -1 * (15 - 32)
    assert w[0, 16] == 2.0 * 5 * (0 - 32)            # element 16 uses scale 1
    assert w[0, 255] == 2.0 * -128 * (58 - 32)


def test_format_sizes_match_page_figures():
    """210 B per 256 q6_K weights reproduces the D3-7 page's attn_v bandwidth
    (1024 x 5120 weights streamed in 24.32 us at ~177 GB/s, Result paragraph);
    the fixture under tests/golden/ carries the figures and their citation."""
    fig = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split("=")
                fig[k.strip()] = float(v)
    nbytes = fig["attn_v_rows"] * fig["attn_v_cols"] / 256 * 210
    gbs = nbytes / (fig["attn_v_us"] * 1e-6) / 1e9
    assert abs(gbs - fig["attn_v_gbs"]) < 1.0
    # r52 page, section 1: one f32 gate (or up) tensor of 3325 x 18944 is 251.9 MB
    mb = fig["swiglu_tokens"] * fig["swiglu_ffn"] * 4 / 1e6
    assert abs(mb - fig["swiglu_gate_mb"]) < 0.1


# ---------------------------------------------------------------- quantiser
def _blocks(y):
    q, D, S = oracle.quantize(y)
    return q, D, S


def test_quantize_invariants_random():
    rng = np.random.default_rng(3)
    y = (rng.standard_normal((64, 512)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    q, D, S = _blocks(y)
    yb = y.reshape(64, 16, 32).astype(np.float64)
    qb = q.reshape(64, 16, 32).astype(np.int64)
    assert np.abs(qb).max() <= 127
    assert np.array_equal(qb.sum(-1), S)
    amax = np.abs(yb).max(-1)
    # D is the correctly rounded f32 quotient amax / 127
    Dd = D.astype(np.float64)
    ulp = np.spacing(D).astype(np.float64)
    assert np.all(np.abs(Dd - amax / 127.0) <= 0.5 * ulp)
    # the element of largest magnitude maps to +-127
    idx = np.abs(yb).argmax(-1)
    top = np.take_along_axis(qb, idx[..., None], -1)[..., 0]
    assert np.all(np.abs(top) == 127)
    # every code is the nearest integer to y / D (within the quotient's rounding)
    r = yb / Dd[..., None]
    assert np.all(np.abs(r - qb) <= 0.5 + 1e-5)


def test_quantize_reduction_order_invariance():
    """Permuting a block leaves D and S bit-identical and permutes the codes."""
    rng = np.random.default_rng(4)
    y = rng.standard_normal((8, 256)).astype(np.float32)
    q, D, S = _blocks(y)
    perm = rng.permutation(32)
    yp = y.reshape(8, 8, 32)[:, :, perm].reshape(8, 256)
    qp, Dp, Sp = _blocks(yp)
    assert np.array_equal(D.view(np.uint32), Dp.view(np.uint32))
    assert np.array_equal(S, Sp)
    assert np.array_equal(q.reshape(8, 8, 32)[:, :, perm], qp.reshape(8, 8, 32))


def test_quantize_power_of_two_scaling():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((4, 256)).astype(np.float32)
    q, D, S = _blocks(y)
    for k in (-3, 1, 7):
        q2, D2, S2 = _blocks((y * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(q, q2) and np.array_equal(S, S2)
        assert np.array_equal(D2, (D * np.float32(2.0 ** k)).astype(np.float32))


def test_quantize_ties_round_half_even():
    y = np.zeros((1, 32), np.float32)
    y[0, 0] = 127.0                          # amax = 127 -> D = 1 exactly
    y[0, 1:9] = [2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 126.5]
    q, D, S = _blocks(y)
    assert D[0, 0] == 1.0
    assert list(q[0, :9]) == [127, 2, 4, -2, -4, 0, 2, 0, 126]
    assert S[0, 0] == sum(q[0].astype(int))


def test_quantize_zero_and_single_nonzero_blocks():
    y = np.zeros((2, 64), np.float32)
    y[1, 37] = -0.123
    q, D, S = _blocks(y)
    assert np.all(q[0] == 0) and np.all(D[0] == 0) and np.all(S[0] == 0)
    assert D[1, 0] == 0 and S[1, 0] == 0
    assert q[1, 37] == -127 and np.count_nonzero(q[1]) == 1 and S[1, 1] == -127
    assert D[1, 1] == np.float32(np.float32(0.123) / np.float32(127.0))


def test_quantize_scale_underflow_is_a_zero_block():
    """Deep subnormal blocks: where the IEEE quotient amax / 127 rounds to
    zero (numpy's own float32 division decides it), the block is the all-zero
    block (q = 0, S = 0); one step above, the scale is the smallest subnormal
    and the codes are the clamped quotients."""
    tiny = np.float32(2.0 ** -149)
    y = np.zeros((3, 32), np.float32)
    y[0, 0] = 10 * tiny; y[0, 5] = -3 * tiny             # amax 10 * 2^-149
    y[1, 0] = 63 * tiny; y[1, 1] = -63 * tiny             # the largest amax that underflows
    y[2, 0] = 190 * tiny; y[2, 1] = 64 * tiny; y[2, 2] = -3 * tiny
    amax = np.abs(y).max(-1)
    Dn = amax / np.float32(127.0)
    assert Dn.dtype == np.float32
    assert Dn[0] == 0 and Dn[1] == 0 and Dn[2] == tiny    # 190/127 rounds to one step
    q, D, S = _blocks(y)
    assert np.array_equal(D[:, 0].view(np.uint32), Dn.view(np.uint32))
    assert np.all(q[:2] == 0) and np.all(S[:2, 0] == 0)
    # D = 2^-149: y / D is the integer multiple itself; 190 clamps to 127
    assert list(q[2, :3]) == [127, 64, -3] and np.count_nonzero(q[2]) == 3
    assert S[2, 0] == 127 + 64 - 3
    # a larger value in the same block lifts the whole block out of underflow
    y2 = y[:1].copy(); y2[0, 31] = np.float32(1e-30)
    q2, D2, S2 = _blocks(y2)
    assert D2[0, 0] > 0 and q2[0, 31] == 127 and np.count_nonzero(q2) == 1


def test_quantize_uses_quotient_not_reciprocal():
    """Find values where rint(y * (1/D)) != rint(y / D) and check the oracle
    follows the quotient (the reading of the plain 'y / scale')."""
    rng = np.random.default_rng(6)
    found = 0
    for _ in range(200):
        amax = np.float32(rng.uniform(0.5, 2.0))
        D = np.float32(amax / np.float32(127.0))
        inv = np.float32(np.float32(1.0) / D)
        k = rng.integers(-126, 126)
        base = np.float32((k + 0.5) * np.float64(D))
        for y0 in (np.nextafter(base, np.float32(-10)), base, np.nextafter(base, np.float32(10))):
            y0 = np.float32(y0)
            a = np.rint(np.float32(y0 / D)); b = np.rint(np.float32(y0 * inv))
            if a != b:
                blk = np.zeros((1, 32), np.float32); blk[0, 0] = amax; blk[0, 1] = y0
                q, Dq, _ = _blocks(blk)
                assert Dq[0, 0] == D and q[0, 1] == a
                found += 1
    assert found > 0


# ---------------------------------------------------------------- producers
def test_rmsnorm_closed_forms():
    d = 256
    x = np.zeros((3, d), np.float32)
    x[0] = 3.0; x[1] = -0.25                 # constant rows -> y = sign(c) * c/sqrt(c^2+eps)
    w = np.ones(d, np.float32)
    y = oracle.rmsnorm(x, w, 1e-6)
    assert abs(y[0, 0] - 3.0 / math.sqrt(9.0 + 1e-6)) < 2e-7
    assert abs(y[1, 0] + 0.25 / math.sqrt(0.0625 + 1e-6)) < 2e-7
    assert np.all(y[2] == 0.0)
    q, D, S = oracle.quantize(y)
    assert np.all(q[0] == 127) and np.all(q[1] == -127) and np.all(q[2] == 0)


def test_rmsnorm_structure_random():
    """y_i / (x_i w_i) is one per-row constant s, and mean((y/w)^2) equals
    ms / (ms + eps) with ms = mean(x^2): pins the divisor d, the eps placement
    and the square root."""
    rng = np.random.default_rng(7)
    for d, eps in ((256, 1e-6), (768, 0.5)):
        x = rng.standard_normal((5, d)).astype(np.float32) * np.float32(0.7)
        w = rng.uniform(0.5, 1.5, d).astype(np.float32)
        y = oracle.rmsnorm(x, w, eps).astype(np.float64)
        xd = x.astype(np.float64); wd = w.astype(np.float64)
        s = y / (xd * wd)
        assert np.all(np.abs(s - s[:, :1]) <= 3 * U24 * np.abs(s[:, :1]))
        ms = (xd ** 2).mean(1)
        assert np.allclose(((y / wd) ** 2).mean(1), ms / (ms + eps), rtol=1e-6)


def test_swiglu_special_values():
    g = np.array([[0.0, 1.0, -1.0, 30.0, -30.0, 2.0, 5.0, -7.0]], np.float32)
    u = np.array([[5.0, 1.0, 1.0, 2.0, 3.0, 0.0, -1.0, 1.0]], np.float32)
    y = oracle.swiglu(g, u)[0]
    assert y[0] == 0.0                               # silu(0) = 0
    assert abs(y[1] - 0.7310585786300049) < 1e-7     # sigmoid(1)
    assert abs(y[2] + 0.2689414213699951) < 1e-7     # -sigmoid(-1)
    assert y[3] == 60.0                              # silu(30) rounds to 30 in f32
    assert abs(y[4]) < 1e-11                         # -30 * e^-30 * 3
    assert y[5] == 0.0                               # u = 0


def test_swiglu_odd_identity():
    """silu(x) - silu(-x) = x."""
    rng = np.random.default_rng(8)
    g = rng.standard_normal((4, 256)).astype(np.float32) * 3
    one = np.ones_like(g)
    a = oracle.swiglu(g, one).astype(np.float64)
    b = oracle.swiglu(-g, one).astype(np.float64)
    assert np.allclose(a - b, g.astype(np.float64), rtol=0, atol=4e-6 * (1 + np.abs(g)).max())


# ---------------------------------------------------------------- matmuls
def _plane(rng, n, id_):
    y = rng.standard_normal((n, id_)).astype(np.float32) * rng.uniform(0.1, 3, (n, 1)).astype(np.float32)
    return oracle.quantize(y)


@pytest.mark.parametrize("n,od,id_", [(1, 3, 256), (5, 7, 512), (8, 16, 256)])
def test_gemm_q4k_vs_bruteforce_f64(n, od, id_):
    rng = np.random.default_rng(100 + n)
    raw, w = random_q4k(rng, od, id_)
    Q, D, S = _plane(rng, n, id_)
    a = Q.astype(np.float64) * np.repeat(D.astype(np.float64), 32, axis=1)
    ref = a @ w.T
    got, gmag = oracle.gemm("q4_K", Q, D, S, raw, od, id_, with_mag=True)
    nsb = id_ // 256
    mag = np.zeros_like(ref)
    for o in range(od):
        for s in range(nsb):
            d, dm, sc, mn, q = oracle.q4k_fields(raw[o, s * 144:(s + 1) * 144])
            j = np.arange(256) // 32
            mag[:, o] += np.abs(a[:, s * 256:(s + 1) * 256]) @ (d * sc[j] * q + dm * mn[j])
    # the plain product up to its one f32 rounding (f64 terms round at 2^-53)
    assert np.all(np.abs(got - ref) <= U24 * np.abs(ref) + 2.0 ** -50 * mag + 1e-30)
    # sum |block term| lies between |sum| and the sum of |element products|
    assert np.all(gmag >= np.abs(ref) * (1 - 1e-12)) and np.all(gmag <= mag * (1 + 1e-12))
    # a dropped min term or sign flip would be far outside that bound
    assert np.abs(ref).max() > 1000 * (4 * U24 * mag.max())


@pytest.mark.parametrize("n,od,id_", [(1, 3, 256), (6, 5, 512), (8, 16, 256)])
def test_gemm_q6k_vs_bruteforce_f64(n, od, id_):
    rng = np.random.default_rng(200 + n)
    raw, w = random_q6k(rng, od, id_)
    Q, D, S = _plane(rng, n, id_)
    a = Q.astype(np.float64) * np.repeat(D.astype(np.float64), 32, axis=1)
    ref = a @ w.T
    got, gmag = oracle.gemm("q6_K", Q, D, S, raw, od, id_, with_mag=True)
    mag = np.abs(a) @ np.abs(w).T
    assert np.all(np.abs(got - ref) <= U24 * np.abs(ref) + 2.0 ** -50 * mag + 1e-30)
    assert np.all(gmag >= np.abs(ref) * (1 - 1e-12)) and np.all(gmag <= mag * (1 + 1e-12))


@pytest.mark.parametrize("n,od,id_", [(1, 3, 256), (4, 6, 512), (8, 16, 256)])
def test_gemm_q5k_vs_bruteforce_f64(n, od, id_):
    rng = np.random.default_rng(300 + n)
    raw, w = random_q5k(rng, od, id_)
    Q, D, S = _plane(rng, n, id_)
    a = Q.astype(np.float64) * np.repeat(D.astype(np.float64), 32, axis=1)
    ref = a @ w.T
    got, gmag = oracle.gemm("q5_K", Q, D, S, raw, od, id_, with_mag=True)
    nsb = id_ // 256
    mag = np.zeros_like(ref)
    for o in range(od):
        for s in range(nsb):
            d, dm, sc, mn, q = oracle.q5k_fields(raw[o, s * 176:(s + 1) * 176])
            j = np.arange(256) // 32
            mag[:, o] += np.abs(a[:, s * 256:(s + 1) * 256]) @ (d * sc[j] * q + dm * mn[j])
    assert np.all(np.abs(got - ref) <= U24 * np.abs(ref) + 2.0 ** -50 * mag + 1e-30)
    assert np.all(gmag >= np.abs(ref) * (1 - 1e-12)) and np.all(gmag <= mag * (1 + 1e-12))
    assert np.abs(ref).max() > 1000 * (4 * U24 * mag.max())


def _unit_plane(rng, n, id_):
    """Integer activations with D = 1 exactly: every block holds a +-127."""
    Q = rng.integers(-127, 128, (n, id_)).astype(np.int8)
    Q.reshape(n, -1, 32)[:, :, 0] = 127
    D = np.ones((n, id_ // 32), np.float32)
    S = Q.reshape(n, -1, 32).astype(np.int32).sum(-1).astype(np.int32)
    return Q, D, S


def test_gemm_q4k_integer_special_case():
    """d = dmin = 1, sc = 1: out = Q q^T - Q-block-sums . m exactly (int64)."""
    rng = np.random.default_rng(9)
    n, od, id_ = 7, 9, 512
    Q, D, S = _unit_plane(rng, n, id_)
    nsb = id_ // 256
    raw = np.zeros((od, nsb * 144), np.uint8)
    qall = np.zeros((od, id_), np.int64); mall = np.zeros((od, id_ // 32), np.int64)
    for o in range(od):
        for s in range(nsb):
            q = rng.integers(0, 16, 256); mn = rng.integers(0, 64, 8)
            raw[o, s * 144:(s + 1) * 144] = q4k_encode(0x3C00, 0x3C00, [1] * 8, mn, q)
            qall[o, s * 256:(s + 1) * 256] = q; mall[o, s * 8:(s + 1) * 8] = mn
    ref = Q.astype(np.int64) @ qall.T - S.astype(np.int64) @ mall.T
    got = oracle.gemm("q4_K", Q, D, S, raw, od, id_)
    assert np.array_equal(got.astype(np.int64), ref)
    # the output is [token][output]: a transposed result would not even match in shape
    assert got.shape == (n, od)


def test_gemm_q5k_integer_special_case():
    """d = dmin = 1, sc = 1: out = Q q^T - Q-block-sums . m exactly, with
    5-bit quants (a dropped fifth bit would be off by 16 per set bit)."""
    rng = np.random.default_rng(12)
    n, od, id_ = 5, 7, 512
    Q, D, S = _unit_plane(rng, n, id_)
    nsb = id_ // 256
    raw = np.zeros((od, nsb * 176), np.uint8)
    qall = np.zeros((od, id_), np.int64); mall = np.zeros((od, id_ // 32), np.int64)
    for o in range(od):
        for s in range(nsb):
            q = rng.integers(0, 32, 256); mn = rng.integers(0, 64, 8)
            raw[o, s * 176:(s + 1) * 176] = q5k_encode(0x3C00, 0x3C00, [1] * 8, mn, q)
            qall[o, s * 256:(s + 1) * 256] = q; mall[o, s * 8:(s + 1) * 8] = mn
    ref = Q.astype(np.int64) @ qall.T - S.astype(np.int64) @ mall.T
    got = oracle.gemm("q5_K", Q, D, S, raw, od, id_)
    assert got.shape == (n, od)
    assert np.array_equal(got.astype(np.int64), ref)


def test_gemm_q6k_integer_special_case_and_halves():
    """d = 1: out = sum over 16-halves of sc_half * (Q . (q - 32)) exactly;
    zeroing every second sub-scale isolates the first halves."""
    rng = np.random.default_rng(10)
    n, od, id_ = 6, 5, 512
    Q, D, S = _unit_plane(rng, n, id_)
    nsb = id_ // 256
    for pattern in ("ones", "first_half_only", "random"):
        raw = np.zeros((od, nsb * 210), np.uint8)
        weff = np.zeros((od, id_), np.int64)
        for o in range(od):
            for s in range(nsb):
                q = rng.integers(0, 64, 256)
                if pattern == "ones":
                    sc = np.ones(16, np.int64)
                elif pattern == "first_half_only":
                    sc = np.tile([1, 0], 8)
                else:
                    sc = rng.integers(-128, 128, 16)
                raw[o, s * 210:(s + 1) * 210] = q6k_encode(0x3C00, sc, q)
                weff[o, s * 256:(s + 1) * 256] = sc[np.arange(256) // 16] * (q - 32)
        ref = Q.astype(np.int64) @ weff.T
        got = oracle.gemm("q6_K", Q, D, S, raw, od, id_)
        assert np.array_equal(got.astype(np.int64), ref), pattern


def test_gemm_sampled_equals_full():
    rng = np.random.default_rng(11)
    raw, _ = random_q4k(rng, 12, 256)
    Q, D, S = _plane(rng, 9, 256)
    full = oracle.gemm("q4_K", Q, D, S, raw, 12, 256)
    tok = np.array([8, 0, 3]); outs = np.array([11, 2])
    part = oracle.gemm("q4_K", Q, D, S, raw, 12, 256, tok=tok, outs=outs)
    assert np.array_equal(part, full[np.ix_(tok, outs)])


# ---------------------------------------------------------------- f32-activation GEMV
def test_gemv_f32_closed_forms():
    """Single q6_K superblock rows with every code 33 (weight d*sc*1) or 31
    (weight -d*sc), d = 1 and sub-scales s_h: out = sum_h s_h * sum_{e in h} x_e."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal(256).astype(np.float32)
    sc = [int(v) for v in rng.integers(-128, 128, 16)]
    rows = [q6k_encode(0x3C00, sc, [33] * 256), q6k_encode(0x3C00, sc, [31] * 256)]
    raw = np.stack(rows)
    got = oracle.gemv_f32("q6_K", raw, 2, 256, x)
    halves = [float(np.sum(x[16 * h:16 * h + 16].astype(np.float64))) for h in range(16)]
    want = sum(s * v for s, v in zip(sc, halves))
    assert abs(got[0] - want) <= 1e-9 * (1 + abs(want))
    assert abs(got[1] + want) <= 1e-9 * (1 + abs(want))


def test_gemv_f32_equals_the_integer_dot_path_on_exact_planes():
    """With integer activations whose every 32-block holds +-127, the q8 plane
    is exact (D = 1, q = x), so the integer-dot matmul (its own decode, block
    dots and rescale) and the f32-activation GEMV compute the same sum."""
    rng = np.random.default_rng(12)
    od, id_ = 7, 512
    raw, _ = random_q6k(rng, od, id_)
    x = rng.integers(-127, 128, id_).astype(np.float32)
    x[::32] = 127.0
    Q, D, S = oracle.quantize(x[None, :])
    assert np.all(D == 1.0) and np.array_equal(Q[0].astype(np.float32), x)
    dot = oracle.gemm("q6_K", Q, D, S, raw, od, id_)[0]
    ref = oracle.gemv_f32("q6_K", raw, od, id_, x)
    scale = np.abs(oracle.dequant("q6_K", raw, od, id_)) @ np.abs(x.astype(np.float64))
    assert np.all(np.abs(dot - ref) <= 1e-6 * scale + 1e-30)
