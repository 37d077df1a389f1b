"""Pins for the symmetric absmax and NF4 oracles (oracle/sym.py, oracle/nf4.py; readings R15,
R16), independent of the oracles' own arithmetic: printed values, brute force in exact
rationals, invariants and the page's 8-bit quantizer."""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN_NF4 = os.path.join(os.path.dirname(__file__), "golden", "nf4_levels.txt")
RNG = np.random.default_rng(31)


# ---------------------------------------------------------------- symmetric absmax
@pytest.mark.parametrize("bits,group", [(4, 4), (4, 16), (3, 8), (3, 16)])
def test_sym_picks_nearest_symmetric_level(bits, group):
    n, g = 16, 5
    w = RNG.standard_normal((n, g * group)) * 0.02
    w[0, :group] = np.linspace(-1, 1, group)
    w[1, :group] = np.abs(w[1, :group]) + 0.5   # one-signed: the symmetric range is half used
    w[2, :group] = 0.0                           # zero group
    q, delta = oracle.quantize_groups_sym(w, bits, group)
    qm = 2 ** (bits - 1) - 1
    for r in range(n):
        for gi in range(g):
            sl = w[r, gi * group:(gi + 1) * group]
            m = max(abs(Fraction(float(v))) for v in sl) or Fraction(1)
            d = Fraction(float(delta[r, gi]))
            assert abs(d - m / qm) <= m / qm * Fraction(2) ** -52  # Delta = m / Q, correctly rounded
            for c, v in enumerate(sl):
                x = Fraction(float(v))
                dist = [abs(x - lv * d) for lv in range(-qm, qm + 1)]
                best = min(dist)
                winners = [lv for lv, dd in zip(range(-qm, qm + 1), dist) if dd == best]
                got = int(q[r, gi * group + c])
                if got not in winners:  # only at an exact-rounding tie of w / Delta
                    t = x / d
                    assert abs(t - (t.numerator // t.denominator) - Fraction(1, 2)) <= abs(t) * Fraction(2) ** -50


def test_sym_extremes_oddness_and_zero_group():
    w = RNG.standard_normal((8, 256)) * 0.05
    w[3, :128] = 0.0
    for bits in (3, 4):
        qm = 2 ** (bits - 1) - 1
        q, delta = oracle.quantize_groups_sym(w, bits, 128)
        qn, dn = oracle.quantize_groups_sym(-w, bits, 128)
        assert np.array_equal(qn, -q) and np.array_equal(dn, delta)  # odd symmetry
        wg, qg = w.reshape(8, 2, 128), q.reshape(8, 2, 128)
        arg = np.abs(wg).argmax(axis=2)
        top = np.take_along_axis(qg, arg[:, :, None], 2)[:, :, 0]
        sign = np.sign(np.take_along_axis(wg, arg[:, :, None], 2)[:, :, 0])
        nz = np.abs(wg).max(axis=2) > 0
        assert np.all(top[nz] == (sign * qm)[nz])  # the largest magnitude sits on the range end
        assert np.all(q[3, :128] == 0) and delta[3, 0] == 1.0 / qm


def _absmax_int8_from_description(x):
    """The guide's absmax quantizer (L19): scale = 127 / max|X|, codes = round(scale * X)."""
    scale = 127.0 / np.max(np.abs(x))
    return np.rint(scale * x)


def test_sym_eight_bit_case_matches_page_absmax_quantizer():
    diff = total = 0
    for _ in range(40):
        r = RNG.standard_normal(512) * RNG.uniform(0.01, 3.0)
        q, _ = oracle.quantize_groups_sym(r[None, :], bits=8, group=r.size)
        page = _absmax_int8_from_description(r)
        d = np.abs(q[0] - page)
        assert d.max() <= 1  # the two float paths (w / (m / 127) vs (127 / m) w) may differ at ties
        diff += int((d != 0).sum())
        total += r.size
    assert diff / total <= 1e-3


@pytest.mark.parametrize("bits", [3, 4])
def test_sym_pack_stores_offset_codes_and_fixed_zero(bits):
    import synth

    W = synth.weights(1, 11, 24, 512)
    s = (0.5 + RNG.random(512)).astype(np.float32)
    qw, sc, zr = oracle.quantize_pack_sym(W, s, bits=bits, group=128)
    q, delta = oracle.quantize_groups_sym(W.astype(np.float64) * s.astype(np.float64), bits, 128)
    assert np.all(zr.astype(np.float64) == 2 ** (bits - 1))
    w_hat = oracle.dequantize(qw, sc, zr, 512, 128, bits)
    assert np.array_equal(w_hat, q * np.repeat(sc.astype(np.float64), 128, axis=1))


# ---------------------------------------------------------------- NF4
def test_nf4_levels_match_the_printed_table():
    printed = np.array([float(l) for l in open(GOLDEN_NF4) if l.strip() and not l.startswith("#")])
    assert printed.size == 16
    assert np.all(np.abs(oracle.NF4_LEVELS - printed) <= 5e-5)
    lv = oracle.NF4_LEVELS
    assert np.all(np.diff(lv) > 0)
    assert lv[0] == -1.0 and lv[-1] == 1.0 and lv[7] == 0.0
    assert (lv > 0).sum() == 8 and (lv < 0).sum() == 7
    # the fp16 codebook is the correctly rounded fp16 of each level
    for a, b in zip(oracle.NF4_LEVELS, oracle.NF4_LEVELS_F16):
        assert abs(float(b) - a) <= np.spacing(np.float16(b)) / 2


def test_nf4_codes_pick_the_nearest_level_brute_force():
    v = np.concatenate([RNG.uniform(-1, 1, 4000), oracle.NF4_LEVELS_F16.astype(np.float64), [-1.0, 1.0, 0.0]])
    lv = [Fraction(float(x)) for x in oracle.NF4_LEVELS_F16]
    mids = [(a + b) / 2 for a, b in zip(lv[:-1], lv[1:])]
    v = np.concatenate([v, [float(m) for m in mids]])  # exact midpoints: ties go to the larger level
    codes = oracle.nf4_codes(v)
    for x, c in zip(v, codes):
        fx = Fraction(float(x))
        dist = [abs(fx - l) for l in lv]
        best = min(dist)
        winners = [i for i, d in enumerate(dist) if d == best]
        assert int(c) == max(winners), (x, c, winners)


def test_nf4_quantize_extremes_round_trip_and_zero_block():
    import synth

    W = synth.weights(1, 12, 16, 256)
    W[2, 64:128] = 0
    codes, a = oracle.quantize_nf4(W, None, 64)
    wg = W.astype(np.float64).reshape(16, 4, 64)
    cg = codes.reshape(16, 4, 64)
    arg = np.abs(wg).argmax(axis=2)
    ext = np.take_along_axis(cg, arg[:, :, None], 2)[:, :, 0]
    nz = a > 0
    assert np.all(np.isin(ext[nz], [0, 15]))  # the largest magnitude maps to level -1 or +1
    assert a[2, 1] == 0 and np.all(cg[2, 1] == 7)
    assert np.all(a.astype(np.float64) == np.abs(wg).max(axis=2).astype(np.float32))
    # weights that are codebook levels times a power of two (exact in fp16), each block holding
    # a level of magnitude 1: quantizing returns those codes and that absmax, and dequantizing
    # returns the weights
    c = RNG.integers(0, 16, size=(8, 256))
    c[:, ::64] = 15
    scale = 2.0 ** RNG.integers(-8, -2, size=(8, 4))
    Wl = (oracle.NF4_LEVELS_F16.astype(np.float64)[c] * np.repeat(scale, 64, axis=1)).astype(np.float16)
    codes2, a2 = oracle.quantize_nf4(Wl, None, 64)
    assert np.array_equal(codes2, c) and np.array_equal(a2.astype(np.float64), scale)
    qw2, _ = oracle.quantize_pack_nf4(Wl, None, 64)
    assert np.array_equal(oracle.dequantize_nf4(qw2, a2, 256, 64), Wl.astype(np.float64))


def test_nf4_linear_matches_exact_rationals():
    import synth

    k, n, m = 128, 4, 2
    W = synth.weights(1, 13, n, k)
    x = synth.activations(1, 13, m, k)
    qw, a = oracle.quantize_pack_nf4(W, None, 64)
    y, b = oracle.linear_nf4(x, qw, a, 64)
    codes = oracle.unpack_codes(qw, k)
    lv = [Fraction(float(v)) for v in oracle.NF4_LEVELS_F16]
    for i in range(m):
        for r in range(n):
            ex = sum(Fraction(float(x[i, c])) * lv[codes[r, c]] * Fraction(float(a[r, c // 64])) for c in range(k))
            assert abs(Fraction(float(y[i, r])) - ex) <= Fraction(k) * Fraction(2) ** -52 * Fraction(float(b[i, r]))
