"""Pins for the RMSNorm-with-1/s-fold oracle (oracle/norm.py, reading R13), independent of
the oracle's own float64 chain: exact rationals with a high-precision square root, closed
forms, and invariants the definition fixes."""

from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle.norm as on
from tests.test_oracle import _f16_to_fraction, _half_bits_exact


def _exact_fold(h_row, gamma, s, eps):
    """The exact value ((h * r) * gamma) / s with r = 1 / sqrt(mean h^2 + eps), as Fractions
    (the square root to 80 significant digits)."""
    hs = [Fraction(float(v)) for v in h_row]
    ms = sum(v * v for v in hs) / len(hs) + Fraction(float(eps))
    getcontext().prec = 80
    sq = Fraction((Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt())
    out = []
    for k, v in enumerate(hs):
        val = v * Fraction(float(gamma[k])) / sq
        if s is not None:
            val /= Fraction(float(np.float32(s[k])))
        out.append(val)
    return out


def _check_against_exact(h, gamma, s, eps):
    got = on.rmsnorm_fold(h, gamma, s, eps).view(np.uint16)
    mismatches = 0
    for m in range(h.shape[0]):
        exact = _exact_fold(h[m], gamma, s, eps)
        for k, v in enumerate(exact):
            want = _half_bits_exact(v)
            if int(got[m, k]) == want:
                continue
            # allowed only at a rounding near-tie: v within 1e-12 (relative) of the midpoint
            a, b = _f16_to_fraction(int(got[m, k])), _f16_to_fraction(want)
            mid = (a + b) / 2
            assert abs(int(got[m, k]) - want) == 1 or abs(a - b) < Fraction(1, 2 ** 20), (m, k)
            assert abs(v - mid) <= abs(mid) * Fraction(1, 10 ** 12), (m, k, float(v), float(a), float(b))
            mismatches += 1
    return mismatches


@pytest.mark.parametrize("k", [1, 8, 33, 128])
def test_matches_exact_rational_value(k):
    rng = np.random.default_rng(100 + k)
    h = (rng.standard_normal((3, k)) * 2.0).astype(np.float16)
    h[1, : max(1, k // 4)] *= 30          # outlier channels
    h[2] = (h[2].astype(np.float64) * 1e-3).astype(np.float16)   # mean h^2 ~ eps: eps changes the result
    gamma = (1.0 + 0.3 * rng.standard_normal(k)).astype(np.float16)
    s = (0.5 + rng.random(k) * 4).astype(np.float32)
    assert _check_against_exact(h, gamma, s, 1e-6) <= 1
    assert _check_against_exact(h, gamma, None, 1e-5) <= 1


def test_constant_row_closed_form():
    # eps = 0, h = c: r = 1/|c|, so the output is sign(c) * gamma / s, exact for powers of two
    k = 16
    gamma = np.array([2.0 ** (i % 5 - 2) for i in range(k)], dtype=np.float16)
    s = np.array([2.0 ** (i % 3) for i in range(k)], dtype=np.float32)
    for c in (0.75, -3.0, 1e-3, 300.0):
        h = np.full((1, k), c, dtype=np.float16)
        got = on.rmsnorm_fold(h, gamma, s, 0.0).astype(np.float64)[0]
        np.testing.assert_array_equal(got, np.sign(c) * gamma.astype(np.float64) / s.astype(np.float64))


def test_zero_row_gives_zero():
    h = np.zeros((2, 64), dtype=np.float16)
    out = on.rmsnorm_fold(h, np.ones(64, np.float16), np.full(64, 3.0, np.float32), 1e-6)
    assert np.all(out.view(np.uint16) == 0)


def test_power_of_two_input_scaling_is_invisible_without_eps():
    rng = np.random.default_rng(7)
    h = rng.standard_normal((4, 96)).astype(np.float16)
    gamma = rng.standard_normal(96).astype(np.float16)
    s = (0.7 + rng.random(96)).astype(np.float32)
    base = on.rmsnorm_fold(h, gamma, s, 0.0).view(np.uint16)
    tried = 0
    for e in (-6, -2, -1, 3, 7):
        scaled = (h.astype(np.float64) * 2.0 ** e).astype(np.float16)
        if not np.array_equal(scaled.astype(np.float64), h.astype(np.float64) * 2.0 ** e):
            continue  # the scaled input is not exact in fp16 (subnormal or overflow): not the same input
        assert np.array_equal(on.rmsnorm_fold(scaled, gamma, s, 0.0).view(np.uint16), base), e
        tried += 1
    assert tried >= 3


def test_fold_by_power_of_two_scale_divides_the_plain_norm():
    # with s a power of two per channel, folding 1/s is an exact division of the unfolded output
    rng = np.random.default_rng(8)
    h = rng.standard_normal((3, 80)).astype(np.float16)
    gamma = (0.5 + rng.random(80)).astype(np.float16)
    s = (2.0 ** rng.integers(-2, 4, size=80)).astype(np.float32)
    folded = on.rmsnorm_fold(h, gamma, s, 1e-6).astype(np.float64)
    plain = on.rmsnorm_fold(h, gamma, None, 1e-6).astype(np.float64)
    np.testing.assert_array_equal(folded, plain / s.astype(np.float64))


def test_mean_square_of_the_plain_norm_is_gamma_weighted_one():
    # with gamma = 1 and eps = 0, sum_k y^2 / K = 1 up to the fp16 rounding of y
    rng = np.random.default_rng(9)
    h = rng.standard_normal((5, 512)).astype(np.float16)
    y = on.rmsnorm_fold(h, np.ones(512, np.float16), None, 0.0).astype(np.float64)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=2e-3)
