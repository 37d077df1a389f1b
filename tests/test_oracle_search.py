"""Pins for the AWQ alpha-search loss (oracle/search.py, reading R14)."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.search as osr
import synth


def test_grid_is_the_stated_one():
    assert len(osr.GRID) == 21 and osr.GRID[0] == 0.0 and osr.GRID[-1] == 1.0
    assert all(abs(b - a - 0.05) < 1e-12 for a, b in zip(osr.GRID, osr.GRID[1:]))


def test_loss_matches_exact_rational_sum_on_a_small_case():
    # the quantizer (already pinned) supplies x_s and w_hat; this checks the loss itself:
    # both products, their difference and the squared norm, in exact rationals
    rng = np.random.default_rng(3)
    t, n, k = 3, 2, 256
    x = rng.standard_normal((t, k)).astype(np.float16)
    x[:, 5] *= 20
    W = (rng.standard_normal((n, k)) * 0.02).astype(np.float16)
    for alpha in (0.0, 0.35, 1.0):
        s = oracle.channel_scale(x, alpha)
        xs = oracle.scale_input(x, s)
        w_hat = oracle.dequantize(*oracle.quantize_pack(W, s), k)
        total = Fraction(0)
        for ti in range(t):
            for ni in range(n):
                acc = Fraction(0)
                for ki in range(k):
                    acc += Fraction(float(xs[ti, ki])) * Fraction(float(w_hat[ni, ki]))
                    acc -= Fraction(float(x[ti, ki])) * Fraction(float(W[ni, ki]))
                total += acc * acc
        got = osr.alpha_loss(x, W, alpha)
        assert abs(Fraction(got) - total) <= total * Fraction(1, 10 ** 9), alpha


def test_weights_on_their_own_grid_give_zero_loss_at_alpha_zero():
    # every group already holds exact multiples of a power-of-two step from 0: with s = 1 the
    # quantizer reproduces W, x_s = x, so the output error is exactly 0
    rng = np.random.default_rng(4)
    n, k = 4, 256
    step = 2.0 ** -6
    codes = rng.integers(0, 16, size=(n, k))
    codes[:, ::128] = 0
    codes[:, 1::128] = 15
    W = (codes * step).astype(np.float16)
    x = rng.standard_normal((5, k)).astype(np.float16)
    assert osr.alpha_loss(x, W, 0.0) == 0.0


def test_scaling_salient_channels_lowers_the_output_error():
    # the pages' claim (L13 AWQ section; chapter 11): with activation outlier channels,
    # s = s_X^0.5 gives a smaller output error than plain round-to-nearest (alpha = 0)
    x_cal = synth.calibration(2, 0, 1024)[:128]
    W = synth.weights(2, 0, 96, 1024)
    l0 = osr.alpha_loss(x_cal, W, 0.0)
    l5 = osr.alpha_loss(x_cal, W, 0.5)
    assert l5 < 0.8 * l0


def test_search_returns_the_first_minimum():
    x_cal = synth.calibration(2, 1, 512)[:64]
    W = synth.weights(2, 1, 48, 512)
    grid = (0.0, 0.5, 0.5, 1.0)
    losses, best = osr.search_alpha(x_cal, W, grid)
    assert losses[1] == losses[2]
    assert best == grid[int(np.argmin(losses))]
    np.testing.assert_array_equal(losses, [osr.alpha_loss(x_cal, W, a) for a in grid])
