"""GPU parity of the AWQ scale search (awq_output_reference, awq_alpha_loss and the device
grid search) against the float64 oracle (oracle/search.py).

* The original output y_ref = x W^T is accumulated in float32: each entry within
  1e-5 * sum_k |x w| of the float64 value.

* The loss kernel is fed the oracle's own s, x_s and packed weights, so both sides
  measure the same quantized layer; the device accumulates each product in float32, the
  oracle in float64. Tolerance from that arithmetic: each product of output (t, n) may be
  off by delta = 1e-5 * A[t][n], A the sum of the magnitudes of everything it adds
  (the x_s * q terms, the z * sum x_s terms, the x * w terms; a float32 sum over at most
  a few hundred roundings per output stays far inside it), so with e the exact residual
  the loss may move by at most sum (2 |e| delta + delta^2).
* The device search builds s, x_s and the packed weights with the library's own kernels;
  at alphas other than 0, 0.5 and 1 its s may sit one float32 ulp from the oracle's
  (a different pow), which can move single codes, so the losses are held to a relative
  1e-3 (or the bound above, if larger) and the chosen alpha must be the oracle's or cost
  no more than 1e-3 over it.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

DELTA = 1e-5
RTOL_SEARCH = 1e-3


def _gpu():
    from tests import _gpu

    return _gpu


def _kernel_loss(lib, x_cal, W, alpha):
    """The device loss on the oracle's s, x_s and packed weights."""
    g = _gpu()
    s = oracle.channel_scale(x_cal, alpha)
    xs = oracle.scale_input(x_cal, s)
    q, sc, z = oracle.quantize_pack(W, s)
    y_ref = lib.output_reference(g.dev(x_cal), g.dev(W))
    out = lib.alpha_loss(g.dev(xs), g.dev(q), g.dev(sc), g.dev(z), y_ref)
    return float(g.host(out)[0])


@pytest.mark.parametrize("t_cal,n,k", [(64, 128, 128), (100, 200, 384), (7, 130, 11008), (512, 4096, 4096),
                                       (65, 129, 256), (1, 1, 128)])
def test_output_reference_matches_oracle(lib, t_cal, n, k):
    g = _gpu()
    W = synth.weights(2, 4, n, k)
    x_cal = synth.calibration(2, 4, k, t_cal)
    print(f"output-reference T={t_cal} N={n} K={k}", flush=True)
    got = g.host(lib.output_reference(g.dev(x_cal), g.dev(W))).astype(np.float64)
    x64, w64 = x_cal.astype(np.float64), W.astype(np.float64)
    want = x64 @ w64.T
    bound = DELTA * (np.abs(x64) @ np.abs(w64).T)
    assert np.all(np.abs(got - want) <= bound), float(np.max(np.abs(got - want) / np.maximum(bound, 1e-300)))


def _loss_bound(x_cal, W, alpha):
    """sum over (t, n) of 2 |e| delta + delta^2 with delta = DELTA * A (module docstring)."""
    k = W.shape[1]
    s = oracle.channel_scale(x_cal, alpha)
    xs = oracle.scale_input(x_cal, s).astype(np.float64)
    q, sc, z = oracle.quantize_pack(W, s)
    codes = oracle.unpack_codes(q, k).astype(np.float64)
    d = np.repeat(sc.astype(np.float64), 128, axis=1)
    zr = np.repeat(np.abs(z.astype(np.float64)), 128, axis=1)
    x64, w64 = x_cal.astype(np.float64), W.astype(np.float64)
    a = np.abs(xs) @ (codes * d).T + np.abs(xs) @ (zr * d).T + np.abs(x64) @ np.abs(w64).T
    e = xs @ oracle.dequantize(q, sc, z, k).T - x64 @ w64.T
    delta = DELTA * a
    return float((2 * np.abs(e) * delta + delta * delta).sum())


def _check_kernel(lib, x_cal, W, alphas, tag, resolvable=True):
    for a in alphas:
        print(f"alpha-loss {tag} T={x_cal.shape[0]} N={W.shape[0]} K={W.shape[1]} alpha={a}", flush=True)
        got = _kernel_loss(lib, x_cal, W, a)
        want = oracle.alpha_loss(x_cal, W, a)
        bound = _loss_bound(x_cal, W, a)
        if resolvable:  # the tolerance stays well below the quantity being measured
            assert bound < 0.1 * want, (tag, a, bound, want)
        assert abs(got - want) <= bound, (tag, a, got, want, bound)


@pytest.mark.parametrize("t_cal,n,k", [(64, 64, 128), (100, 200, 384), (512, 320, 2048), (1, 1, 128),
                                       (65, 63, 256), (7, 130, 11008)])
def test_alpha_loss_matches_oracle(lib, t_cal, n, k):
    W = synth.weights(2, 1, n, k)
    x_cal = synth.calibration(2, 1, k, t_cal)
    _check_kernel(lib, x_cal, W, (0.0, 0.35, 0.5, 1.0), "small")


@pytest.mark.parametrize("kind", ["positive", "negative", "mixed", "constant", "ties"])
def test_alpha_loss_edge_weights(lib, kind):
    # one-signed groups give zeros far outside the code range, handled by the same route; there
    # the residual can be small next to outputs whose float32 sums are large, so the bound may
    # exceed the loss itself (float32 cannot resolve it): only the bound is checked
    W = synth.edge_weights(kind, 96, 512)
    x_cal = synth.calibration(1, 2, 512, 80)
    _check_kernel(lib, x_cal, W, (0.0, 0.5), kind, resolvable=False)


def test_alpha_loss_full_layer(lib):
    # a LLaMA2-7B q projection at its full size, 512 calibration tokens
    W = synth.weights(2, 0, 4096, 4096)
    x_cal = synth.calibration(2, 0, 4096)
    _check_kernel(lib, x_cal, W, (0.5,), "q-proj")


def test_alpha_loss_is_reproducible_and_zero_for_exact_weights(lib):
    g = _gpu()
    W = synth.weights(1, 3, 200, 1024)
    x_cal = synth.calibration(1, 3, 1024, 300)
    a = _kernel_loss(lib, x_cal, W, 0.5)
    b = _kernel_loss(lib, x_cal, W, 0.5)
    assert a == b
    # weights already on their grid: every group holds (q - z0) * 2^-6 with codes 0 and 15
    # present, so quantization gives back the same weights; at s = 1 the loss is the float32
    # rounding of two equal products, zero up to that rounding
    rng = np.random.default_rng(11)
    n, k = 200, 1024
    q = rng.integers(0, 16, size=(n, k))
    q[:, 0::128] = 0
    q[:, 1::128] = 15
    z0 = np.repeat(rng.integers(0, 16, size=(n, k // 128)), 128, axis=1)
    w_grid = ((q - z0) * 2.0 ** -6).astype(np.float16)
    qp, sc, z = oracle.quantize_pack(w_grid, None)
    assert np.array_equal(oracle.dequantize(qp, sc, z, k), w_grid.astype(np.float64))
    xs = oracle.scale_input(x_cal, np.ones(k, np.float32))
    y_ref = lib.output_reference(g.dev(x_cal), g.dev(w_grid))
    out = lib.alpha_loss(g.dev(xs), g.dev(qp), g.dev(sc), g.dev(z), y_ref)
    loss0 = float(g.host(out)[0])
    y = x_cal.astype(np.float64) @ w_grid.astype(np.float64).T
    assert loss0 <= 1e-9 * float((y * y).sum()), loss0


@pytest.mark.parametrize("layer", ["q", "down"])
def test_search_alpha_matches_oracle(lib, layer):
    g = _gpu()
    k, n = {"q": (4096, 512), "down": (11008, 256)}[layer]
    W = synth.weights(2, 6, n, k)
    x_cal = synth.calibration(2, 6, k)
    print(f"search {layer} T={x_cal.shape[0]} N={n} K={k}", flush=True)
    losses_d, best_d, alpha_d, s_d = lib.search_alpha(g.dev(x_cal), g.dev(W))
    losses = g.host(losses_d)
    best = int(g.host(best_d)[0])
    want, want_best = oracle.search_alpha(x_cal, W)
    tol = np.array([max(RTOL_SEARCH * w, _loss_bound(x_cal, W, a)) for w, a in zip(want, oracle.ALPHA_GRID)])
    assert np.all(np.abs(losses - want) <= tol), (losses, want)
    grid = list(oracle.ALPHA_GRID)
    # the device's own choice is the first minimum of its own losses
    assert best == int(np.argmin(losses)) and float(g.host(alpha_d)[0]) == grid[best]
    assert want[best] <= want.min() * (1 + RTOL_SEARCH), (grid[best], want_best)
    # the chosen scale is the oracle's channel scale at the chosen alpha, bit for bit
    assert np.array_equal(g.host(s_d).view(np.uint32), oracle.channel_scale(x_cal, grid[best]).view(np.uint32))
    if grid[best] != want_best:
        print(f"chosen alpha {grid[best]} vs oracle {want_best}: losses {want[best]} vs {want.min()}")


def test_search_alpha_equals_the_steps_one_by_one(lib):
    """awq_search_alpha runs the same kernels as the separate calls: its losses are bit-identical
    to output_reference, then per alpha channel_scale, scale_input, quantize_pack, alpha_loss."""
    import torch

    g = _gpu()
    k, n = 2048, 300
    W = g.dev(synth.weights(2, 7, n, k))
    x_cal = g.dev(synth.calibration(2, 7, k))
    losses_d, best_d, alpha_d, s_d = lib.search_alpha(x_cal, W)
    y_ref = lib.output_reference(x_cal, W)
    step = torch.empty(21, dtype=torch.float64, device=x_cal.device)
    for i in range(21):
        s = lib.channel_scale(x_cal, i / 20)
        xs = lib.scale_input(x_cal, s)
        lib.alpha_loss(xs, *lib.quantize_pack(W, s), y_ref, out=step[i:i + 1])
    assert np.array_equal(g.host(losses_d).view(np.uint64), g.host(step).view(np.uint64))
    best = int(g.host(best_d)[0])
    assert np.array_equal(g.host(s_d).view(np.uint32), g.host(lib.channel_scale(x_cal, best / 20)).view(np.uint32))


def test_search_alpha_first_minimum_on_ties(lib):
    """Equal losses keep the smaller alpha: with W = 0 every candidate's loss is exactly 0, so
    the choice is alpha = 0 and the copied scale is all ones."""
    g = _gpu()
    k, n = 256, 40
    W = np.zeros((n, k), dtype=np.float16)
    x_cal = synth.calibration(2, 8, k)
    losses_d, best_d, alpha_d, s_d = lib.search_alpha(g.dev(x_cal), g.dev(W))
    assert np.all(g.host(losses_d) == 0.0)
    assert int(g.host(best_d)[0]) == 0 and float(g.host(alpha_d)[0]) == 0.0
    assert np.all(g.host(s_d) == 1.0)
