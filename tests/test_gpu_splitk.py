"""GPU parity of the split-K MFMA GEMM (w4a16_linear_splitk) against the float64 oracle: every
output within 1e-3 * sum_k |x * w_hat| + 1e-5, on ragged shapes, every split count, the
serving shapes (LLaMA2-7B projections at M = 128 and 256), zeros outside the exact fp16
range (the general route), and run-to-run reproducibility."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _gpu():
    from tests import _gpu

    return _gpu


def _check(lib, x, packed, splits, tag, rows=None):
    g = _gpu()
    m, k = x.shape
    n = packed[0].shape[0]
    print(f"split-K {tag} M={m} N={n} K={k} splits={splits}", flush=True)
    y = g.host(lib.linear_splitk(g.dev(x), *[g.dev(t) for t in packed], splits=splits))
    y_ref, b = oracle.linear(x, *packed, rows=rows)
    if rows is not None:
        y = y[:, rows]
    ok = oracle.within_tolerance(y.astype(np.float64), y_ref, b)
    assert np.all(ok), (tag, np.argwhere(~ok)[:3])
    return y


@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (33, 97, 384), (64, 128, 1024), (65, 129, 1408), (100, 300, 2048),
                                   (128, 200, 11008), (257, 64, 4096)])
@pytest.mark.parametrize("splits", [0, 1, 2, 3, 5])
def test_splitk_ragged_shapes(lib, m, n, k, splits):
    if splits > k // 128:
        pytest.skip("more splits than groups")
    s = oracle.channel_scale(synth.calibration(5, 1, k))
    packed = oracle.quantize_pack(synth.weights(5, 1, n, k), s)
    x = oracle.scale_input(synth.activations(5, 1, m, k), s)
    _check(lib, x, packed, splits, "ragged")


@pytest.mark.parametrize("m", [128, 256])
def test_splitk_serving_shapes(lib, m):
    g = _gpu()
    for lid, (name, k, n) in enumerate(synth.CONFIGS[synth.LLAMA2_7B_SERVING]["layers"]):
        s = oracle.channel_scale(synth.calibration(5, lid, k))
        W = synth.weights(5, lid, n, k)
        packed = tuple(g.host(t) for t in lib.quantize_pack(g.dev(W), g.dev(s)))
        packed = (packed[0].view(np.uint32), packed[1], packed[2])
        x = oracle.scale_input(synth.activations(5, lid, m, k), s)
        rows = np.linspace(0, n - 1, 256).astype(int)
        for splits in (0, 4, 16):
            _check(lib, x, packed, splits, name, rows=rows)


@pytest.mark.parametrize("kind", ["positive", "negative", "mixed", "wide"])
def test_splitk_edge_weights(lib, kind):
    W = synth.edge_weights(kind, 96, 1024, seed=13)
    packed = oracle.quantize_pack(W, None)
    x = synth.activations(1, 14, 80, 1024)
    for splits in (1, 3, 8):
        _check(lib, x, packed, splits, kind)


def test_splitk_is_reproducible_and_matches_tiled_within_tolerance(lib):
    g = _gpu()
    k, n, m = 4096, 512, 128
    s = oracle.channel_scale(synth.calibration(5, 9, k))
    packed = oracle.quantize_pack(synth.weights(5, 9, n, k), s)
    x = oracle.scale_input(synth.activations(5, 9, m, k), s)
    xd, dev = g.dev(x), [g.dev(t) for t in packed]
    y1 = g.host(lib.linear_splitk(xd, *dev, splits=4))
    y2 = g.host(lib.linear_splitk(xd, *dev, splits=4))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    y_ref, b = oracle.linear(x, *packed)
    yt = g.host(lib.linear(xd, *dev, path=2))
    assert np.all(oracle.within_tolerance(yt.astype(np.float64), y_ref, b))
    assert np.all(oracle.within_tolerance(y1.astype(np.float64), y_ref, b))
