"""The seeded generator: reproducible, the stated shapes and distributions."""

import numpy as np
import pytest

import synth


def test_reproducible():
    a = synth.layer(1, 0, 64, 2048, 2)
    b = synth.layer(1, 0, 64, 2048, 2)
    for key in a:
        assert np.array_equal(a[key], b[key])
    c = synth.layer(1, 1, 64, 2048, 2)
    assert not np.array_equal(a["W"], c["W"])


@pytest.mark.parametrize("k,count", [(2048, 20), (4096, 41), (8192, 82), (11008, 110), (22016, 220)])
def test_outlier_count(k, count):
    idx = synth.outlier_channels(3, 0, k)
    assert idx.size == count and np.unique(idx).size == count and idx.max() < k


def test_distributions():
    w = synth.weights(2, 0, 512, 4096).astype(np.float64)
    assert abs(w.std() - 0.02) < 2e-4 and abs(w.mean()) < 2e-4
    x = synth.calibration(2, 0, 4096).astype(np.float64)
    out = synth.outlier_channels(2, 0, 4096)
    normal = np.setdiff1d(np.arange(4096), out)
    assert abs(x[:, normal].std() - 1.0) < 0.01
    assert abs(x[:, out].std() - 20.0) < 0.5
    assert x.shape == (512, 4096)


def test_configs_shapes():
    assert synth.CONFIGS[synth.LLAMA65B_DECODE]["layers"][0] == ("q", 8192, 8192)
    for cfg in synth.CONFIGS.values():
        for _, k, n in cfg["layers"]:
            assert k % 128 == 0 and n > 0


@pytest.mark.parametrize("kind", ["ties", "constant", "positive", "negative", "subnormal", "wide", "mixed"])
def test_edge_kinds_finite(kind):
    w = synth.edge_weights(kind, 8, 512, seed=2)
    assert w.dtype == np.float16 and w.shape == (8, 512) and np.all(np.isfinite(w))
