"""Seeded synthetic inputs for the W4A16 path (shared by tests, smoke and bench).

This module only draws random numbers and arranges them into the workload's
shapes. It holds none of the method's arithmetic: the AWQ scale, the input
fold, quantization and the linear layer live in the oracle (CPU) and in the
HIP library (GPU), never here.

Workload recipe (stand-ins for real checkpoints and calibration data, which
are not available): LLaMA-shaped layers whose weights are N(0, 0.02^2) in fp16
and whose activations are N(0, 1) in fp16 with round(1% of K) seeded outlier
input channels multiplied by 20 - the systematic, fixed-channel outliers the
pages describe ("MIT 6.5940 L13" guide, slides 5-7; "Quantization for LLMs"
section 11.1). Calibration activations have T_cal = 512 rows, the block length
of the Lab 4 calibration setup.

Seeds: numpy PCG64 from SeedSequence([20261203, config_id, layer_id, tensor]).
"""

import numpy as np

SEED_BASE = 20261203
T_CAL = 512
W_STD = 0.02
OUTLIER_FRAC = 0.01
OUTLIER_GAIN = 20.0

# tensor ids inside one layer's seed sequence
_T_W, _T_OUTL, _T_XCAL, _T_X = 0, 1, 2, 3

# The five workloads, each under a named id that also enters the seed sequence of its
# tensors (so the ids keep these values): list of (layer name, K, N) and the M values.
SINGLE_2048 = 1
LLAMA2_7B_BLOCK = 2
LLAMA65B_DECODE = 3
SWEEP_8192 = 4
LLAMA2_7B_SERVING = 5

CONFIGS = {
    SINGLE_2048: {"name": "single layer 2048->2048", "layers": [("single", 2048, 2048)], "M": [1]},
    LLAMA2_7B_BLOCK: {
        "name": "LLaMA2-7B decoder block",
        "layers": [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
                   ("gate", 4096, 11008), ("up", 4096, 11008), ("down", 11008, 4096)],
        "M": [1],
    },
    LLAMA65B_DECODE: {
        "name": "LLaMA-65B decode set",
        "layers": [("q", 8192, 8192), ("k", 8192, 8192), ("v", 8192, 8192), ("o", 8192, 8192),
                   ("gate", 8192, 22016), ("up", 8192, 22016), ("down", 22016, 8192)],
        "M": [1],
    },
    SWEEP_8192: {"name": "small-batch sweep 8192->8192", "layers": [("sweep", 8192, 8192)], "M": [2, 4, 8, 16, 32]},
    LLAMA2_7B_SERVING: {
        "name": "LLaMA2-7B batched serving",
        "layers": [("qkvo", 4096, 4096), ("gate_up", 4096, 11008), ("down", 11008, 4096)],
        "M": [128, 256],
    },
}


def _rng(config_id, layer_id, tensor):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, config_id, layer_id, tensor])))


def outlier_channels(config_id, layer_id, k):
    """round(1% of K) distinct input channels, drawn without replacement."""
    n_out = int(round(OUTLIER_FRAC * k))
    idx = _rng(config_id, layer_id, _T_OUTL).choice(k, size=n_out, replace=False)
    return np.sort(idx)


def weights(config_id, layer_id, n, k):
    """fp16 [N][K] nn.Linear weight, N(0, 0.02^2) drawn in float64 then rounded."""
    return (_rng(config_id, layer_id, _T_W).standard_normal((n, k)) * W_STD).astype(np.float16)


def _activations(config_id, layer_id, tensor, rows, k):
    a = _rng(config_id, layer_id, tensor).standard_normal((rows, k))
    a[:, outlier_channels(config_id, layer_id, k)] *= OUTLIER_GAIN
    return a.astype(np.float16)


def calibration(config_id, layer_id, k, t_cal=T_CAL):
    """fp16 [T_cal][K] calibration activations with the layer's outlier channels."""
    return _activations(config_id, layer_id, _T_XCAL, t_cal, k)


def activations(config_id, layer_id, m, k):
    """fp16 [M][K] decode activations (before the 1/s fold), same outliers."""
    return _activations(config_id, layer_id, _T_X, m, k)


def layer(config_id, layer_id, n, k, m, t_cal=T_CAL):
    """All raw inputs of one layer: dict(W, x_cal, x, outliers)."""
    return {
        "W": weights(config_id, layer_id, n, k),
        "x_cal": calibration(config_id, layer_id, k, t_cal),
        "x": activations(config_id, layer_id, m, k),
        "outliers": outlier_channels(config_id, layer_id, k),
    }


_EDGE_KINDS = {"ties": 1, "constant": 2, "positive": 3, "negative": 4, "subnormal": 5, "wide": 6, "mixed": 7}


def edge_weights(kind, n, k, seed=0):
    """fp16 [N][K] weights that exercise the quantizer's corner cases.

    kinds: 'ties' (values on exact half steps of small dyadic grids),
    'constant' (every group constant, including all-zero rows),
    'positive' / 'negative' (one-signed groups, large |zero|),
    'subnormal' (fp16 subnormal magnitudes), 'wide' (|w| up to 60000),
    'mixed' (a random mix of the above per group).
    """
    if kind not in _EDGE_KINDS:
        raise ValueError(f"unknown edge kind {kind!r}")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, 99, seed, _EDGE_KINDS[kind]])))
    if kind == "ties":
        # integers 0..30 times 2^-e: max - min is often a multiple of 15 steps, so
        # w / Delta lands on exact halves
        e = rng.integers(3, 9, size=(n, k // 128, 1))
        v = rng.integers(-15, 16, size=(n, k // 128, 128)).astype(np.float64) * (0.5 ** e)
        return v.reshape(n, k).astype(np.float16)
    if kind == "constant":
        c = rng.standard_normal((n, k // 128, 1)) * W_STD
        c[0] = 0.0
        return np.broadcast_to(c, (n, k // 128, 128)).reshape(n, k).astype(np.float16)
    if kind == "positive":
        base = rng.uniform(0.5, 2.0, size=(n, k // 128, 1))
        v = base + rng.uniform(0, 1e-2, size=(n, k // 128, 128))
        return v.reshape(n, k).astype(np.float16)
    if kind == "negative":
        base = -rng.uniform(0.5, 2.0, size=(n, k // 128, 1))
        v = base - rng.uniform(0, 1e-2, size=(n, k // 128, 128))
        return v.reshape(n, k).astype(np.float16)
    if kind == "subnormal":
        bits = rng.integers(0, 1024, size=(n, k)).astype(np.uint16)
        sign = (rng.integers(0, 2, size=(n, k)).astype(np.uint16) << 15)
        return (bits | sign).view(np.float16)
    if kind == "wide":
        v = rng.uniform(-60000.0, 60000.0, size=(n, k))
        return v.astype(np.float16)
    if kind == "mixed":
        parts = [edge_weights(kd, n, k, seed) for kd in ("ties", "constant", "positive", "negative", "subnormal", "wide")]
        parts.append(weights(0, seed, n, k))
        pick = rng.integers(0, len(parts), size=(n, k // 128))
        out = np.empty((n, k), dtype=np.float16)
        for i, p in enumerate(parts):
            mask = np.repeat(pick == i, 128, axis=1)
            out[mask] = p[mask]
        return out
    raise ValueError(f"unknown edge kind {kind!r}")
