"""GPU parity of the decoder-block pieces around the quantized projections:

* the RMSNorm with the AWQ 1/s folded in (awq_rmsnorm_fold) against the float64 oracle:
  identical fp16 outputs except where the float64 value sits within 1e-9 (relative) of an
  fp16 rounding midpoint, where the two sides may round apart by one ulp because their
  sums of squares are accumulated in different orders;
* q/k/v and gate/up run as one launch over their stacked rows: every output bit-identical
  to the separate launches, and within tolerance of the oracle.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _gpu():
    from tests import _gpu

    return _gpu


def _fold_ref64(h, gamma, s, eps):
    h64 = h.astype(np.float64)
    r = oracle.rms_factor(h, eps)
    v = (h64 * r[:, None]) * gamma.astype(np.float64)[None, :]
    if s is not None:
        v = v / s.astype(np.float64)[None, :]
    return v


def _check_fold(lib, h, gamma, s, eps, tag):
    g = _gpu()
    print(f"rmsnorm-fold {tag} M={h.shape[0]} K={h.shape[1]} fold={s is not None}", flush=True)
    got = g.host(lib.rmsnorm_fold(g.dev(h), g.dev(gamma), None if s is None else g.dev(s), eps))
    want = oracle.rmsnorm_fold(h, gamma, s, eps)
    gb, wb = got.view(np.uint16), want.view(np.uint16)
    diff = np.argwhere(gb != wb)
    if len(diff):
        v = _fold_ref64(h, gamma, s, eps)
        for m, k in diff:
            a, b = float(got[m, k]), float(want[m, k])
            assert abs(int(gb[m, k]) - int(wb[m, k])) == 1, (tag, m, k, a, b)
            mid = (a + b) / 2
            assert abs(v[m, k] - mid) <= 1e-9 * abs(mid), (tag, m, k, v[m, k], a, b)
    return len(diff)


def _block_inputs(cfg, k, m, seed):
    rng = np.random.default_rng(seed)
    h = synth.activations(cfg, seed, m, k)
    gamma = (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float16)
    s = oracle.channel_scale(synth.calibration(cfg, seed, k))
    return h, gamma, s


@pytest.mark.parametrize("cfg,k,m", [(2, 4096, 1), (3, 8192, 1), (2, 4096, 512), (3, 22016, 3), (6, 8, 5), (6, 128, 2)])
def test_rmsnorm_fold_matches_oracle(lib, cfg, k, m):
    h, gamma, s = _block_inputs(cfg, k, m, 5)
    total = h.size
    mism = _check_fold(lib, h, gamma, s, 1e-5, "folded")
    mism += _check_fold(lib, h, gamma, None, 1e-6, "plain")
    assert mism <= max(2, total // 10000)


def test_rmsnorm_fold_edge_rows(lib):
    k = 256
    h = np.zeros((6, k), dtype=np.float16)
    h[1] = 1e-4                                   # mean square far below eps
    h[2] = 60000.0                                # large: float64 keeps the exact square sum
    h[3, ::7] = -3.0                              # sparse row
    h[4] = np.float16(6e-8)                       # subnormal inputs
    h[5] = np.linspace(-50, 50, k).astype(np.float16)
    gamma = np.linspace(0.5, 2.0, k).astype(np.float16)
    s = np.linspace(0.3, 5.0, k).astype(np.float32)
    assert _check_fold(lib, h, gamma, s, 1e-5, "edge") <= 1
    g = _gpu()
    out = g.host(lib.rmsnorm_fold(g.dev(h), g.dev(gamma), g.dev(s), 1e-5))
    assert np.all(out[0].view(np.uint16) == 0)   # a zero row stays exactly zero


@pytest.mark.parametrize("m,k", [(1, 4096), (3, 11008), (70, 2056)])
def test_rmsnorm_fold_unaligned_gamma_and_s(lib, m, k):
    # gamma and s 16-byte aligned take vector loads; at 2 and 4 bytes (the entry's minimum) the
    # kernel loads them element by element: the same bits either way
    import torch

    g = _gpu()
    h, gamma, s = _block_inputs(2, k, m, 11)
    hd = g.dev(h)
    gbig = torch.zeros(k + 1, dtype=torch.float16, device=g.DEV)
    sbig = torch.zeros(k + 1, dtype=torch.float32, device=g.DEV)
    gbig[1:] = g.dev(gamma)
    sbig[1:] = g.dev(s)
    print(f"rmsnorm-fold unaligned M={m} K={k}", flush=True)
    a = g.host(lib.rmsnorm_fold(hd, g.dev(gamma), g.dev(s), 1e-5))
    b = g.host(lib.rmsnorm_fold(hd, gbig[1:], sbig[1:], 1e-5))
    c = g.host(lib.rmsnorm_fold(hd, gbig[1:], None, 1e-5))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(c.view(np.uint16), g.host(lib.rmsnorm_fold(hd, g.dev(gamma), None, 1e-5)).view(np.uint16))
    assert _check_fold(lib, h, gamma, s, 1e-5, "aligned") <= max(2, h.size // 10000)


def _stacked_vs_separate(lib, cfg, names, m):
    g = _gpu()
    layers = {n: (k, nn) for n, k, nn in synth.CONFIGS[cfg]["layers"]}
    k = layers[names[0]][0]
    x_cal = synth.calibration(cfg, 0, k)
    s = oracle.channel_scale(x_cal)
    xs = oracle.scale_input(synth.activations(cfg, 0, m, k), s)
    Ws = [synth.weights(cfg, i, layers[n][1], k) for i, n in enumerate(names)]
    parts = [oracle.quantize_pack(W, s) for W in Ws]
    stacked = [np.concatenate([p[i] for p in parts], axis=0) for i in range(3)]
    x_d = g.dev(xs)
    print(f"stacked {'+'.join(names)} M={m} K={k} N={stacked[0].shape[0]}", flush=True)
    y_all = g.host(lib.linear(x_d, *[g.dev(t) for t in stacked]))
    y_sep = np.concatenate([g.host(lib.linear(x_d, *[g.dev(t) for t in p])) for p in parts], axis=1)
    assert np.array_equal(y_all.view(np.uint16), y_sep.view(np.uint16))
    rows = np.linspace(0, stacked[0].shape[0] - 1, 300).astype(int)
    y_ref, b = oracle.linear(xs, *stacked, rows=rows)
    assert np.all(oracle.within_tolerance(y_all[:, rows].astype(np.float64), y_ref, b))


@pytest.mark.parametrize("m", [1, 4])
def test_qkv_as_one_launch(lib, m):
    _stacked_vs_separate(lib, synth.LLAMA2_7B_BLOCK, ["q", "k", "v"], m)


@pytest.mark.parametrize("m", [1, 4])
def test_gate_up_as_one_launch(lib, m):
    _stacked_vs_separate(lib, synth.LLAMA2_7B_BLOCK, ["gate", "up"], m)
