"""GPU parity of the AWQ statistic, the 1/s fold and quantize-pack: bit-exact
against the CPU oracle on every config's layer shapes and the edge tensors."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _gpu():
    from tests import _gpu

    return _gpu


def _qp_compare(lib, W, s, rows=None):
    g = _gpu()
    qw_d, sc_d, zr_d = lib.quantize_pack(g.dev(W), None if s is None else g.dev(s))
    qw, sc, zr = g.host_u32(qw_d), g.bits16(g.host(sc_d)), g.bits16(g.host(zr_d))
    if rows is not None:
        qw, sc, zr = qw[rows], sc[rows], zr[rows]
        W = W[rows]
    qo, so, zo = oracle.quantize_pack(W, s)
    assert np.array_equal(qw, qo), g.report_mismatch("qweight", qw, qo)
    assert np.array_equal(sc, g.bits16(so)), g.report_mismatch("scales", sc, g.bits16(so))
    assert np.array_equal(zr, g.bits16(zo)), g.report_mismatch("zeros", zr, g.bits16(zo))


@pytest.mark.parametrize("cfg", [synth.SINGLE_2048, synth.LLAMA2_7B_BLOCK])
def test_quantize_pack_full_layers(lib, cfg):
    for layer_id, (name, k, n) in enumerate(synth.CONFIGS[cfg]["layers"]):
        if cfg == synth.LLAMA2_7B_BLOCK and name in ("k", "v", "o", "up"):
            continue  # same shapes as q / gate
        print(f"workload {synth.CONFIGS[cfg]['name']} layer {name} K={k} N={n}", flush=True)
        L = synth.layer(cfg, layer_id, n, k, 1)
        s = oracle.channel_scale(L["x_cal"])
        _qp_compare(lib, L["W"], s)


@pytest.mark.parametrize("layer_id", [0, 4, 6])
def test_quantize_pack_llama65b_sampled_rows(lib, layer_id):
    name, k, n = synth.CONFIGS[synth.LLAMA65B_DECODE]["layers"][layer_id]
    print(f"LLaMA-65B layer {name} K={k} N={n}", flush=True)
    W = synth.weights(3, layer_id, n, k)
    s = oracle.channel_scale(synth.calibration(3, layer_id, k))
    rows = np.sort(np.random.default_rng(layer_id).choice(n, size=96, replace=False))
    rows[-1] = n - 1
    _qp_compare(lib, W, s, rows)


@pytest.mark.parametrize("kind", ["ties", "constant", "positive", "negative", "subnormal", "wide", "mixed"])
@pytest.mark.parametrize("with_s", [False, True])
def test_quantize_pack_edge_tensors(lib, kind, with_s):
    n, k = 37, 384  # ragged: odd N, K = 3 groups
    W = synth.edge_weights(kind, n, k, seed=5)
    s = None
    if with_s:
        s = np.random.default_rng(3).uniform(0.25, 4.0, size=k).astype(np.float32)
        if kind == "wide":
            s = np.minimum(s, 1.0).astype(np.float32)
    _qp_compare(lib, W, s)


def test_quantize_pack_single_group_and_power_of_two_s(lib):
    W = synth.weights(1, 9, 1, 128)
    _qp_compare(lib, W, None)
    s = (2.0 ** np.random.default_rng(0).integers(-3, 4, size=128)).astype(np.float32)
    _qp_compare(lib, W, s)


@pytest.mark.parametrize("alpha", [0.5, 1.0, 0.0])
@pytest.mark.parametrize("cfg,k", [(1, 2048), (3, 8192), (2, 11008)])
def test_channel_scale_bit_exact(lib, alpha, cfg, k):
    g = _gpu()
    xc = synth.calibration(cfg, 0, k)
    xc[:, 7] = 0  # an all-zero channel
    got = g.host(lib.channel_scale(g.dev(xc), alpha))
    want = oracle.channel_scale(xc, alpha)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), g.report_mismatch("s", got, want)


@pytest.mark.parametrize("t_cal,k,misalign", [(7, 4096, False), (100, 37, False), (513, 136, False), (1, 8, False),
                                              (64, 1024, True), (33, 120, True)])
def test_channel_scale_token_split_and_fallback(lib, t_cal, k, misalign):
    # K % 8 == 0 with 16-byte alignment takes the token-split kernel, anything else the
    # per-channel kernel; the float64 sum is exact, so both must give identical bits
    import torch

    g = _gpu()
    xc = synth.calibration(1, 4, k, t_cal)
    if misalign:
        flat = torch.empty(t_cal * k + 1, dtype=torch.float16, device=g.DEV)
        xd = flat[1:].view(t_cal, k)
        xd.copy_(torch.from_numpy(xc))
        assert xd.data_ptr() % 16 != 0
    else:
        xd = g.dev(xc)
    for alpha in (0.5, 1.0):
        got = g.host(lib.channel_scale(xd, alpha))
        want = oracle.channel_scale(xc, alpha)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), g.report_mismatch("s", got, want)


def test_channel_scale_general_alpha_within_an_ulp(lib):
    g = _gpu()
    xc = synth.calibration(1, 1, 2048)
    got = g.host(lib.channel_scale(g.dev(xc), 0.3)).astype(np.float64)
    want = oracle.channel_scale(xc, 0.3).astype(np.float64)
    assert np.all(np.abs(got - want) <= np.spacing(want.astype(np.float32)).astype(np.float64))


@pytest.mark.parametrize("m,k", [(1, 8192), (32, 4096), (3, 384)])
def test_scale_input_bit_exact(lib, m, k):
    g = _gpu()
    x = synth.activations(4, 0, m, k)
    s = oracle.channel_scale(synth.calibration(4, 0, k))
    got = g.bits16(g.host(lib.scale_input(g.dev(x), g.dev(s))))
    want = g.bits16(oracle.scale_input(x, s))
    assert np.array_equal(got, want), g.report_mismatch("x_s", got, want)
