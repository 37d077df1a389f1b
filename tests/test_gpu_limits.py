"""GPU parity at the size limits of the C ABI: the largest K (W4A16_MAX_K = 131072) on
every linear path, a million output rows (grids of 10^5 - 10^6 workgroups), the
largest batch (M = 65536), a 65536-token calibration set for the AWQ loss (the size of
a 128 x 512-token calibration set), and a million rows through the norm fold. Outputs
are compared with the float64 oracle, on sampled rows where the full oracle would be
slow."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

MAX_K = 131072


def _gpu():
    from tests import _gpu

    return _gpu


def _close(y, y_ref, b, tag):
    ok = oracle.within_tolerance(np.asarray(y, dtype=np.float64), y_ref, b)
    assert np.all(ok), (tag, int((~ok).sum()), np.argwhere(~ok)[:3])


@pytest.mark.parametrize("m,path", [(1, 1), (5, 3), (40, 2), (1, 0), (40, 0)])
def test_max_k_every_path(lib, m, path):
    g = _gpu()
    n = 40
    x_cal = synth.calibration(4, 70, MAX_K, 64)
    s = oracle.channel_scale(x_cal)
    packed = oracle.quantize_pack(synth.weights(4, 70, n, MAX_K), s)
    x = oracle.scale_input(synth.activations(4, 70, m, MAX_K), s)
    print(f"max-K linear M={m} path={path}", flush=True)
    y = g.host(lib.linear(g.dev(x), *[g.dev(t) for t in packed], path=path))
    y_ref, b = oracle.linear(x, *packed)
    _close(y, y_ref, b, f"path {path}")
    if m == 40:
        ys = g.host(lib.linear_splitk(g.dev(x), *[g.dev(t) for t in packed], splits=16))
        _close(ys, y_ref, b, "split-K")


@pytest.mark.parametrize("fmt", ["3bit", "g32", "nf4"])
def test_max_k_other_formats(lib, fmt):
    g = _gpu()
    n, m = 24, 3
    W = synth.weights(4, 71, n, MAX_K)
    x = synth.activations(4, 71, m, MAX_K)
    print(f"max-K {fmt}", flush=True)
    if fmt == "nf4":
        qw, a = oracle.quantize_pack_nf4(W, None, 64)
        y = g.host(lib.nf4_linear(g.dev(x), g.dev(qw), g.dev(a), block=64))
        y_ref, b = oracle.linear_nf4(x, qw, a, 64)
    else:
        bits, group = (3, 128) if fmt == "3bit" else (4, 32)
        packed = oracle.quantize_pack(W, None, bits=bits, group=group)
        y = g.host(lib.linear(g.dev(x), *[g.dev(t) for t in packed], group=group, bits=bits))
        y_ref, b = oracle.linear(x, *packed, group=group, bits=bits)
    _close(y, y_ref, b, fmt)


def test_million_output_rows(lib):
    # N = 2^20 rows of K = 128: quantize-pack on the device (bit-exact on sampled rows), then
    # the GEMV (131072 workgroups), the small-batch kernel and the tiled kernel
    g = _gpu()
    n, k = 1 << 20, 128
    W = synth.weights(4, 72, n, k)
    rows = np.linspace(0, n - 1, 512).astype(int)
    print("million-row quantize-pack", flush=True)
    qd = lib.quantize_pack(g.dev(W))
    want = oracle.quantize_pack(W[rows])
    assert np.array_equal(g.host_u32(qd[0])[rows], want[0])
    assert np.array_equal(g.bits16(g.host(qd[1])[rows]), g.bits16(want[1]))
    assert np.array_equal(g.bits16(g.host(qd[2])[rows]), g.bits16(want[2]))
    packed_rows = (want[0], want[1], want[2])
    for m, path in ((1, 1), (4, 3), (40, 2)):
        x = synth.activations(4, 72, m, k)
        print(f"million-row linear M={m} path={path}", flush=True)
        y = g.host(lib.linear(g.dev(x), *qd, path=path))[:, rows]
        y_ref, b = oracle.linear(x, *packed_rows)
        _close(y, y_ref, b, f"path {path}")


def test_max_batch(lib):
    # M = 65536 (the ABI limit) on the tiled and split-K kernels
    g = _gpu()
    m, n, k = 1 << 16, 64, 256
    packed = oracle.quantize_pack(synth.weights(4, 73, n, k))
    x = synth.activations(4, 73, m, k)
    y_ref, b = oracle.linear(x, *packed)
    print("max-batch tiled", flush=True)
    y = g.host(lib.linear(g.dev(x), *[g.dev(t) for t in packed], path=2))
    _close(y, y_ref, b, "tiled")
    print("max-batch split-K", flush=True)
    ys = g.host(lib.linear_splitk(g.dev(x), *[g.dev(t) for t in packed], splits=2))
    _close(ys, y_ref, b, "split-K")


def test_alpha_loss_large_calibration_set(lib):
    # 65536 calibration tokens (128 samples x 512 tokens)
    g = _gpu()
    t_cal, n, k = 1 << 16, 96, 256
    W = synth.weights(2, 74, n, k)
    x_cal = synth.calibration(2, 74, k, t_cal)
    s = oracle.channel_scale(x_cal, 0.5)
    xs = oracle.scale_input(x_cal, s)
    q, sc, z = oracle.quantize_pack(W, s)
    print("alpha-loss T=65536", flush=True)
    y_ref = lib.output_reference(g.dev(x_cal), g.dev(W))
    got = float(g.host(lib.alpha_loss(g.dev(xs), g.dev(q), g.dev(sc), g.dev(z), y_ref))[0])
    want = oracle.alpha_loss(x_cal, W, 0.5)
    assert abs(got - want) <= 1e-3 * want, (got, want)
    # the device statistic at this size is still bit-exact
    got_s = g.host(lib.channel_scale(g.dev(x_cal), 0.5))
    assert np.array_equal(got_s.view(np.uint32), s.view(np.uint32))


def test_norm_fold_million_rows(lib):
    g = _gpu()
    m, k = 1 << 20, 8
    rng = np.random.default_rng(75)
    h = rng.standard_normal((m, k)).astype(np.float16)
    gamma = (1 + 0.1 * rng.standard_normal(k)).astype(np.float16)
    s = (0.5 + rng.random(k)).astype(np.float32)
    print("norm fold M=2^20", flush=True)
    got = g.host(lib.rmsnorm_fold(g.dev(h), g.dev(gamma), g.dev(s), 1e-5))
    rows = np.linspace(0, m - 1, 4096).astype(int)
    want = oracle.rmsnorm_fold(h[rows], gamma, s, 1e-5)
    diff = got[rows].view(np.uint16).astype(np.int64) - want.view(np.uint16).astype(np.int64)
    assert np.all(np.abs(diff) <= 1) and np.mean(diff != 0) < 1e-3
