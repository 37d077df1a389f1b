"""GPU parity of the x-resident small-batch MFMA kernel (w4a16_linear_xres) against the float64
oracle: every output within 1e-3 * sum_k |x * w_hat| + 1e-5 on ragged shapes (rows past M,
columns past N, K ranges shorter than 2048 inputs and waves past the last group), the full
K = N = 8192 layer at M = 16 and 32 (every output), zeros outside the exact fp16 range (the
general route), one K range (y written directly), a workspace full of NaN (every partial is
written before it is read), and run-to-run reproducibility."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _gpu():
    from tests import _gpu

    return _gpu


def _packed(seed, lid, n, k):
    s = oracle.channel_scale(synth.calibration(seed, lid, k))
    return s, oracle.quantize_pack(synth.weights(seed, lid, n, k), s)


def _check(lib, x, packed, tag, workspace=None):
    g = _gpu()
    m, k = x.shape
    n = packed[0].shape[0]
    print(f"x-resident {tag} M={m} N={n} K={k}", flush=True)
    y = g.host(lib.linear_xres(g.dev(x), *[g.dev(t) for t in packed], workspace=workspace))
    y_ref, b = oracle.linear(x, *packed)
    ok = oracle.within_tolerance(y.astype(np.float64), y_ref, b)
    assert np.all(ok), (tag, np.argwhere(~ok)[:3])
    return y


@pytest.mark.parametrize("m", [1, 2, 5, 16, 17, 31, 32])
@pytest.mark.parametrize("n,k", [(1, 256), (97, 2048), (128, 2304), (300, 4352), (129, 11008)])
def test_xres_ragged_shapes(lib, m, n, k):
    s, packed = _packed(7, 1, n, k)
    x = oracle.scale_input(synth.activations(7, 1, m, k), s)
    _check(lib, x, packed, "ragged")




def test_xres_small_batch_layer_every_output(lib):
    # the small-batch decode sweep's layer, K = N = 8192, 4-bit groups of 128: every output at
    # M = 12, 16, 24 and 32 (rows are independent, so the oracle runs once on 32 rows)
    g = _gpu()
    k = n = 8192
    s = oracle.channel_scale(synth.calibration(3, 0, k))
    W = synth.weights(3, 0, n, k)
    packed = tuple(g.host(t) for t in lib.quantize_pack(g.dev(W), g.dev(s)))
    packed = (packed[0].view(np.uint32), packed[1], packed[2])
    x = oracle.scale_input(synth.activations(3, 0, 32, k), s)
    y_ref, b = oracle.linear(x, *packed)
    dev = [g.dev(t) for t in packed]
    for m in (12, 16, 24, 32):
        print(f"x-resident 8192x8192 M={m}", flush=True)
        y = g.host(lib.linear_xres(g.dev(x[:m]), *dev))
        ok = oracle.within_tolerance(y.astype(np.float64), y_ref[:m], b[:m])
        assert np.all(ok), (m, np.argwhere(~ok)[:3])


@pytest.mark.parametrize("m", [17, 32])
def test_xres_four_wave_ranges(lib, m):
    # M > 16 on a grid of at least 512 eight-wave workgroups (ceil(32769 / 128) * ceil(2304 / 2048)
    # = 514): four-wave workgroups and K ranges of 1024 inputs (8, 8 and 2 groups: the last
    # range's second wave and above idle); a ragged last column tile; every output
    n, k = 32769, 2304
    s, packed = _packed(9, 2, n, k)
    x = oracle.scale_input(synth.activations(9, 2, m, k), s)
    assert lib.xres_workspace_bytes(m, n, k) == 3 * m * n * 4
    if m == 17:
        # and M <= 16 on the same layer: 64-column workgroups of eight waves (514 of them)
        x16 = oracle.scale_input(synth.activations(9, 2, 16, k), s)
        _check(lib, x16, packed, "64-column")
    _check(lib, x, packed, "four-wave")


@pytest.mark.parametrize("m", [1, 5, 16, 17, 32])
@pytest.mark.parametrize("n,k", [(97, 2048), (300, 4352), (129, 11008)])
def test_xres_groups_of_64(lib, m, n, k):
    # groups of 64: each MFMA step takes 32 contiguous inputs (codes word-transposed through
    # the stage, x fragments in the same order), two steps per group, each group scaled after
    # its steps; ragged rows, columns and K ranges as above
    g = _gpu()
    s = oracle.channel_scale(synth.calibration(9, 2, k))
    packed = oracle.quantize_pack(synth.weights(9, 2, n, k), s, group=64)
    x = oracle.scale_input(synth.activations(9, 2, m, k), s)
    print(f"x-resident groups of 64 M={m} N={n} K={k}", flush=True)
    y = g.host(lib.linear_xres(g.dev(x), *[g.dev(t) for t in packed], group=64))
    y_ref, b = oracle.linear(x, *packed, group=64)
    ok = oracle.within_tolerance(y.astype(np.float64), y_ref, b)
    assert np.all(ok), np.argwhere(~ok)[:3]


@pytest.mark.parametrize("kind", ["positive", "negative", "wide"])
def test_xres_groups_of_64_edge_weights(lib, kind):
    # one-signed and wide groups: zeros outside [-2032, 1024] send their waves to the general
    # route (exact q and z * sum x per group of 64)
    g = _gpu()
    packed = oracle.quantize_pack(synth.edge_weights(kind, 96, 4096, seed=13), None, group=64)
    for m in (3, 32):
        x = synth.activations(1, 14, m, 4096)
        print(f"x-resident groups of 64 {kind} M={m}", flush=True)
        y = g.host(lib.linear_xres(g.dev(x), *[g.dev(t) for t in packed], group=64))
        y_ref, b = oracle.linear(x, *packed, group=64)
        assert np.all(oracle.within_tolerance(y.astype(np.float64), y_ref, b)), (kind, m)


def test_xres_groups_of_64_full_layer(lib):
    # K = N = 8192 with groups of 64: every output at M = 16 and 32
    g = _gpu()
    k = n = 8192
    s = oracle.channel_scale(synth.calibration(4, 0, k))
    packed = oracle.quantize_pack(synth.weights(4, 0, n, k), s, group=64)
    x = oracle.scale_input(synth.activations(4, 0, 32, k), s)
    y_ref, b = oracle.linear(x, *packed, group=64)
    dev = [g.dev(t) for t in packed]
    for m in (16, 32):
        print(f"x-resident groups of 64 8192^2 M={m}", flush=True)
        y = g.host(lib.linear_xres(g.dev(x[:m]), *dev, group=64))
        ok = oracle.within_tolerance(y.astype(np.float64), y_ref[:m], b[:m])
        assert np.all(ok), (m, np.argwhere(~ok)[:3])


@pytest.mark.parametrize("kind", ["positive", "negative", "mixed", "wide"])
def test_xres_edge_weights(lib, kind):
    W = synth.edge_weights(kind, 96, 4096, seed=13)
    packed = oracle.quantize_pack(W, None)
    for m in (3, 32):
        x = synth.activations(1, 14, m, 4096)
        _check(lib, x, packed, kind)


def test_xres_nan_workspace_and_reproducible(lib):
    import torch

    g = _gpu()
    k, n, m = 8192, 640, 20
    s, packed = _packed(5, 9, n, k)
    x = oracle.scale_input(synth.activations(5, 9, m, k), s)
    ws = torch.full((lib.xres_workspace_bytes(m, n, k) // 4,), float("nan"), dtype=torch.float32, device=g.DEV)
    y1 = _check(lib, x, packed, "nan workspace", workspace=ws)
    y2 = g.host(lib.linear_xres(g.dev(x), *[g.dev(t) for t in packed]))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_auto_path_falls_back_on_two_byte_aligned_scales(lib):
    # scales and zeros only 2-byte aligned: the automatic path with a workspace declines the
    # x-resident kernel (which loads (scale, zero) pairs as 4-byte words) and takes the earlier
    # choice within the same workspace; the kernel's own entry point refuses them
    import torch

    g = _gpu()
    m, n, k = 16, 8192, 8192
    assert lib.linear_ws_kernel(m, n, k) == 2
    s, (qw, sc, zr) = _packed(4, 3, n, k)
    x = oracle.scale_input(synth.activations(4, 3, m, k), s)
    G = k // 128

    def shifted(a):
        buf = torch.zeros(a.size + 1, dtype=torch.float16, device=g.DEV)
        buf[1:] = torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).to(g.DEV)
        return buf[1:].view(n, G)

    sc_d, zr_d = shifted(sc), shifted(zr)
    assert sc_d.data_ptr() % 4 == 2 and zr_d.data_ptr() % 4 == 2
    print("x-resident fallback on 2-byte aligned scales", flush=True)
    y = g.host(lib.linear(g.dev(x), g.dev(qw), sc_d, zr_d)).astype(np.float64)
    y_ref, b = oracle.linear(x, qw, sc, zr)
    assert np.all(oracle.within_tolerance(y, y_ref, b))
    with pytest.raises(lib.W4A16Error):
        lib.linear_xres(g.dev(x), g.dev(qw), sc_d, zr_d)
