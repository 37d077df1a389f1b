"""GPU parity of the fused dequantize GEMV / MFMA GEMM against the float64
oracle: every output within |y - y_ref| <= 1e-3 * sum|x * w_hat| + 1e-5.

The kernels are fed oracle-packed weights and the oracle's 1/s-folded input,
so this checks the linear layer independently of the GPU quantizer."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _gpu():
    from tests import _gpu

    return _gpu


def _packed(cfg, layer_id, n, k, m, W=None):
    L = synth.layer(cfg, layer_id, n, k, m)
    if W is None:
        W = L["W"]
    s = oracle.channel_scale(L["x_cal"])
    xs = oracle.scale_input(L["x"], s)
    qw, sc, zr = oracle.quantize_pack(W, s)
    return xs, qw, sc, zr


def _check(lib, xs, qw, sc, zr, path, rows=None, tag=""):
    g = _gpu()
    print(f"linear {tag} M={xs.shape[0]} N={qw.shape[0]} K={xs.shape[1]} path={path}", flush=True)
    y = g.host(lib.linear(g.dev(xs), g.dev(qw), g.dev(sc), g.dev(zr), path=path)).astype(np.float64)
    if rows is not None:
        y = y[:, rows]
    y_ref, b = oracle.linear(xs, qw, sc, zr, rows=rows)
    ok = oracle.within_tolerance(y, y_ref, b)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{(~ok).sum()} outputs out of tolerance; first {tuple(i)}: y={y[tuple(i)]} "
                             f"ref={y_ref[tuple(i)]} B={b[tuple(i)]}")
    rel = np.abs(y - y_ref) / (b + 1e-30)
    return float(rel.max())


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("n,k", [(300, 2048), (97, 11008), (64, 384), (1, 128)])
def test_gemv_small_shapes(lib, m, n, k):
    xs, qw, sc, zr = _packed(4, 10 + m, n, k, m)
    _check(lib, xs, qw, sc, zr, path=1, tag="gemv")


def test_gemv_long_rows_take_several_pieces_per_thread(lib):
    # K = 22016 (two pieces per thread) and K = 65536 (eight) on M = 1; K = 32768 at M = 4
    for m, k in [(1, 22016), (1, 65536), (2, 40960), (4, 32768)]:
        xs, qw, sc, zr = _packed(4, 40, 33, k, m)
        _check(lib, xs, qw, sc, zr, path=1, tag="gemv-long")


@pytest.mark.parametrize("m", [1, 9, 16, 33, 64, 100])
@pytest.mark.parametrize("n,k", [(200, 1024), (64, 384), (130, 11008)])
def test_mfma_small_shapes(lib, m, n, k):
    xs, qw, sc, zr = _packed(5, 20 + m, n, k, m)
    _check(lib, xs, qw, sc, zr, path=2, tag="mfma")


@pytest.mark.parametrize("m", [1, 2, 3, 7, 16, 17, 31, 32])
@pytest.mark.parametrize("n,k", [(300, 2048), (97, 11008), (64, 384), (1, 128), (40, 1408), (8200, 1024)])
def test_skinny_small_shapes(lib, m, n, k):
    # K = 384 and 128 leave some of the eight K-splitting waves without a group; K = 1408 (11 groups)
    # and 11008 give uneven splits and half-filled last stages; N = 8200 takes the two-tile-per-wave
    # variant with a ragged last workgroup
    xs, qw, sc, zr = _packed(4, 50 + m, n, k, m)
    _check(lib, xs, qw, sc, zr, path=3, tag="skinny")


@pytest.mark.parametrize("m", [33, 40, 48, 63, 64])
@pytest.mark.parametrize("n,k", [(300, 2048), (97, 11008), (8192, 1024)])
def test_auto_two_small_batch_passes(lib, m, n, k):
    # 33 <= M <= 64 on layers with N <= 8192 and K <= 16384: the automatic path runs the
    # small-batch kernel on rows 0..31 and then on the rest; every row against the oracle, and
    # the result equals the small-batch kernel run on the two row blocks separately
    import torch

    g = _gpu()
    xs, qw, sc, zr = _packed(4, 60 + m, n, k, m)
    _check(lib, xs, qw, sc, zr, path=0, tag="auto-two-passes")
    dev = [g.dev(t) for t in (xs, qw, sc, zr)]
    y = g.host(lib.linear(*dev))
    y1 = g.host(lib.linear(dev[0][:32].contiguous(), *dev[1:], path=3))
    y2 = g.host(lib.linear(dev[0][32:].contiguous(), *dev[1:], path=3))
    assert np.array_equal(y.view(np.uint16), np.concatenate([y1, y2]).view(np.uint16))


def test_skinny_long_rows(lib):
    for m, k in [(2, 22016), (9, 65536), (32, 22016)]:
        xs, qw, sc, zr = _packed(4, 41, 70, k, m)
        _check(lib, xs, qw, sc, zr, path=3, tag="skinny-long")


def test_skinny_rejects_large_batches(lib):
    import torch

    from w4a16_decode_gemv_amd import W4A16Error

    g = _gpu()
    x = torch.zeros((33, 128), dtype=torch.float16, device=g.DEV)
    qw = torch.zeros((16, 16), dtype=torch.int32, device=g.DEV)
    sz = torch.zeros((16, 1), dtype=torch.float16, device=g.DEV)
    with pytest.raises(W4A16Error, match="small-batch"):
        lib.linear(x, qw, sz, sz, path=3)


def test_single_layer_2048(lib):
    xs, qw, sc, zr = _packed(1, 0, 2048, 2048, 1)
    for path in (0, 1, 2, 3):
        _check(lib, xs, qw, sc, zr, path=path, tag="single-2048")


@pytest.mark.parametrize("layer_id", [0, 4, 6])
def test_llama2_7b_block(lib, layer_id):
    name, k, n = synth.CONFIGS[synth.LLAMA2_7B_BLOCK]["layers"][layer_id]
    xs, qw, sc, zr = _packed(2, layer_id, n, k, 1)
    _check(lib, xs, qw, sc, zr, path=0, tag=f"llama2-7b-{name}")


def _sampled_rows(n, seed, count=256):
    rows = np.sort(np.random.default_rng(seed).choice(n, size=count, replace=False))
    rows[0], rows[-1] = 0, n - 1
    return rows


@pytest.mark.parametrize("layer_id", [0, 4, 6])
def test_llama65b_full_size_sampled(lib, layer_id):
    name, k, n = synth.CONFIGS[synth.LLAMA65B_DECODE]["layers"][layer_id]
    xs, qw, sc, zr = _packed(3, layer_id, n, k, 1)
    _check(lib, xs, qw, sc, zr, path=0, rows=_sampled_rows(n, layer_id), tag=f"llama65b-{name}")


@pytest.mark.parametrize("m", [2, 4, 8, 16, 32])
def test_batch_sweep_8192_all_paths(lib, m):
    xs, qw, sc, zr = _packed(4, 0, 8192, 8192, m)
    rows = _sampled_rows(8192, m)
    paths = (1, 2, 3) if m <= 8 else (2, 3)
    for path in paths:
        _check(lib, xs, qw, sc, zr, path=path, rows=rows, tag="sweep-8192")
    _check(lib, xs, qw, sc, zr, path=0, rows=rows, tag="sweep-8192-auto")


@pytest.mark.parametrize("m", [128, 256])
@pytest.mark.parametrize("layer_id", [0, 1, 2])
def test_llama2_7b_batched_serving(lib, m, layer_id):
    name, k, n = synth.CONFIGS[synth.LLAMA2_7B_SERVING]["layers"][layer_id]
    xs, qw, sc, zr = _packed(5, layer_id, n, k, m)
    _check(lib, xs, qw, sc, zr, path=0, rows=_sampled_rows(n, layer_id, 128), tag=f"serving-{name}")


@pytest.mark.parametrize("kind", ["positive", "negative", "constant", "ties", "mixed"])
@pytest.mark.parametrize("path,m", [(1, 1), (1, 3), (2, 1), (2, 20), (3, 2), (3, 32)])
def test_edge_weights(lib, kind, path, m):
    n, k = 70, 1024
    W = synth.edge_weights(kind, n, k, seed=11)
    xs, qw, sc, zr = _packed(6, 1, n, k, m, W=W)
    _check(lib, xs, qw, sc, zr, path=path, tag=f"edge-{kind}")


@pytest.mark.parametrize("kind", ["positive", "negative", "mixed"])
@pytest.mark.parametrize("path,m", [(1, 1), (1, 4), (2, 1), (2, 20), (3, 2), (3, 32)])
def test_zeros_outside_the_exact_fp16_range(lib, kind, path, m):
    # quantized without the AWQ scale, narrow one-signed groups get |zero| up to ~3400; the MFMA kernels
    # cannot form (q - z) exactly in fp16 beyond [-2032, 1024] and must take their general route there,
    # in waves that also hold in-range groups
    n, k = 70, 1024
    W = synth.edge_weights(kind, n, k, seed=11)
    qw, sc, zr = oracle.quantize_pack(W, None)
    z = zr.astype(np.float64)
    assert ((z < -2032) | (z > 1024)).any()
    xs = synth.activations(6, 3, m, k)
    _check(lib, xs, qw, sc, zr, path=path, tag=f"large-zero-{kind}")


def test_all_zero_rows_give_exact_zeros(lib):
    g = _gpu()
    n, k = 48, 2048
    W = synth.weights(6, 2, n, k)
    W[5] = 0
    W[47] = 0
    for path, m in [(1, 1), (1, 4), (2, 1), (2, 17), (3, 5), (3, 32)]:
        xs, qw, sc, zr = _packed(6, 2, n, k, m, W=W)
        y = g.host(lib.linear(g.dev(xs), g.dev(qw), g.dev(sc), g.dev(zr), path=path))
        assert np.all(y[:, 5] == 0) and np.all(y[:, 47] == 0)
        _check(lib, xs, qw, sc, zr, path=path, tag="zero-rows")


@pytest.mark.parametrize("path,m", [(1, 1), (1, 8), (2, 16), (2, 128), (3, 2), (3, 32)])
def test_deterministic_and_writes_only_its_output(lib, path, m):
    import torch

    g = _gpu()
    n, k = 515, 4096
    xs, qw, sc, zr = _packed(7, 0, n, k, m)
    x_d, q_d, s_d, z_d = g.dev(xs), g.dev(qw), g.dev(sc), g.dev(zr)
    canary = 0x7E5A
    pad = 4096
    buf = torch.full((m * n + 2 * pad,), canary, dtype=torch.int16, device=g.DEV)
    out = buf[pad:pad + m * n].view(torch.float16).view(m, n)
    lib.linear(x_d, q_d, s_d, z_d, out=out, path=path)
    first = g.host(out).copy()
    lib.linear(x_d, q_d, s_d, z_d, out=out, path=path)
    second = g.host(out)
    assert np.array_equal(first.view(np.uint16), second.view(np.uint16))
    b = g.host(buf).view(np.uint16)
    assert np.all(b[:pad] == canary) and np.all(b[pad + m * n:] == canary)


def test_gpu_pipeline_end_to_end_single_2048(lib):
    """channel scale -> fold -> quantize-pack -> linear, all on the GPU, against
    the oracle doing the same steps."""
    g = _gpu()
    L = synth.layer(1, 0, 2048, 2048, 1)
    s_d = lib.channel_scale(g.dev(L["x_cal"]))
    xs_d = lib.scale_input(g.dev(L["x"]), s_d)
    qw_d, sc_d, zr_d = lib.quantize_pack(g.dev(L["W"]), s_d)
    y = g.host(lib.linear(xs_d, qw_d, sc_d, zr_d)).astype(np.float64)
    s = oracle.channel_scale(L["x_cal"])
    xs = oracle.scale_input(L["x"], s)
    qw, sc, zr = oracle.quantize_pack(L["W"], s)
    y_ref, b = oracle.linear(xs, qw, sc, zr)
    assert np.all(oracle.within_tolerance(y, y_ref, b))
