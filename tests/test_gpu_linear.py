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


def _check(lib, xs, qw, sc, zr, path, rows=None, tag="", workspace="auto"):
    g = _gpu()
    print(f"linear {tag} M={xs.shape[0]} N={qw.shape[0]} K={xs.shape[1]} path={path}", flush=True)
    y = g.host(lib.linear(g.dev(xs), g.dev(qw), g.dev(sc), g.dev(zr), path=path, workspace=workspace)).astype(np.float64)
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


@pytest.mark.parametrize("bits,group", [(4, 128), (4, 64), (3, 128)])
@pytest.mark.parametrize("n,k", [(300, 2048), (97, 11008), (4100, 4096)])
def test_gemv_output_independent_of_batch(lib, bits, group, n, k):
    # Each thread runs over the same inputs in the same order at any batch size up to 8 (one
    # piece per thread on these rows), and the wave sums every output's lane partials in one
    # fixed order however many (row, input) values share the batched reduction (sets of 8, 4,
    # 2 and single values; M = 3, 5, 6 and 7 reach all four). So an output of a batch of M equals,
    # bit for bit, that of its x row run alone.
    g = _gpu()
    L = synth.layer(4, 70, n, k, 8)
    s = oracle.channel_scale(L["x_cal"])
    xs = oracle.scale_input(L["x"], s)
    packed = oracle.quantize_pack(L["W"], s, bits=bits, group=group)
    dev = [g.dev(t) for t in packed]
    print(f"gemv batch independence bits={bits} group={group} N={n} K={k}", flush=True)
    alone = np.concatenate([g.host(lib.linear(g.dev(np.ascontiguousarray(xs[i:i + 1])), *dev, group=group,
                                              bits=bits, path=1)) for i in range(8)])
    y_ref, b = oracle.linear(xs, *packed, group=group, bits=bits)
    assert np.all(oracle.within_tolerance(alone.astype(np.float64), y_ref, b))
    for m in range(2, 9):
        y = g.host(lib.linear(g.dev(np.ascontiguousarray(xs[:m])), *dev, group=group, bits=bits, path=1))
        assert np.array_equal(y.view(np.uint16), alone[:m].view(np.uint16)), m


def test_gemv_long_rows_take_several_pieces_per_thread(lib):
    # K = 22016 (two pieces per thread) and K = 65536 (eight) on M = 1; K = 32768 at M = 4
    # K = 22016 and 32768 at M = 2: one piece per thread in 688- and 1024-thread workgroups (the
    # automatic route of the LLaMA-65B down projection at M = 2)
    for m, k in [(1, 22016), (1, 65536), (2, 22016), (2, 32768), (2, 40960), (4, 32768)]:
        xs, qw, sc, zr = _packed(4, 40, 33, k, m)
        _check(lib, xs, qw, sc, zr, path=1, tag="gemv-long")


@pytest.mark.parametrize("m", [1, 9, 16, 33, 64, 100])
@pytest.mark.parametrize("n,k", [(200, 1024), (64, 384), (130, 11008)])
def test_mfma_small_shapes(lib, m, n, k):
    xs, qw, sc, zr = _packed(5, 20 + m, n, k, m)
    _check(lib, xs, qw, sc, zr, path=2, tag="mfma")


@pytest.mark.parametrize("m", [1, 2, 3, 7, 12, 13, 16, 17, 31, 32])
@pytest.mark.parametrize("n,k", [(300, 2048), (97, 11008), (64, 384), (1, 128), (40, 1408), (8200, 1024)])
def test_skinny_small_shapes(lib, m, n, k):
    # M = 12..16: x rows through LDS (eight full-width loads, rows past M read as zero)
    # K = 384 and 128 leave some of the eight K-splitting waves without a group; K = 1408 (11 groups)
    # and 11008 give uneven splits and half-filled last stages; N = 8200 takes the two-tile-per-wave
    # variant with a ragged last workgroup
    xs, qw, sc, zr = _packed(4, 50 + m, n, k, m)
    _check(lib, xs, qw, sc, zr, path=3, tag="skinny")


@pytest.mark.parametrize("m", [33, 40, 48, 63, 64])
@pytest.mark.parametrize("n,k", [(300, 2048), (97, 11008), (8192, 1024)])
def test_auto_33_to_64_rows(lib, m, n, k):
    # 33 <= M <= 64 on layers with N <= 8192: the tiled kernel would start at most 256
    # workgroups, so the automatic path takes the K-lane kernel (4-bit codes, groups of 128;
    # the other formats run the small-batch kernel twice there). Every row against the oracle,
    # and bit-identical to forcing the K-lane kernel; the small-batch kernel run on the two
    # row blocks separately (path 3) is checked against the oracle too
    g = _gpu()
    xs, qw, sc, zr = _packed(4, 60 + m, n, k, m)
    _check(lib, xs, qw, sc, zr, path=0, tag="auto-33-64")
    dev = [g.dev(t) for t in (xs, qw, sc, zr)]
    y = g.host(lib.linear(*dev, workspace=None))  # w4a16_linear: no workspace, no split-K
    assert np.array_equal(g.bits16(y), g.bits16(g.host(lib.linear(*dev, path=4))))
    y1 = g.host(lib.linear(dev[0][:32].contiguous(), *dev[1:], path=3)).astype(np.float64)
    y2 = g.host(lib.linear(dev[0][32:].contiguous(), *dev[1:], path=3)).astype(np.float64)
    y_ref, b = oracle.linear(xs, qw, sc, zr)
    assert np.all(oracle.within_tolerance(np.concatenate([y1, y2]), y_ref, b))


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


@pytest.mark.parametrize("layer_id,m", [(0, 1), (4, 1), (6, 1), (6, 2)])
def test_llama65b_full_size_all_rows(lib, layer_id, m):
    # every output of the LLaMA-65B decode layers (8192^2, 8192 -> 22016, 22016 -> 8192) on the
    # automatic path, as the bench launches them
    name, k, n = synth.CONFIGS[synth.LLAMA65B_DECODE]["layers"][layer_id]
    xs, qw, sc, zr = _packed(3, layer_id, n, k, m)
    _check(lib, xs, qw, sc, zr, path=0, tag=f"llama65b-{name}-all-rows")


@pytest.mark.parametrize("m", [2, 4, 8, 16, 32])
def test_batch_sweep_8192_all_paths(lib, m):
    xs, qw, sc, zr = _packed(4, 0, 8192, 8192, m)
    rows = _sampled_rows(8192, m)
    paths = (1, 2, 3) if m <= 8 else (2, 3)
    for path in paths:
        _check(lib, xs, qw, sc, zr, path=path, rows=rows, tag="sweep-8192")
    _check(lib, xs, qw, sc, zr, path=0, tag="sweep-8192-auto-all-rows")


@pytest.mark.parametrize("m", [128, 256])
@pytest.mark.parametrize("layer_id", [0, 1, 2])
def test_llama2_7b_batched_serving(lib, m, layer_id):
    # every output of the LLaMA2-7B serving GEMMs on the automatic path
    name, k, n = synth.CONFIGS[synth.LLAMA2_7B_SERVING]["layers"][layer_id]
    xs, qw, sc, zr = _packed(5, layer_id, n, k, m)
    _check(lib, xs, qw, sc, zr, path=0, tag=f"serving-{name}-all-rows")


@pytest.mark.parametrize("kind", ["positive", "negative", "constant", "ties", "mixed"])
@pytest.mark.parametrize("path,m", [(1, 1), (1, 3), (2, 1), (2, 20), (3, 2), (3, 32), (4, 20), (4, 70)])
def test_edge_weights(lib, kind, path, m):
    n, k = 70, 1024
    W = synth.edge_weights(kind, n, k, seed=11)
    xs, qw, sc, zr = _packed(6, 1, n, k, m, W=W)
    _check(lib, xs, qw, sc, zr, path=path, tag=f"edge-{kind}")


@pytest.mark.parametrize("kind", ["positive", "negative", "mixed"])
@pytest.mark.parametrize("path,m", [(1, 1), (1, 4), (2, 1), (2, 20), (3, 2), (3, 32), (4, 20), (4, 70)])
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


@pytest.mark.parametrize("path,m", [(1, 1), (1, 8), (2, 16), (2, 128), (3, 2), (3, 32), (4, 33), (4, 128)])
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


@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (33, 97, 384), (64, 32, 128), (65, 33, 256), (100, 300, 2048),
                                   (128, 200, 11008), (257, 64, 4096), (70, 130, 640), (192, 4096, 4096)])
def test_klane_ragged_shapes(lib, m, n, k):
    # the K-lane kernel (path 4): rows past M and columns past N, K-lanes with no group
    # (K = 128, 256) and uneven group ranges (K = 384, 640, 11008)
    xs, qw, sc, zr = _packed(8, 1, n, k, m)
    _check(lib, xs, qw, sc, zr, path=4, tag="klane")


@pytest.mark.parametrize("bits,group,n,k,path", [
    (4, 128, 8192, 8192, 1), (4, 128, 8192, 22016, 1), (4, 128, 8192, 28672, 3), (4, 128, 4096, 4096, 1),
    (4, 64, 8192, 28672, 1), (4, 32, 4096, 11008, 1),
    (3, 128, 8192, 8192, 1), (3, 128, 11008, 4096, 1), (3, 128, 4096, 11008, 3), (3, 128, 4096, 4096, 3)])
def test_auto_m2_route(lib, bits, group, n, k, path):
    # M = 2: the automatic choice between the GEMV (path 1) and the small-batch kernel (path 3),
    # bit-identical to forcing the kernel the dispatch rule names for the shape. Random codes,
    # scales and zeros: this checks the route; parity of each kernel is checked elsewhere.
    g = _gpu()
    rng = np.random.default_rng(7)
    words = k // 8 if bits == 4 else 3 * k // 32
    qw = rng.integers(-2**31, 2**31, size=(n, words), dtype=np.int64).astype(np.int32)
    sc = rng.uniform(1e-3, 1e-2, size=(n, k // group)).astype(np.float16)
    zr = rng.integers(0, 2**bits, size=(n, k // group)).astype(np.float16)
    x = rng.standard_normal((2, k)).astype(np.float16)
    dev = [g.dev(t) for t in (x, qw, sc, zr)]
    print(f"auto M=2 route bits={bits} group={group} N={n} K={k} -> path {path}", flush=True)
    a = g.host(lib.linear(*dev, group=group, bits=bits, workspace=None))
    b = g.host(lib.linear(*dev, group=group, bits=bits, path=path))
    assert np.array_equal(g.bits16(a), g.bits16(b))


@pytest.mark.parametrize("m,k,n", [(48, 4096, 4096), (64, 11008, 4096), (128, 4096, 4096), (256, 11008, 4096),
                                   (64, 8192, 8192), (96, 22016, 8192), (24, 22016, 1024), (32, 22016, 8192),
                                   (96, 8192, 8192), (384, 11008, 4096), (512, 8192, 1024)])
def test_auto_klane_route(lib, m, k, n):
    # shapes the automatic dispatch of w4a16_linear (no workspace) sends to the K-lane kernel:
    # every output against the oracle, and bit-identical to forcing path 4
    g = _gpu()
    xs, qw, sc, zr = _packed(8, 2, n, k, m)
    _check(lib, xs, qw, sc, zr, path=0, tag="auto-klane", workspace=None)
    a = g.host(lib.linear(g.dev(xs), g.dev(qw), g.dev(sc), g.dev(zr), path=0, workspace=None))
    b = g.host(lib.linear(g.dev(xs), g.dev(qw), g.dev(sc), g.dev(zr), path=4))
    assert np.array_equal(g.bits16(a), g.bits16(b))


@pytest.mark.parametrize("m,k,n", [(64, 11008, 4096), (256, 4096, 4096), (48, 4096, 11008), (24, 8192, 1024),
                                   (256, 8192, 8192), (40, 4096, 1000), (128, 8192, 1024), (32, 16384, 1024)])
def test_auto_with_workspace_takes_split_k(lib, m, k, n):
    # the automatic path with a workspace (w4a16_linear_ws, the binding's default): shapes where
    # it splits K (8, 2, 2, 8, 2, 4, 8 and 8 ranges; the 32-row tiles of the partial kernel up to
    # M = 32): every output against the oracle, and bit-identical to the split-K entry point with
    # the same ranges
    g = _gpu()
    splits = lib.linear_ws_splits(m, n, k)
    assert splits > 0 and lib.linear_ws_kernel(m, n, k) == 1
    xs, qw, sc, zr = _packed(8, 3, n, k, m)
    _check(lib, xs, qw, sc, zr, path=0, tag=f"auto-ws-S{splits}")
    dev = [g.dev(t) for t in (xs, qw, sc, zr)]
    a = g.host(lib.linear(*dev))
    b = g.host(lib.linear_splitk(*dev, splits=splits))
    assert np.array_equal(g.bits16(a), g.bits16(b))
    # a caller's workspace of exactly the size asked for gives the same bits
    import torch

    ws = torch.empty(lib.linear_workspace_bytes(m, n, k) // 4, dtype=torch.float32, device=g.DEV)
    c = g.host(lib.linear(*dev, workspace=ws))
    assert np.array_equal(g.bits16(a), g.bits16(c))


@pytest.mark.parametrize("m,k,n", [(32, 22016, 8192), (21, 8192, 22016), (30, 4096, 11008), (17, 22016, 8192),
                                   (12, 4096, 11008), (24, 8192, 8192), (16, 4096, 20480), (8, 22016, 8192),
                                   (16, 8192, 8192), (4, 22016, 8192), (8, 8192, 1024), (12, 11008, 4096),
                                   (24, 11008, 4096)])
def test_auto_with_workspace_takes_x_resident(lib, m, k, n):
    # shapes where the automatic path with a workspace runs the x-resident small-batch kernel:
    # every output against the oracle,
    # bit-identical to its own entry point, and with a workspace of exactly the size asked for
    g = _gpu()
    assert lib.linear_ws_kernel(m, n, k) == 2
    xs, qw, sc, zr = _packed(8, 4, n, k, m)
    _check(lib, xs, qw, sc, zr, path=0, tag="auto-ws-x-resident")
    dev = [g.dev(t) for t in (xs, qw, sc, zr)]
    a = g.host(lib.linear(*dev))
    b = g.host(lib.linear_xres(*dev))
    assert np.array_equal(g.bits16(a), g.bits16(b))
    import torch

    ws = torch.empty(max(1, lib.linear_workspace_bytes(m, n, k) // 4), dtype=torch.float32, device=g.DEV)
    c = g.host(lib.linear(*dev, workspace=ws))
    assert np.array_equal(g.bits16(a), g.bits16(c))


@pytest.mark.parametrize("m,k,n", [(16, 22016, 8192), (32, 8192, 8192), (21, 8192, 22016), (12, 4096, 11008),
                                   (8, 8192, 1024), (32, 11008, 4096)])
def test_auto_with_workspace_takes_x_resident_groups_of_64(lib, m, k, n):
    # groups of 64 follow the same rule: every output against the oracle, bit-identical to the
    # kernel's own entry point, with a workspace of exactly the size asked for
    import torch

    g = _gpu()
    assert lib.linear_ws_kernel(m, n, k, group=64) == 2
    s = oracle.channel_scale(synth.calibration(8, 5, k))
    packed = oracle.quantize_pack(synth.weights(8, 5, n, k), s, group=64)
    x = oracle.scale_input(synth.activations(8, 5, m, k), s)
    print(f"auto-ws-x-resident groups of 64 M={m} K={k} N={n}", flush=True)
    dev = [g.dev(t) for t in (x, *packed)]
    ws = torch.empty(lib.linear_workspace_bytes(m, n, k, group=64) // 4, dtype=torch.float32, device=g.DEV)
    a = g.host(lib.linear(*dev, group=64, workspace=ws))
    y_ref, b = oracle.linear(x, *packed, group=64)
    assert np.all(oracle.within_tolerance(a.astype(np.float64), y_ref, b))
    c = g.host(lib.linear_xres(*dev, group=64))
    assert np.array_equal(g.bits16(a), g.bits16(c))


@pytest.mark.parametrize("m,k,n", [(512, 4096, 4096), (256, 2048, 16384), (300, 1024, 32768), (512, 8192, 8192)])
def test_auto_one_range_route(lib, m, k, n):
    # from M = 256, where the one-range split-K kernel's 64 x 128 tiles fill the 256 CUs a whole
    # number of times or come to at least 1280, the automatic path (with or without a
    # workspace) runs it: every output against the oracle, bit-identical to forcing path 5 and
    # to the split-K entry point with one range
    g = _gpu()
    assert lib.linear_ws_splits(m, n, k) == 0
    assert lib.linear_workspace_bytes(m, n, k) == 0
    xs, qw, sc, zr = _packed(8, 5, n, k, m)
    _check(lib, xs, qw, sc, zr, path=0, tag="auto-one-range", workspace=None)
    dev = [g.dev(t) for t in (xs, qw, sc, zr)]
    a = g.host(lib.linear(*dev, workspace=None))
    b = g.host(lib.linear(*dev, path=5))
    c = g.host(lib.linear(*dev))
    d = g.host(lib.linear_splitk(*dev, splits=1))
    for other in (b, c, d):
        assert np.array_equal(g.bits16(a), g.bits16(other))


@pytest.mark.parametrize("m,k,n", [(1, 128, 1), (70, 384, 300), (33, 4096, 1000), (200, 2048, 129)])
def test_one_range_kernel(lib, m, k, n):
    # path 5 forced on ragged shapes (rows and columns past the tiles, one group, odd N)
    xs, qw, sc, zr = _packed(8, 6, n, k, m)
    _check(lib, xs, qw, sc, zr, path=5, tag="one-range")


def test_auto_with_workspace_refuses_a_short_one(lib):
    import torch

    g = _gpu()
    m, k, n = 64, 11008, 4096
    xs, qw, sc, zr = _packed(8, 4, n, k, m)
    dev = [g.dev(t) for t in (xs, qw, sc, zr)]
    short = torch.empty(lib.linear_workspace_bytes(m, n, k) // 4 - 1, dtype=torch.float32, device=g.DEV)
    with pytest.raises(lib.W4A16Error):
        lib.linear(*dev, workspace=short)
