"""GPU parity of the symmetric absmax and NF4 variants against the float64 oracle
(oracle/sym.py, oracle/nf4.py).

* quantize-pack: codes, scales/absmax and zeros bit-identical to the oracle's;
* the linear layer: every output within 1e-3 * sum_k |x * w_hat| + 1e-5 of the oracle, on
  the GEMV and tiled MFMA kernels, fed the oracle's packed weights. Symmetric weights run
  through the ordinary linear entry points (their zero is fixed); NF4 through nf4_linear.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _gpu():
    from tests import _gpu

    return _gpu


# ---------------------------------------------------------------- symmetric absmax
def _sym_compare(lib, W, s, bits, group, tag):
    g = _gpu()
    print(f"sym quantize-pack {tag} bits={bits} group={group} N={W.shape[0]} K={W.shape[1]}", flush=True)
    got = lib.quantize_pack_sym(g.dev(W), None if s is None else g.dev(s), bits=bits, group=group)
    want = oracle.quantize_pack_sym(W, s, bits=bits, group=group)
    assert np.array_equal(g.host_u32(got[0]), want[0])
    assert np.array_equal(g.bits16(g.host(got[1])), g.bits16(want[1]))
    assert np.array_equal(g.bits16(g.host(got[2])), g.bits16(want[2]))


@pytest.mark.parametrize("bits,group", [(4, 128), (4, 64), (4, 32), (3, 128), (3, 32)])
@pytest.mark.parametrize("n,k", [(37, 384), (256, 4096)])
def test_sym_quantize_pack_bit_exact(lib, bits, group, n, k):
    W = synth.weights(2, 7, n, k)
    s = oracle.channel_scale(synth.calibration(2, 7, k))
    _sym_compare(lib, W, s, bits, group, "scaled")
    _sym_compare(lib, W, None, bits, group, "plain")


@pytest.mark.parametrize("kind", ["ties", "constant", "positive", "negative", "subnormal", "wide", "mixed"])
def test_sym_quantize_pack_edge_tensors(lib, kind):
    W = synth.edge_weights(kind, 40, 512, seed=9)
    W[3, :128] = 0  # an all-zero group
    for bits, group in ((4, 128), (3, 64)):
        _sym_compare(lib, W, None, bits, group, kind)


@pytest.mark.parametrize("bits,group", [(4, 128), (4, 64), (4, 32), (3, 128)])
@pytest.mark.parametrize("m", [1, 3, 8, 17, 64])
def test_sym_linear_all_paths(lib, bits, group, m):
    g = _gpu()
    k, n = 2048, 300
    s = oracle.channel_scale(synth.calibration(2, 8, k))
    packed = oracle.quantize_pack_sym(synth.weights(2, 8, n, k), s, bits=bits, group=group)
    x = oracle.scale_input(synth.activations(2, 8, m, k), s)
    y_ref, b = oracle.linear(x, *packed, group=group, bits=bits)
    paths = [0, 2] + ([1] if m <= 8 else []) + ([3] if m <= 32 else [])
    for path in paths:
        print(f"sym linear bits={bits} group={group} M={m} path={path}", flush=True)
        y = g.host(lib.linear(g.dev(x), *[g.dev(t) for t in packed], group=group, path=path, bits=bits))
        assert np.all(oracle.within_tolerance(y.astype(np.float64), y_ref, b)), path


# ---------------------------------------------------------------- NF4
def _nf4_compare(lib, W, s, block, tag):
    g = _gpu()
    print(f"nf4 quantize-pack {tag} block={block} N={W.shape[0]} K={W.shape[1]}", flush=True)
    qw, a = lib.nf4_quantize_pack(g.dev(W), None if s is None else g.dev(s), block=block)
    want_q, want_a = oracle.quantize_pack_nf4(W, s, block)
    gq = g.host_u32(qw)
    assert np.array_equal(gq, want_q), g.report_mismatch("qweight", gq, want_q)
    ga = g.host(a)
    assert np.array_equal(ga.view(np.uint32), want_a.view(np.uint32)), g.report_mismatch("absmax", ga, want_a)


@pytest.mark.parametrize("block", [64, 32, 128])
@pytest.mark.parametrize("n,k", [(37, 384), (300, 2048), (64, 11008)])
def test_nf4_quantize_pack_bit_exact(lib, block, n, k):
    W = synth.weights(3, 2, n, k)
    _nf4_compare(lib, W, None, block, "plain")
    s = oracle.channel_scale(synth.calibration(3, 2, k))
    _nf4_compare(lib, W, s, block, "scaled")


@pytest.mark.parametrize("kind", ["ties", "constant", "positive", "negative", "subnormal", "wide", "mixed"])
def test_nf4_quantize_pack_edge_tensors(lib, kind):
    W = synth.edge_weights(kind, 40, 512, seed=11)
    W[5, 64:128] = 0  # an all-zero block
    _nf4_compare(lib, W, None, 64, kind)


def test_nf4_quantize_pack_codebook_levels_exactly(lib):
    # weights that are codebook levels times powers of two: every code must come back
    rng = np.random.default_rng(4)
    c = rng.integers(0, 16, size=(64, 1024))
    c[:, ::64] = 0  # level -1 in every block
    scale = 2.0 ** rng.integers(-9, -3, size=(64, 16))
    W = (oracle.NF4_LEVELS_F16.astype(np.float64)[c] * np.repeat(scale, 64, axis=1)).astype(np.float16)
    _nf4_compare(lib, W, None, 64, "levels")


def _nf4_linear_check(lib, x, qw, a, block, path, tag, rows=None):
    g = _gpu()
    print(f"nf4 linear {tag} block={block} path={path} M={x.shape[0]} N={qw.shape[0]} K={x.shape[1]}", flush=True)
    y = g.host(lib.nf4_linear(g.dev(x), g.dev(qw), g.dev(a), block=block, path=path))
    y_ref, b = oracle.linear_nf4(x, qw, a, block, rows=rows)
    if rows is not None:
        y = y[:, rows]
    ok = oracle.within_tolerance(y.astype(np.float64), y_ref, b)
    assert np.all(ok), (tag, np.argwhere(~ok)[:3])


@pytest.mark.parametrize("block", [64, 32, 128])
@pytest.mark.parametrize("m", [1, 2, 5, 8])
@pytest.mark.parametrize("n,k", [(1, 128), (37, 384), (300, 2048), (97, 11008), (64, 22016)])
def test_nf4_gemv(lib, block, m, n, k):
    if k > 16384 and m > 4:
        pytest.skip("the GEMV variant takes M <= 4 above K = 16384")
    qw, a = oracle.quantize_pack_nf4(synth.weights(3, 4, n, k), None, block)
    x = synth.activations(3, 4, m, k)
    _nf4_linear_check(lib, x, qw, a, block, 1, "gemv")


@pytest.mark.parametrize("block", [64, 32])
@pytest.mark.parametrize("m", [1, 9, 33, 100])
@pytest.mark.parametrize("n,k", [(37, 384), (300, 2048), (130, 11008)])
def test_nf4_mfma(lib, block, m, n, k):
    qw, a = oracle.quantize_pack_nf4(synth.weights(3, 5, n, k), None, block)
    x = synth.activations(3, 5, m, k)
    _nf4_linear_check(lib, x, qw, a, block, 2, "mfma")


@pytest.mark.parametrize("block", [128, 64, 32])
@pytest.mark.parametrize("m", [2, 3, 5, 8, 9, 16, 17, 32])
@pytest.mark.parametrize("n,k", [(1, 128), (37, 384), (300, 2048), (97, 11008), (40, 32768)])
def test_nf4_skinny(lib, block, m, n, k):
    # the small-batch MFMA kernel with the codebook in LDS and 1, 2 or 4 float32 absmax
    # values per 128 inputs
    qw, a = oracle.quantize_pack_nf4(synth.weights(3, 6, n, k), None, block)
    x = synth.activations(3, 6, m, k)
    _nf4_linear_check(lib, x, qw, a, block, 3, "skinny")


@pytest.mark.parametrize("block", [64, 32])
@pytest.mark.parametrize("m", [2, 8, 32])
def test_nf4_skinny_wide_layer(lib, block, m):
    # N = 8200: two 16-column tiles per wave where they fit in registers
    qw, a = oracle.quantize_pack_nf4(synth.weights(3, 7, 8200, 1024), None, block)
    x = synth.activations(3, 7, m, 1024)
    _nf4_linear_check(lib, x, qw, a, block, 3, "skinny-wide")


@pytest.mark.parametrize("m", [1, 4, 128])
def test_nf4_full_size_sampled_and_deterministic(lib, m):
    # LLaMA-65B q projection 8192 x 8192, packed on the device, 256 sampled rows
    g = _gpu()
    W = synth.weights(3, 0, 8192, 8192)
    qw_d, a_d = lib.nf4_quantize_pack(g.dev(W), None, block=64)
    x = synth.activations(3, 0, m, 8192)
    xd = g.dev(x)
    y1 = g.host(lib.nf4_linear(xd, qw_d, a_d, block=64))
    y2 = g.host(lib.nf4_linear(xd, qw_d, a_d, block=64))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    rows = np.linspace(0, 8191, 256).astype(int)
    y_ref, b = oracle.linear_nf4(x, g.host_u32(qw_d), g.host(a_d), 64, rows=rows)
    assert np.all(oracle.within_tolerance(y1[:, rows].astype(np.float64), y_ref, b))


@pytest.mark.parametrize("block", [64, 32])
@pytest.mark.parametrize("m", [40, 64])
def test_nf4_auto_two_small_batch_passes(lib, block, m):
    # 33 <= M <= 64 on a layer with N <= 8192 and K <= 16384: two small-batch launches
    g = _gpu()
    qw, a = oracle.quantize_pack_nf4(synth.weights(3, 8, 300, 2048), None, block)
    x = synth.activations(3, 8, m, 2048)
    _nf4_linear_check(lib, x, qw, a, block, 0, "auto-two-passes")
    qd, ad, xd = g.dev(qw), g.dev(a), g.dev(x)
    y = g.host(lib.nf4_linear(xd, qd, ad, block=block))
    y1 = g.host(lib.nf4_linear(xd[:32].contiguous(), qd, ad, block=block, path=3))
    y2 = g.host(lib.nf4_linear(xd[32:].contiguous(), qd, ad, block=block, path=3))
    assert np.array_equal(y.view(np.uint16), np.concatenate([y1, y2]).view(np.uint16))


@pytest.mark.parametrize("block", [64, 32])
@pytest.mark.parametrize("k", [384, 512])
def test_nf4_mfma_64_row_tiles(lib, block, k):
    # M = 512, N = 4096: 512 tiles of 64 rows (the tiled kernel's 64-row tiles and load ring);
    # K = 384 is not a multiple of the ring; every output compared
    qw, a = oracle.quantize_pack_nf4(synth.weights(3, 9, 4096, k), None, block)
    x = synth.activations(3, 9, 512, k)
    _nf4_linear_check(lib, x, qw, a, block, 2, "mfma-64-row-tiles")


@pytest.mark.parametrize("path", [0, 1])
def test_nf4_gemv_long_row_one_token(lib, path):
    # M = 1, K = 65536 on a layer under 2^26 weights: the tuned GEMV's NF4 form takes it
    qw, a = oracle.quantize_pack_nf4(synth.weights(3, 10, 40, 65536), None, 64)
    x = synth.activations(3, 10, 1, 65536)
    _nf4_linear_check(lib, x, qw, a, 64, path, "gemv-long-one-token")


@pytest.mark.parametrize("n,k,m,path", [(22016, 8192, 2, 3), (8192, 8192, 2, 3), (8192, 22016, 1, 1), (2048, 2048, 1, 1)])
def test_nf4_auto_route(lib, n, k, m, path):
    # the automatic choice for NF4: the GEMV at M = 1, the small-batch kernel at M = 2 (bit-identical
    # to forcing it). Random codes and absmax: this checks the route, not the kernels' parity.
    g = _gpu()
    rng = np.random.default_rng(3)
    qw = rng.integers(-2**31, 2**31, size=(n, k // 8), dtype=np.int64).astype(np.int32)
    am = rng.uniform(1e-3, 1e-2, size=(n, k // 64)).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float16)
    dev = [g.dev(t) for t in (x, qw, am)]
    print(f"nf4 auto route M={m} N={n} K={k} -> path {path}", flush=True)
    a = g.host(lib.nf4_linear(*dev, block=64))
    b = g.host(lib.nf4_linear(*dev, block=64, path=path))
    assert np.array_equal(g.bits16(a), g.bits16(b))
