"""GPU parity of the other code formats: 3-bit codes (packed 3-bit layout) and groups of
32 and 64, against the float64 oracle.

* quantize-pack: codes, scales and zeros bit-identical to the oracle's for bits 3/4 and
  groups 32/64/128, on ragged and full-size layers and on the edge tensors;
* the linear layer: every output within 1e-3 * sum_k |x * w_hat| + 1e-5 of the oracle, on
  every kernel (the GEMV variant for M <= 8, the small-batch MFMA kernel at
  M <= 32, the tiled MFMA variant for any M), fed the oracle's packed weights.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

FORMATS = [(4, 64), (4, 32), (3, 128), (3, 64), (3, 32)]


def _gpu():
    from tests import _gpu

    return _gpu


def _torch():
    import torch

    return torch


def _qp_compare(lib, W, s, bits, group, tag):
    g = _gpu()
    print(f"quantize-pack {tag} bits={bits} group={group} N={W.shape[0]} K={W.shape[1]}", flush=True)
    got = lib.quantize_pack(g.dev(W), None if s is None else g.dev(s), bits=bits, group=group)
    want = oracle.quantize_pack(W, s, bits=bits, group=group)
    gq = g.host_u32(got[0])
    assert np.array_equal(gq, want[0]), g.report_mismatch("qweight", gq, want[0])
    for name, a, b in (("scales", got[1], want[1]), ("zeros", got[2], want[2])):
        ab = g.bits16(g.host(a))
        bb = g.bits16(b)
        assert np.array_equal(ab, bb), g.report_mismatch(name, ab, bb)


@pytest.mark.parametrize("bits,group", FORMATS + [(4, 128)])
@pytest.mark.parametrize("n,k", [(37, 384), (300, 2048), (64, 11008)])
def test_quantize_pack_bit_exact(lib, bits, group, n, k):
    W = synth.weights(2, 3, n, k)
    s = oracle.channel_scale(synth.calibration(2, 3, k))
    _qp_compare(lib, W, s, bits, group, "scaled")
    _qp_compare(lib, W, None, bits, group, "plain")


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("kind", ["ties", "constant", "positive", "negative", "subnormal", "wide", "mixed"])
def test_quantize_pack_edge_tensors(lib, bits, group, kind):
    W = synth.edge_weights(kind, 40, 512, seed=5)
    _qp_compare(lib, W, None, bits, group, kind)


@pytest.mark.parametrize("bits,group", FORMATS)
def test_quantize_pack_full_layer_sampled_rows(lib, bits, group):
    # LLaMA-65B q projection, 8192 x 8192: packed on the device in full, 64 rows compared
    g = _gpu()
    W = synth.weights(3, 0, 8192, 8192)
    s = oracle.channel_scale(synth.calibration(3, 0, 8192))
    print(f"quantize-pack full bits={bits} group={group}", flush=True)
    got = lib.quantize_pack(g.dev(W), g.dev(s), bits=bits, group=group)
    rows = np.linspace(0, 8191, 64).astype(int)
    want = oracle.quantize_pack(W[rows], s, bits=bits, group=group)
    assert np.array_equal(g.host_u32(got[0])[rows], want[0])
    assert np.array_equal(g.bits16(g.host(got[1])[rows]), g.bits16(want[1]))
    assert np.array_equal(g.bits16(g.host(got[2])[rows]), g.bits16(want[2]))


def _linear_check(lib, x, packed, bits, group, path, tag, rows=None):
    g = _gpu()
    m, k = x.shape
    print(f"linear {tag} bits={bits} group={group} path={path} M={m} N={packed[0].shape[0]} K={k}", flush=True)
    y = g.host(lib.linear(g.dev(x), *[g.dev(t) for t in packed], group=group, path=path, bits=bits))
    y_ref, b = oracle.linear(x, *packed, group=group, rows=rows, bits=bits)
    if rows is not None:
        y = y[:, rows]
    ok = oracle.within_tolerance(y.astype(np.float64), y_ref, b)
    assert np.all(ok), (tag, np.argwhere(~ok)[:3])


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("n,k", [(1, 128), (37, 384), (300, 2048), (97, 11008), (64, 22016), (40, 32768)])
def test_gemv_variant(lib, bits, group, m, n, k):
    if k > 16384 and m > 4:
        pytest.skip("the GEMV variant takes M <= 4 above K = 16384")
    x_cal = synth.calibration(2, 5, k)
    s = oracle.channel_scale(x_cal)
    packed = oracle.quantize_pack(synth.weights(2, 5, n, k), s, bits=bits, group=group)
    x = oracle.scale_input(synth.activations(2, 5, m, k), s)
    _linear_check(lib, x, packed, bits, group, 1, "gemv")


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("m", [1, 9, 17, 33, 100])
@pytest.mark.parametrize("n,k", [(37, 384), (300, 2048), (130, 11008)])
def test_mfma_variant(lib, bits, group, m, n, k):
    x_cal = synth.calibration(4, 6, k)
    s = oracle.channel_scale(x_cal)
    packed = oracle.quantize_pack(synth.weights(4, 6, n, k), s, bits=bits, group=group)
    x = oracle.scale_input(synth.activations(4, 6, m, k), s)
    _linear_check(lib, x, packed, bits, group, 2, "mfma")


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("m", [2, 3, 5, 8, 9, 13, 16, 17, 32])
@pytest.mark.parametrize("n,k", [(1, 128), (37, 384), (300, 2048), (97, 11008), (64, 22016), (40, 32768)])
def test_skinny_variant(lib, bits, group, m, n, k):
    # the small-batch MFMA kernel with 1, 2 or 4 (scale, zero) pairs per 128 inputs and 4- or
    # 3-bit codes: every x path (one, two, four or eight full-width x loads, and 16-row fragment
    # loads), one and two m-tiles, one chunk and several chunks of stages per wave, ragged N, K
    x_cal = synth.calibration(2, 15, k)
    s = oracle.channel_scale(x_cal)
    packed = oracle.quantize_pack(synth.weights(2, 15, n, k), s, bits=bits, group=group)
    x = oracle.scale_input(synth.activations(2, 15, m, k), s)
    _linear_check(lib, x, packed, bits, group, 3, "skinny")


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("m", [2, 8, 16, 32])
def test_skinny_variant_wide_layer(lib, bits, group, m):
    # N = 8200: 257 two-column tiles, so M > 4 takes two 16-column tiles per wave
    x_cal = synth.calibration(2, 16, 1024)
    s = oracle.channel_scale(x_cal)
    packed = oracle.quantize_pack(synth.weights(2, 16, 8200, 1024), s, bits=bits, group=group)
    x = oracle.scale_input(synth.activations(2, 16, m, 1024), s)
    _linear_check(lib, x, packed, bits, group, 3, "skinny-wide")


@pytest.mark.parametrize("bits,group", [(4, 64), (4, 32), (3, 64), (3, 32)])
def test_skinny_variant_misaligned_scales_fall_back(lib, bits, group):
    # scales and zeros at a 2-byte but not 4-byte aligned address: the automatic choice takes
    # another kernel, the explicit small-batch path refuses
    torch, g = _torch(), _gpu()
    n, k, m = 64, 1024, 4
    s = oracle.channel_scale(synth.calibration(2, 17, k))
    packed = oracle.quantize_pack(synth.weights(2, 17, n, k), s, bits=bits, group=group)
    x = oracle.scale_input(synth.activations(2, 17, m, k), s)

    def shifted(a):
        buf = torch.empty(a.size + 1, dtype=torch.float16, device="cuda")
        v = buf[1:].view(a.shape)
        v.copy_(torch.from_numpy(a).to(v.device))
        assert v.data_ptr() % 4 == 2
        return v

    sc, zr = shifted(packed[1]), shifted(packed[2])
    print(f"linear misaligned scales bits={bits} group={group}", flush=True)
    y = g.host(lib.linear(g.dev(x), g.dev(packed[0]), sc, zr, group=group, bits=bits))
    y_ref, b = oracle.linear(x, *packed, group=group, bits=bits)
    assert np.all(oracle.within_tolerance(y.astype(np.float64), y_ref, b))
    with pytest.raises(RuntimeError, match="aligned"):
        lib.linear(g.dev(x), g.dev(packed[0]), sc, zr, group=group, path=3, bits=bits)


def test_skinny_3bit_group128_takes_2byte_aligned_scales(lib):
    # with one scale per 128 inputs the small-batch kernel loads scales and zeros 2 bytes at a
    # time, so 2-byte alignment is enough on the explicit path
    torch, g = _torch(), _gpu()
    n, k, m = 64, 1024, 4
    s = oracle.channel_scale(synth.calibration(2, 18, k))
    packed = oracle.quantize_pack(synth.weights(2, 18, n, k), s, bits=3, group=128)
    x = oracle.scale_input(synth.activations(2, 18, m, k), s)
    bufs = []
    for a in packed[1:]:
        buf = torch.empty(a.size + 1, dtype=torch.float16, device="cuda")
        v = buf[1:].view(a.shape)
        v.copy_(torch.from_numpy(a).to(v.device))
        assert v.data_ptr() % 4 == 2
        bufs.append(v)
    print("linear 3-bit g128 2-byte aligned scales, path 3", flush=True)
    y = g.host(lib.linear(g.dev(x), g.dev(packed[0]), *bufs, group=128, path=3, bits=3))
    y_ref, b = oracle.linear(x, *packed, group=128, bits=3)
    assert np.all(oracle.within_tolerance(y.astype(np.float64), y_ref, b))


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("kind", ["positive", "negative", "mixed", "wide"])
def test_variants_on_edge_weights(lib, bits, group, kind):
    # one-signed groups quantized without the AWQ scale give zeros far outside the exact
    # fp16 (q - z) range, mixed with ordinary groups: the tiled kernel's general route, and
    # the small-batch kernel's zero term for any stored zero
    W = synth.edge_weights(kind, 96, 1024, seed=7)
    packed = oracle.quantize_pack(W, None, bits=bits, group=group)
    x = synth.activations(1, 8, 40, 1024)
    cases = ((1, 1), (1, 8), (2, 3), (2, 40), (3, 2), (3, 7), (3, 20))
    for path, m in cases:
        _linear_check(lib, x[:m], packed, bits, group, path, kind)


@pytest.mark.parametrize("bits,group", [(3, 128), (4, 32), (4, 64)])
@pytest.mark.parametrize("m", [1, 4, 16, 64])
def test_full_size_layers_sampled(lib, bits, group, m):
    # LLaMA-65B projections: 8192 -> 8192 and 8192 -> 22016, 256 sampled output rows
    g = _gpu()
    for lid, (name, k, n) in enumerate(synth.CONFIGS[synth.LLAMA65B_DECODE]["layers"][3:5]):
        x_cal = synth.calibration(3, lid, k)
        s = oracle.channel_scale(x_cal)
        W = synth.weights(3, lid, n, k)
        packed = tuple(g.host(t) for t in lib.quantize_pack(g.dev(W), g.dev(s), bits=bits, group=group))
        packed = (packed[0].view(np.uint32), packed[1], packed[2])
        x = oracle.scale_input(synth.activations(3, lid, m, k), s)
        rows = np.linspace(0, n - 1, 256).astype(int)
        _linear_check(lib, x, packed, bits, group, 0, f"full-{name}", rows=rows)


@pytest.mark.parametrize("bits,group", FORMATS)
def test_auto_dispatch_and_determinism(lib, bits, group):
    g = _gpu()
    k, n = 4096, 512
    s = oracle.channel_scale(synth.calibration(2, 9, k))
    packed = oracle.quantize_pack(synth.weights(2, 9, n, k), s, bits=bits, group=group)
    dev = [g.dev(t) for t in packed]
    for m in (1, 8, 9, 128):
        x = oracle.scale_input(synth.activations(2, 9, m, k), s)
        xd = g.dev(x)
        y1 = g.host(lib.linear(xd, *dev, group=group, bits=bits))
        y2 = g.host(lib.linear(xd, *dev, group=group, bits=bits))
        assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
        y_ref, b = oracle.linear(x, *packed, group=group, bits=bits)
        assert np.all(oracle.within_tolerance(y1.astype(np.float64), y_ref, b))


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("m", [40, 64])
@pytest.mark.parametrize("n,k", [(300, 2048), (97, 11008)])
def test_auto_two_small_batch_passes(lib, bits, group, m, n, k):
    # 33 <= M <= 64 on layers with N <= 8192 and K <= 16384: the automatic path runs the
    # small-batch kernel on rows 0..31 and then on the rest
    g = _gpu()
    s = oracle.channel_scale(synth.calibration(2, 19, k))
    packed = oracle.quantize_pack(synth.weights(2, 19, n, k), s, bits=bits, group=group)
    x = oracle.scale_input(synth.activations(2, 19, m, k), s)
    _linear_check(lib, x, packed, bits, group, 0, "auto-two-passes")
    dev = [g.dev(t) for t in packed]
    xd = g.dev(x)
    y = g.host(lib.linear(xd, *dev, group=group, bits=bits))
    y1 = g.host(lib.linear(xd[:32].contiguous(), *dev, group=group, bits=bits, path=3))
    y2 = g.host(lib.linear(xd[32:].contiguous(), *dev, group=group, bits=bits, path=3))
    assert np.array_equal(y.view(np.uint16), np.concatenate([y1, y2]).view(np.uint16))


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("k", [384, 512])
def test_mfma_variant_64_row_tiles(lib, bits, group, k):
    # M = 512, N = 4096: (512 / 64) * (4096 / 64) = 512 tiles of 64 rows, so the tiled variant
    # takes its 64-row tiles and their two-stage load ring; K = 384 (3 groups of 128) is not a
    # multiple of the ring. Every output is compared.
    m, n = 512, 4096
    x_cal = synth.calibration(4, 8, k)
    s = oracle.channel_scale(x_cal)
    packed = oracle.quantize_pack(synth.weights(4, 8, n, k), s, bits=bits, group=group)
    x = oracle.scale_input(synth.activations(4, 8, m, k), s)
    _linear_check(lib, x, packed, bits, group, 2, "mfma-64-row-tiles")


@pytest.mark.parametrize("bits,group", [(4, 64), (4, 32)])
@pytest.mark.parametrize("path", [0, 1])
def test_gemv_4bit_groups_long_row_one_token(lib, bits, group, path):
    # M = 1, K = 65536: beyond the GEMV variant's K, but the tuned GEMV takes 4-bit groups of
    # 64 and 32 there (eight pieces per thread); the automatic path must route it to that GEMV
    n, k = 40, 65536
    x_cal = synth.calibration(2, 9, k)
    s = oracle.channel_scale(x_cal)
    packed = oracle.quantize_pack(synth.weights(2, 9, n, k), s, bits=bits, group=group)
    x = oracle.scale_input(synth.activations(2, 9, 1, k), s)
    _linear_check(lib, x, packed, bits, group, path, "gemv-long-one-token")


@pytest.mark.parametrize("bits,group", FORMATS + [(4, 128)])
def test_skinny_variant_one_row(lib, bits, group):
    # the small-batch kernel forced at M = 1 (rows past M read as zero)
    n, k = 97, 11008
    x_cal = synth.calibration(4, 10, k)
    s = oracle.channel_scale(x_cal)
    packed = oracle.quantize_pack(synth.weights(4, 10, n, k), s, bits=bits, group=group)
    x = oracle.scale_input(synth.activations(4, 10, 1, k), s)
    _linear_check(lib, x, packed, bits, group, 3, "skinny-one-row")
