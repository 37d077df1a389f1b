"""Exact weight rebuild on every kernel.

With one-hot inputs (x = 1 at one position per row of x), power-of-two scales and integer
zeros inside the code range, each output is a single weight (q - z) * d (or, for NF4, an
fp16 level times a power-of-two absmax). Every such value is exactly representable in
fp16, and every kernel forms it without rounding: the code -> fp16 rebuild is exact, the
products are exact and the sums only add zeros. So each path must return the oracle's
value bit for bit. A relative tolerance on long sums could not see a rebuild that is off
by a small relative amount; this test can, at every nibble position of a word, for both
halves of the fp16 pairs, and for every code value.
"""

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


def _gpu():
    from tests import _gpu

    return _gpu


def _weights(seed, n, k, bits=4, group=128):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 2**bits, size=(n, k))
    q[:, :2**bits] = np.arange(2**bits)  # every code value at the start of each row
    qw = oracle.pack_codes(q) if bits == 4 else oracle.pack_codes3(q)
    g = k // group
    sc = (2.0 ** rng.integers(-8, 1, size=(n, g))).astype(np.float16)
    zr = rng.integers(0, 2**bits, size=(n, g)).astype(np.float16)
    return qw, sc, zr


def _one_hot(cols, k):
    x = np.zeros((len(cols), k), np.float16)
    x[np.arange(len(cols)), cols] = 1.0
    return x


def _exact_ref(y_ref):
    y16 = y_ref.astype(np.float16)
    assert np.array_equal(y16.astype(np.float64), y_ref)  # the test's premise
    return y16


def _check(lib, x, packed, path, bits=4, group=128, tag=""):
    g = _gpu()
    y = g.host(lib.linear(g.dev(x), *[g.dev(t) for t in packed], group=group, path=path, bits=bits))
    want = _exact_ref(oracle.linear(x, *packed, group=group, bits=bits)[0])
    assert np.array_equal(g.bits16(y), g.bits16(want)), (tag, g.report_mismatch("y", g.bits16(y), g.bits16(want)))


@pytest.mark.parametrize("m", [1, 3, 8])
def test_gemv_every_position(lib, m):
    # N = 67: the last workgroup's tile is ragged, so rows past N sit in rotated slots
    n, k = 67, 256
    packed = _weights(1, n, k)
    print(f"exact GEMV M={m}", flush=True)
    for c0 in range(0, k, m):
        cols = [min(c, k - 1) for c in range(c0, c0 + m)]
        _check(lib, _one_hot(cols, k), packed, 1, tag=f"cols {cols}")


@pytest.mark.parametrize("k", [32768, 65536])
def test_gemv_long_rows(lib, k):
    # several pieces per thread: positions inside the first and the last pieces of a row
    n = 19
    packed = _weights(2, n, k)
    cols = list(range(0, 32)) + list(range(k // 2 - 16, k // 2 + 16)) + list(range(k - 32, k))
    m = 8 // (k // 16384)  # the GEMV takes M * ceil(K / 16384) <= 8
    print(f"exact GEMV K={k}", flush=True)
    for c0 in range(0, len(cols), m):
        _check(lib, _one_hot(cols[c0:c0 + m], k), packed, 1, tag=f"K={k} cols {cols[c0:c0 + m]}")


@pytest.mark.parametrize("m,path", [(2, 3), (32, 3), (64, 2), (33, 2), (64, 4), (33, 4), (128, 4)])
def test_mfma_paths_every_position(lib, m, path):
    n, k = 97, 256
    packed = _weights(3, n, k)
    print(f"exact path={path} M={m}", flush=True)
    for c0 in range(0, k, m):
        cols = [min(c, k - 1) for c in range(c0, c0 + m)]
        _check(lib, _one_hot(cols, k), packed, path, tag=f"cols {cols[:3]}...")


def test_splitk_every_position(lib):
    g = _gpu()
    n, k = 97, 512
    packed = _weights(4, n, k)
    print("exact split-K", flush=True)
    for c0 in range(0, k, 64):
        x = _one_hot(list(range(c0, c0 + 64)), k)
        want = _exact_ref(oracle.linear(x, *packed)[0])
        for splits in (2, 4):
            y = g.host(lib.linear_splitk(g.dev(x), *[g.dev(t) for t in packed], splits=splits))
            assert np.array_equal(g.bits16(y), g.bits16(want)), (c0, splits)


@pytest.mark.parametrize("m,group", [(16, 128), (32, 128), (16, 64), (32, 64)])
def test_xres_every_position(lib, m, group):
    # the x-resident kernel: K = 4352 is three K ranges (the last one of two 128-input blocks,
    # its other waves idle); every input position of the first range, and the last range's.
    # Groups of 64 pin the other k-to-lane order (each MFMA step 32 contiguous inputs)
    g = _gpu()
    n, k = 131, 4352
    packed = _weights(7, n, k, 4, group)
    dev = [g.dev(t) for t in packed]
    print(f"exact x-resident M={m} group={group}", flush=True)
    for c0 in list(range(0, 2048, m)) + list(range(4096, k, m)):
        x = _one_hot([min(c, k - 1) for c in range(c0, c0 + m)], k)
        y = g.host(lib.linear_xres(g.dev(x), *dev, group=group))
        want = _exact_ref(oracle.linear(x, *packed, group=group)[0])
        assert np.array_equal(g.bits16(y), g.bits16(want)), c0


@pytest.mark.parametrize("bits,group", [(3, 128), (4, 32), (4, 64), (3, 32)])
@pytest.mark.parametrize("m,path", [(8, 1), (64, 2)])
def test_variants_every_position(lib, bits, group, m, path):
    n, k = 41, 256
    packed = _weights(5, n, k, bits, group)
    print(f"exact bits={bits} group={group} path={path}", flush=True)
    for c0 in range(0, k, m):
        cols = [min(c, k - 1) for c in range(c0, c0 + m)]
        _check(lib, _one_hot(cols, k), packed, path, bits, group, tag=f"cols {cols[:3]}...")


@pytest.mark.parametrize("m,path", [(8, 1), (64, 2)])
def test_nf4_every_position(lib, m, path):
    g = _gpu()
    n, k, block = 41, 256, 64
    rng = np.random.default_rng(6)
    q = rng.integers(0, 16, size=(n, k))
    q[:, :16] = np.arange(16)
    qw = oracle.pack_codes(q)
    a = (2.0 ** rng.integers(-6, 3, size=(n, k // block))).astype(np.float32)
    print(f"exact NF4 path={path}", flush=True)
    for c0 in range(0, k, m):
        x = _one_hot([min(c, k - 1) for c in range(c0, c0 + m)], k)
        y = g.host(lib.nf4_linear(g.dev(x), g.dev(qw), g.dev(a), block=block, path=path))
        want = _exact_ref(oracle.linear_nf4(x, qw, a, block)[0])
        assert np.array_equal(g.bits16(y), g.bits16(want)), c0


@pytest.mark.parametrize("bits,group", [(3, 128), (4, 32), (4, 64), (3, 32), (3, 64)])
def test_variants_64_row_tiles_every_position(lib, bits, group):
    # M = 512, N = 4096: 512 tiles of 64 rows, the tiled variant's 64-row tiles and load ring;
    # row i of x is one-hot at input i % K, so one call rebuilds every input position
    n, k, m = 4096, 384, 512
    packed = _weights(7, n, k, bits, group)
    print(f"exact 64-row tiles bits={bits} group={group}", flush=True)
    _check(lib, _one_hot([i % k for i in range(m)], k), packed, 2, bits, group, tag="64-row tiles")


def test_nf4_64_row_tiles_every_position(lib):
    g = _gpu()
    n, k, m, block = 4096, 384, 512, 64
    rng = np.random.default_rng(8)
    q = rng.integers(0, 16, size=(n, k))
    q[:, :16] = np.arange(16)
    qw = oracle.pack_codes(q)
    a = (2.0 ** rng.integers(-6, 3, size=(n, k // block))).astype(np.float32)
    print("exact NF4 64-row tiles", flush=True)
    x = _one_hot([i % k for i in range(m)], k)
    y = g.host(lib.nf4_linear(g.dev(x), g.dev(qw), g.dev(a), block=block, path=2))
    want = _exact_ref(oracle.linear_nf4(x, qw, a, block)[0])
    assert np.array_equal(g.bits16(y), g.bits16(want))


@pytest.mark.parametrize("k", [128, 384, 1152])
def test_klane_every_position_ragged_k_lanes(lib, k):
    # the K-lane kernel with 1, 3 and 9 groups over its four K-lanes (lanes with no group, and
    # uneven ranges); row i of x is one-hot at input i % K, so one call rebuilds every input
    n, m = 97, 192
    packed = _weights(9, n, k)
    print(f"exact K-lane K={k}", flush=True)
    _check(lib, _one_hot([i % k for i in range(m)], k), packed, 4, tag=f"K-lane K={k}")
