"""The split-K GEMM without a caller workspace (w4a16_linear_splitk_noalloc): its partials go
to the library's static per-GPU scratch. Checked through the C ABI against the same kernels
with a caller workspace (w4a16_linear_splitk): bit-identical outputs, on two calls in a row
(the second with a smaller input, which must not see the first call's scratch contents),
then the first shape again; and against the float64 oracle."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _layer(m, n, k, seed):
    rng = np.random.default_rng(seed)
    W = (0.02 * rng.standard_normal((n, k))).astype(np.float16)
    x = rng.standard_normal((m, k)).astype(np.float16)
    qw, sc, zr = oracle.quantize_pack(W, None)
    return x, (qw, sc, zr)


def test_noalloc_matches_workspace_entry_point(lib):
    from tests import _gpu as g
    import torch

    shapes = [((256, 4096, 4096), 0), ((65, 129, 1408), 3), ((256, 4096, 4096), 0)]
    cache = {}
    for (m, n, k), splits in shapes:
        print(f"no-alloc split-K M={m} N={n} K={k} splits={splits}", flush=True)
        if (m, n, k) not in cache:
            cache[(m, n, k)] = _layer(m, n, k, m + n + k)
        x, packed = cache[(m, n, k)]
        xd = g.dev(x)
        pd = [g.dev(t) for t in packed]
        y_ws = lib.linear_splitk(xd, *pd, splits=splits)
        y_na = torch.empty((m, n), dtype=torch.float16, device="cuda:0")
        out = lib.linear_splitk_noalloc(xd, *pd, out=y_na, splits=splits)
        assert out.data_ptr() == y_na.data_ptr()
        torch.cuda.synchronize()
        a, b = g.host(y_ws).view(np.uint16), g.host(y_na).view(np.uint16)
        assert np.array_equal(a, b), g.report_mismatch("no-alloc vs workspace", b, a)
        rows = np.arange(0, n, max(1, n // 64))
        y_ref, bound = oracle.linear(x, *packed, rows=rows)
        ok = oracle.within_tolerance(g.host(y_na)[:, rows].astype(np.float64), y_ref, bound)
        assert ok.all()


def test_noalloc_refuses_beyond_scratch(lib):
    import torch

    from tests import _gpu as g

    x = torch.zeros((256, 4096), dtype=torch.float16, device="cuda:0")
    qw = torch.zeros((11008, 512), dtype=torch.int32, device="cuda:0")
    sz = torch.zeros((11008, 32), dtype=torch.float16, device="cuda:0")
    y = torch.empty((256, 11008), dtype=torch.float16, device="cuda:0")
    with pytest.raises(lib.W4A16Error):
        lib.linear_splitk_noalloc(x, qw, sz, sz, out=y, splits=4)
