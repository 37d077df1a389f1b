"""The Python binding refuses output and workspace tensors the kernels could not safely write
through (wrong shape, dtype, device or layout) with an exception, before any launch."""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def test_bad_out_and_workspace_tensors_are_refused(lib):
    import torch

    from tests import _gpu as g

    m, k, n = 4, 256, 64
    packed = [g.dev(t) for t in oracle.quantize_pack(synth.weights(1, 15, n, k))]
    x = g.dev(synth.activations(1, 15, m, k))
    dev = x.device
    good = torch.empty((m, n), dtype=torch.float16, device=dev)
    lib.linear(x, *packed, out=good)  # accepted
    bad = [torch.empty((m, n + 1), dtype=torch.float16, device=dev),     # shape
           torch.empty((n, m), dtype=torch.float16, device=dev),         # transposed shape
           torch.empty((m, n), dtype=torch.float32, device=dev),         # dtype
           torch.empty((n, m), dtype=torch.float16, device=dev).t(),     # not contiguous
           torch.empty((m, n), dtype=torch.float16)]                     # host memory
    for out in bad:
        with pytest.raises((ValueError, TypeError)):
            lib.linear(x, *packed, out=out)
    with pytest.raises((ValueError, TypeError)):
        lib.channel_scale(x, 0.5, out=torch.empty(k + 8, dtype=torch.float32, device=dev))
    with pytest.raises((ValueError, TypeError)):
        lib.quantize_pack(g.dev(synth.weights(1, 15, n, k)),
                          out=(packed[0], packed[1], torch.empty((n, 1), dtype=torch.float16, device=dev)))
    with pytest.raises(ValueError):
        lib.quantize_pack(g.dev(synth.weights(1, 15, n, k)), out=(packed[0], packed[1]))
    ws_host = torch.empty(lib.splitk_workspace_bytes(m, n, k, 2) // 4, dtype=torch.float32)
    with pytest.raises(ValueError):
        lib.linear_splitk(x, *packed, splits=2, workspace=ws_host)
    ws64 = torch.empty(lib.splitk_workspace_bytes(m, n, k, 2) // 8, dtype=torch.float64, device=dev)
    with pytest.raises(ValueError):
        lib.linear_splitk(x, *packed, splits=2, workspace=ws64)
    # the automatic path's workspace: a float32 tensor on the same device, or "auto" / None
    for ws in (ws_host, ws64, "scratch"):
        with pytest.raises(ValueError):
            lib.linear(x, *packed, workspace=ws)
    torch.cuda.synchronize()
    # nothing was written through the refused tensors' pointers: the accepted output is intact
    want = lib.linear(x, *packed)
    assert torch.equal(good.view(torch.int16), want.view(torch.int16))
    assert np.isfinite(g.host(want).astype(np.float64)).all()
