"""The library's launches inside captured HIP graphs.

Decode loops run their launches as graph replays (the benchmark times its steps that way).
Each entry point is captured into a graph that writes its own output buffers, then replayed
several times. The inputs are rewritten by ordinary eager work between the replays, with
synchronizations. Every replay must reproduce, bit for bit, what the same call gives
eagerly on the same inputs. No entry point records a memset, and the split-K workspace is
fully overwritten by each call, so nothing may carry over from one replay to the next.
"""

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _torch():
    import torch

    return torch


def _gpu():
    from tests import _gpu

    return _gpu


def _replay_and_compare(torch, capture, inputs, outputs, make_inputs, eager, replays=3):
    """capture(): launches writing `outputs`; make_inputs(i) -> new input arrays for replay i;
    eager(): the same launches as fresh eager calls, returning new tensors."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        capture()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        capture()
    for i in range(replays):
        for dst, src in zip(inputs, make_inputs(i)):
            dst.copy_(torch.from_numpy(np.ascontiguousarray(src)).to(dst.device))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = eager()
        torch.cuda.synchronize()
        for got, exp in zip(outputs, want):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.float16 else got,
                               exp.view(torch.int16) if exp.dtype == torch.float16 else exp), i


@pytest.mark.parametrize("m,n", [(1, 1000), (2, 1000), (4, 1000), (40, 1000), (128, 1000), (512, 4096)])
def test_linear_in_graph(lib, m, n):
    # (512, 4096): the automatic path takes the one-range split-K kernel (256 tiles of 64 x 128)
    torch, g = _torch(), _gpu()
    k = 4096
    packed = [g.dev(t) for t in oracle.quantize_pack(synth.weights(2, 11, n, k))]
    x = g.dev(synth.activations(2, 11, m, k))
    y = torch.empty((m, n), dtype=torch.float16, device=x.device)
    print(f"graph linear M={m}", flush=True)
    _replay_and_compare(
        torch,
        lambda: lib.linear(x, *packed, out=y),
        [x], [y],
        lambda i: [synth.activations(2, 20 + i, m, k)],
        lambda: [lib.linear(x, *packed)])
    # and the replayed result is the oracle's, within tolerance
    y_ref, b = oracle.linear(g.host(x), g.host_u32(packed[0]), g.host(packed[1]), g.host(packed[2]))
    assert np.all(oracle.within_tolerance(g.host(y).astype(np.float64), y_ref, b))


@pytest.mark.parametrize("m,group", [(8, 128), (24, 128), (16, 64)])
def test_x_resident_in_graph(lib, m, group):
    # 4096 -> 11008: the automatic path with the binding's workspace (allocated inside the
    # capture) runs the x-resident kernel and its range reduction; its own entry point with a
    # caller workspace too. 64-column four-wave workgroups at M = 8, 128-column eight-wave ones
    # at M = 24; groups of 64 at M = 16
    torch, g = _torch(), _gpu()
    k, n = 4096, 11008
    assert lib.linear_ws_kernel(m, n, k, group=group) == 2
    packed = [g.dev(t) for t in oracle.quantize_pack(synth.weights(2, 13, n, k), group=group)]
    x = g.dev(synth.activations(2, 13, m, k))
    y = torch.empty((m, n), dtype=torch.float16, device=x.device)
    y2 = torch.empty((m, n), dtype=torch.float16, device=x.device)
    ws = torch.empty(lib.xres_workspace_bytes(m, n, k) // 4, dtype=torch.float32, device=x.device)
    print(f"graph x-resident M={m} group={group}", flush=True)

    def capture():
        lib.linear(x, *packed, out=y, group=group)
        lib.linear_xres(x, *packed, workspace=ws, out=y2, group=group)

    _replay_and_compare(
        torch, capture, [x], [y, y2],
        lambda i: [synth.activations(2, 40 + i, m, k)],
        lambda: [lib.linear(x, *packed, group=group), lib.linear_xres(x, *packed, group=group)])
    y_ref, b = oracle.linear(g.host(x), g.host_u32(packed[0]), g.host(packed[1]), g.host(packed[2]), group=group)
    assert np.all(oracle.within_tolerance(g.host(y).astype(np.float64), y_ref, b))


def test_splitk_in_graph(lib):
    torch, g = _torch(), _gpu()
    m, k, n = 128, 4096, 1000
    packed = [g.dev(t) for t in oracle.quantize_pack(synth.weights(2, 12, n, k))]
    x = g.dev(synth.activations(2, 12, m, k))
    ws = torch.empty(lib.splitk_workspace_bytes(m, n, k, 4) // 4, dtype=torch.float32, device=x.device)
    y = torch.empty((m, n), dtype=torch.float16, device=x.device)
    print("graph split-K", flush=True)
    _replay_and_compare(
        torch,
        lambda: lib.linear_splitk(x, *packed, splits=4, workspace=ws, out=y),
        [x], [y],
        lambda i: [synth.activations(2, 30 + i, m, k)],
        lambda: [lib.linear_splitk(x, *packed, splits=4)])


def test_quantize_and_norm_in_graph(lib):
    torch, g = _torch(), _gpu()
    n, k, m = 300, 2048, 3
    W = g.dev(synth.weights(2, 13, n, k))
    x_cal = g.dev(synth.calibration(2, 13, k))
    s = torch.empty(k, dtype=torch.float32, device=W.device)
    qout = (torch.empty((n, k // 8), dtype=torch.int32, device=W.device),
            torch.empty((n, k // 128), dtype=torch.float16, device=W.device),
            torch.empty((n, k // 128), dtype=torch.float16, device=W.device))
    rng = np.random.default_rng(14)
    h = g.dev(rng.standard_normal((m, k)).astype(np.float16))
    gamma = g.dev((1 + 0.1 * rng.standard_normal(k)).astype(np.float16))
    xs = torch.empty((m, k), dtype=torch.float16, device=W.device)

    def capture():
        lib.channel_scale(x_cal, 0.5, out=s)
        lib.quantize_pack(W, s, out=qout)
        lib.rmsnorm_fold(h, gamma, s, 1e-5, out=xs)

    def eager():
        s2 = lib.channel_scale(x_cal, 0.5)
        q2 = lib.quantize_pack(W, s2)
        return [s2, *q2, lib.rmsnorm_fold(h, gamma, s2, 1e-5)]

    print("graph quantize + norm", flush=True)
    _replay_and_compare(
        torch, capture, [W, x_cal, h], [s, *qout, xs],
        lambda i: [synth.weights(2, 40 + i, n, k), synth.calibration(2, 40 + i, k),
                   np.random.default_rng(50 + i).standard_normal((m, k)).astype(np.float16)],
        eager)


@pytest.mark.parametrize("bits,group", [(4, 64), (3, 32)])
@pytest.mark.parametrize("m", [1, 4, 40])
def test_formats_in_graph(lib, bits, group, m):
    # the GEMV variant (M = 1), the small-batch kernel (M = 4) and its two passes (M = 40)
    torch, g = _torch(), _gpu()
    k, n = 2048, 600
    packed = [g.dev(t) for t in oracle.quantize_pack(synth.weights(2, 15, n, k), None, bits=bits, group=group)]
    x = g.dev(synth.activations(2, 15, m, k))
    y = torch.empty((m, n), dtype=torch.float16, device=x.device)
    print(f"graph linear bits={bits} group={group} M={m}", flush=True)
    _replay_and_compare(
        torch,
        lambda: lib.linear(x, *packed, group=group, bits=bits, out=y),
        [x], [y],
        lambda i: [synth.activations(2, 60 + i, m, k)],
        lambda: [lib.linear(x, *packed, group=group, bits=bits)])


@pytest.mark.parametrize("m", [4, 40])
def test_nf4_in_graph(lib, m):
    torch, g = _torch(), _gpu()
    k, n = 2048, 600
    qw, a = oracle.quantize_pack_nf4(synth.weights(2, 16, n, k), None, 64)
    qd, ad = g.dev(qw), g.dev(a)
    x = g.dev(synth.activations(2, 16, m, k))
    y = torch.empty((m, n), dtype=torch.float16, device=x.device)
    print(f"graph nf4 M={m}", flush=True)
    _replay_and_compare(
        torch,
        lambda: lib.nf4_linear(x, qd, ad, block=64, out=y),
        [x], [y],
        lambda i: [synth.activations(2, 70 + i, m, k)],
        lambda: [lib.nf4_linear(x, qd, ad, block=64)])
