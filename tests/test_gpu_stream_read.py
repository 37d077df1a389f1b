"""The stream-read measurement aid reads every 16-byte piece of its buffer once: a sink word
is written only where one thread's words XOR to the magic value, so planting that value in
single pieces shows which workgroup read them (the split documented in include/w4a16.h:
W = max(min(1024, ceil(P/256)), ceil(P/4096)) workgroups of ceil(P/W) pieces)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _split(pieces):
    w = max(min(1024, -(-pieces // 256)), -(-pieces // 4096))
    chunk = -(-pieces // w)
    return -(-pieces // chunk), chunk


@pytest.mark.parametrize("nbytes", [32768 * 3, 32768 * 2 + 16 * 37, 16, 35684352])
def test_stream_read_reads_every_piece(lib, nbytes):
    import torch

    pieces = nbytes // 16
    blocks, chunk = _split(pieces)
    print(f"stream read bytes={nbytes}", flush=True)
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.full((blocks,), 7, dtype=torch.int32, device="cuda:0")
    lib.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert (sink.cpu().numpy() == 7).all()  # every XOR is 0: nothing written
    for p in sorted(q for q in {0, chunk - 1, chunk, pieces // 2, pieces - 1} if q < pieces):
        word = 4 * p + (p % 4)  # any of the piece's four words
        buf.zero_()
        buf[word] = lib.STREAM_READ_MAGIC
        sink.fill_(7)
        lib.stream_read(buf, sink)
        torch.cuda.synchronize()
        want = np.full(blocks, 7, dtype=np.int32)
        want[p // chunk] = lib.STREAM_READ_MAGIC
        assert np.array_equal(sink.cpu().numpy(), want), p


@pytest.mark.parametrize("nbytes,threads,blocks,unroll", [
    (35684352, 256, 1024, 4),     # more tiles than workgroups: the grid-stride loop runs
    (35684352, 1024, 256, 8),
    (16 * 1000 + 16 * 37, 64, 3, 2),  # ragged last tile
    (16, 128, 4, 16),             # one piece, workgroups with nothing to read
])
def test_stream_read_grid_reads_every_piece(lib, nbytes, threads, blocks, unroll):
    import torch

    pieces = nbytes // 16
    tile = threads * unroll
    print(f"grid read bytes={nbytes} threads={threads} blocks={blocks} unroll={unroll}", flush=True)
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.full((blocks,), 7, dtype=torch.int32, device="cuda:0")
    lib.stream_read_grid(buf, threads, blocks, unroll, sink)
    torch.cuda.synchronize()
    assert (sink.cpu().numpy() == 7).all()
    for p in sorted(q for q in {0, tile - 1, tile, pieces // 2, pieces - 1} if q < pieces):
        buf.zero_()
        buf[4 * p + (p % 4)] = lib.STREAM_READ_MAGIC
        sink.fill_(7)
        lib.stream_read_grid(buf, threads, blocks, unroll, sink)
        torch.cuda.synchronize()
        want = np.full(blocks, 7, dtype=np.int32)
        want[(p // tile) % blocks] = lib.STREAM_READ_MAGIC
        assert np.array_equal(sink.cpu().numpy(), want), p
