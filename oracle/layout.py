"""Oracle: layout v1 of the packed 4-bit codes (packer and unpacker).

Test infrastructure only; see the package docstring.

The pages give the principle only: TinyChat reorders 4-bit weights offline so
that one AND plus a shift unpacks them at run time ("MIT 6.5940 L13 LLM
Deployment" guide, TinyChat, hardware-aware packing, slide 36), and the Lab 5
guide ("why reorder 4-bit weights first") shows the CPU interleavings that
put w_i and w_{i+16} (ARM) or w_i and w_{i+32} (x86) side by side. Layout v1
applies the same idea to fp16 pairs:

* qweight is uint32 [N][K/8], row-major, little-endian; word j of row n holds
  the codes of inputs k = 8j .. 8j+7.
* nibble i (bits 4i .. 4i+3, i = 0..3) holds q[8j + 2i];
  nibble i+4 (bits 16+4i .. 16+4i+3) holds q[8j + 2i + 1].

So (word >> 4i) & 0x000F000F yields the pair (q[8j+2i], q[8j+2i+1]) in its low
and high 16-bit halves, the same order as an fp16 input pair. The worked word
for q = 0, 1, ..., 7 is 0x75316420.

This packer is written from that text alone and shares no code with the
device kernels.
"""

import numpy as np

LAYOUT_VERSION = 1


def pack_codes(q):
    """Pack integer codes q [N][K] (values 0..15, K % 8 == 0) into layout v1."""
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[1] % 8 != 0:
        raise ValueError("codes must be [N][K] with K % 8 == 0")
    if q.size and (q.min() < 0 or q.max() > 15):
        raise ValueError("codes must lie in [0, 15]")
    n, k = q.shape
    c = q.astype(np.uint32).reshape(n, k // 8, 8)
    word = np.zeros((n, k // 8), dtype=np.uint32)
    for i in range(4):
        word |= c[:, :, 2 * i] << np.uint32(4 * i)
        word |= c[:, :, 2 * i + 1] << np.uint32(16 + 4 * i)
    return word


def unpack_codes(qweight, k=None):
    """Inverse of ``pack_codes``: uint32 [N][K/8] -> int64 codes [N][K]."""
    w = np.asarray(qweight, dtype=np.uint32)
    if w.ndim != 2:
        raise ValueError("qweight must be [N][K/8]")
    n, kw = w.shape
    if k is not None and k != 8 * kw:
        raise ValueError("K does not match qweight")
    out = np.empty((n, kw, 8), dtype=np.int64)
    for i in range(4):
        out[:, :, 2 * i] = (w >> np.uint32(4 * i)) & np.uint32(0xF)
        out[:, :, 2 * i + 1] = (w >> np.uint32(16 + 4 * i)) & np.uint32(0xF)
    return out.reshape(n, 8 * kw)
