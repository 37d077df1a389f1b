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

3-bit codes (the Lab 4 setting of the "MIT 6.5940 Lab 4 + Lab 5" guide, 3-bit
with groups of 128; the L13 AWQ section's INT3 g128 example) use the same idea in
bit-plane form, so that a pair of codes still ORs straight into an fp16 pair:

* qweight is uint32 [N][3K/32]; the 32 inputs k = 32b .. 32b+31 of row n own
  words 3b, 3b+1, 3b+2;
* word 3b + h (h = 0, 1) holds the low two bits of the codes of inputs
  32b + 16h .. 32b + 16h + 15: bits 2i .. 2i+1 (i = 0..7) hold q[32b+16h+2i] & 3,
  bits 16+2i .. 16+2i+1 hold q[32b+16h+2i+1] & 3;
* word 3b + 2 holds the high bit of all 32: bit i (i = 0..15) is q[32b+2i] >> 2,
  bit 16+i is q[32b+2i+1] >> 2.

So ((lo >> 2i) & 0x00030003) | (((hi >> j) & 0x00010001) << 2) is the code pair of
inputs (2j, 2j+1) of the block, j = 8h + i. The worked words for q[i] = i mod 8,
i = 0..31, are 0xDDDD8888, 0xDDDD8888, 0xCCCCCCCC.

These packers are written from that text alone and share no code with the
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


def pack_codes3(q):
    """Pack integer codes q [N][K] (values 0..7, K % 32 == 0) into the 3-bit layout."""
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[1] % 32 != 0:
        raise ValueError("codes must be [N][K] with K % 32 == 0")
    if q.size and (q.min() < 0 or q.max() > 7):
        raise ValueError("codes must lie in [0, 7]")
    n, k = q.shape
    c = q.astype(np.uint32).reshape(n, k // 32, 32)
    lo = c & np.uint32(3)
    hi = c >> np.uint32(2)
    words = np.zeros((n, k // 32, 3), dtype=np.uint32)
    for h in range(2):
        for i in range(8):
            words[:, :, h] |= lo[:, :, 16 * h + 2 * i] << np.uint32(2 * i)
            words[:, :, h] |= lo[:, :, 16 * h + 2 * i + 1] << np.uint32(16 + 2 * i)
    for i in range(16):
        words[:, :, 2] |= hi[:, :, 2 * i] << np.uint32(i)
        words[:, :, 2] |= hi[:, :, 2 * i + 1] << np.uint32(16 + i)
    return words.reshape(n, 3 * (k // 32))


def unpack_codes3(qweight, k=None):
    """Inverse of ``pack_codes3``: uint32 [N][3K/32] -> int64 codes [N][K]."""
    w = np.asarray(qweight, dtype=np.uint32)
    if w.ndim != 2 or w.shape[1] % 3 != 0:
        raise ValueError("qweight must be [N][3K/32]")
    n, kw = w.shape
    blocks = kw // 3
    if k is not None and k != 32 * blocks:
        raise ValueError("K does not match qweight")
    w = w.reshape(n, blocks, 3)
    out = np.empty((n, blocks, 32), dtype=np.int64)
    for h in range(2):
        for i in range(8):
            out[:, :, 16 * h + 2 * i] = (w[:, :, h] >> np.uint32(2 * i)) & np.uint32(3)
            out[:, :, 16 * h + 2 * i + 1] = (w[:, :, h] >> np.uint32(16 + 2 * i)) & np.uint32(3)
    for i in range(16):
        out[:, :, 2 * i] |= ((w[:, :, 2] >> np.uint32(i)) & np.uint32(1)).astype(np.int64) << 2
        out[:, :, 2 * i + 1] |= ((w[:, :, 2] >> np.uint32(16 + i)) & np.uint32(1)).astype(np.int64) << 2
    return out.reshape(n, 32 * blocks)
