"""Oracle: symmetric absmax quantization of weight groups (float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The "CMU 11-868 Model Quantization" guide (L19, "absmax and zero-point") gives
the absmax quantizer: the scale comes from the largest magnitude of the tensor
and the values are scaled linearly onto the symmetric integer range (-127..127
for 8 bits) and rounded; the "MIT 6.5940 L13 LLM Deployment" guide (AWQ section,
slides 26/28) writes the same kind of quantizer as Q(w) = Delta * Round(w / Delta)
with Delta taken from max |w|.

Reading R15 (b-bit groups, where the pages give only the 8-bit tensor form):

    m     = max_k |w|  over the group (float64), replaced by 1 when it is 0
    Delta = m / (2^(b-1) - 1)                       (IEEE float64 division)
    q     = clip(rint(w / Delta), -(2^(b-1) - 1), 2^(b-1) - 1)

so the largest magnitude lands exactly on the end of the symmetric range (the
guide's absmax form, 127 for 8 bits), and the code range is symmetric. Stored in
the packed layouts as the unsigned code q + 2^(b-1) with a zero of 2^(b-1), so
the dequantized weight is (code - zero) * Delta: the same form the zero-point
quantizer uses, with a fixed zero.
"""

import numpy as np

from .quant import f64_to_f16


def quantize_groups_sym(w, bits=4, group=128):
    """Symmetric absmax codes of groups of `group` inputs.

    w: float64 [N][K]. Returns (q int64 [N][K] in [-(2^(b-1)-1), 2^(b-1)-1],
    delta float64 [N][K/g]).
    """
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    if k % group != 0:
        raise ValueError("K must be a multiple of the group size")
    qmax = float(2 ** (bits - 1) - 1)
    wg = w.reshape(n, k // group, group)
    m = np.abs(wg).max(axis=2)
    m = np.where(m == 0.0, 1.0, m)
    delta = m / qmax
    q = np.clip(np.rint(wg / delta[:, :, None]), -qmax, qmax)
    return q.astype(np.int64).reshape(n, k), delta


def quantize_pack_sym(W, s=None, bits=4, group=128):
    """Symmetric absmax quantize-pack of an nn.Linear weight (fp16 [N][K]).

    w = float64(W) * float64(s) (exact), then ``quantize_groups_sym``; stored as
    codes q + 2^(b-1) in layout v1 (bits 4) or the 3-bit layout (bits 3),
    scales = f16(Delta), zeros = 2^(b-1). Returns (qweight, scales, zeros) as
    ``quantize_pack`` does.
    """
    from .layout import pack_codes, pack_codes3

    W = np.asarray(W, dtype=np.float16)
    n, k = W.shape
    if bits not in (3, 4):
        raise ValueError("the packed layouts store 3-bit or 4-bit codes")
    w = W.astype(np.float64)
    if s is not None:
        w = w * np.asarray(s, dtype=np.float32).astype(np.float64)[None, :]
    q, delta = quantize_groups_sym(w, bits, group)
    off = 2 ** (bits - 1)
    qweight = (pack_codes if bits == 4 else pack_codes3)(q + off)
    zeros = np.full((n, k // group), off, dtype=np.float16)
    return qweight, f64_to_f16(delta), zeros
