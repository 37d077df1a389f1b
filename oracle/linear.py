"""Oracle: dequantize and the W4A16 linear layer, in float64.

Test infrastructure only; see the package docstring.

What it follows:

* "MIT 6.5940 L13 LLM Deployment" guide, TinyChat, kernel fusion (slide 37):
  the dequantization is fused with the matrix multiply; weights come back as
  w_hat = (q - z) * Delta. QServe table: W4-A16, weights 4-bit per group of
  128, activations fp16.
* "CMU 11-868 Model Quantization" guide, "where the speed comes from": single
  batch inference is a GEMV that is memory-bound; the computation itself is
  unchanged (weights are restored before the multiply).
* "Quantization for LLMs" chapter 11, section 11.1: W4A16 keeps the multiply in
  fp16; section 11.3: Y = X W^T.

The dequant uses the *stored* fp16 scale and zero, i.e. exactly what a device
kernel reads. y_ref[m, n] = sum_k x[m, k] * w_hat[n, k] and
B[m, n] = sum_k |x[m, k] * w_hat[n, k]| are float64 (numpy matmul). The
acceptance rule for any device result y is
|y - y_ref| <= TOL_REL * B + TOL_ABS.
"""

import numpy as np

from .layout import unpack_codes, unpack_codes3

TOL_REL = 1e-3
TOL_ABS = 1e-5

_ROW_BLOCK = 512


def dequantize(qweight, scales, zeros, k, group=128, bits=4):
    """w_hat[n, k] = (q[n, k] - zero[n, g]) * scale[n, g], float64 [N][K].

    qweight is in layout v1 (bits = 4) or the 3-bit bit-plane layout (bits = 3).
    """
    if bits not in (3, 4):
        raise ValueError("bits must be 3 or 4")
    q = (unpack_codes(qweight, k) if bits == 4 else unpack_codes3(qweight, k)).astype(np.float64)
    n = q.shape[0]
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    z = np.asarray(zeros, dtype=np.float16).astype(np.float64)
    g = k // group
    if s.shape != (n, g) or z.shape != (n, g):
        raise ValueError("scales/zeros must be [N][K/group]")
    w = (q.reshape(n, g, group) - z[:, :, None]) * s[:, :, None]
    return w.reshape(n, k)


def linear(x, qweight, scales, zeros, group=128, rows=None, bits=4):
    """y_ref = x @ w_hat^T and B = |x| @ |w_hat|^T, both float64 [M][N].

    x: float16 [M][K] (the input after the 1/s fold). ``rows`` optionally
    selects output rows n (for sampled checks on full-size layers); the result
    then has one column per selected row.
    """
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    if x64.ndim != 2:
        raise ValueError("x must be [M][K]")
    k = x64.shape[1]
    qweight = np.asarray(qweight, dtype=np.uint32)
    scales = np.asarray(scales, dtype=np.float16)
    zeros = np.asarray(zeros, dtype=np.float16)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        qweight, scales, zeros = qweight[rows], scales[rows], zeros[rows]
    n = qweight.shape[0]
    y = np.empty((x64.shape[0], n), dtype=np.float64)
    b = np.empty((x64.shape[0], n), dtype=np.float64)
    ax = np.abs(x64)
    for r0 in range(0, n, _ROW_BLOCK):
        r1 = min(n, r0 + _ROW_BLOCK)
        w = dequantize(qweight[r0:r1], scales[r0:r1], zeros[r0:r1], k, group, bits)
        y[:, r0:r1] = x64 @ w.T
        b[:, r0:r1] = ax @ np.abs(w).T
    return y, b


F16_OVERFLOW = 65520.0  # the least magnitude that rounds to infinity in binary16


def within_tolerance(y, y_ref, bound):
    """Boolean mask of |y - y_ref| <= TOL_REL * B + TOL_ABS (float64).

    Reading R11: y is stored as fp16 (round to nearest even), so an output whose
    exact value, widened by the tolerance, reaches the fp16 overflow threshold
    may also be the infinity of the same sign.
    """
    y = np.asarray(y, dtype=np.float64)
    tol = TOL_REL * bound + TOL_ABS
    ok = np.abs(y - y_ref) <= tol
    overflow = np.isinf(y) & (np.sign(y) == np.sign(y_ref)) & (np.abs(y_ref) + tol >= F16_OVERFLOW)
    return ok | overflow
