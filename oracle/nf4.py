"""Oracle: the NormalFloat-4 codebook and blockwise absmax NF4 quantization (float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Quantization for LLMs" chapter 11, section 11.5 (NF4 and QLoRA): trained
weights are roughly normal; after dividing each block of 64 weights by the
block's largest magnitude they lie in [-1, 1]; NF4 puts its 16 levels at
quantiles of the standard normal so that each level carries about the same
share of the data: 8 positive levels at the quantiles of the probabilities from
`offset` down to 1/2 in 8 equal steps (the 1/2 end excluded), 7 negative levels
mirrored from 7 equal steps over the same range, an exact 0, all divided by the
largest level, with offset = 0.9677083. The section prints the resulting levels
to four decimals (the test fixture tests/golden/nf4_levels.txt). Each block
keeps its absmax as a float32 constant.

Readings (R16), where the section leaves the step open:

* the codebook a kernel multiplies with is the fp16 rounding of the levels
  (``LEVELS_F16``), code i naming the i-th level in ascending order;
* a = f32(max |w|) per block of `block` inputs of one row (block 64 as on the
  page); the code of w is the index of the fp16 level nearest to w / a (float64
  division), a tie at an exact midpoint going to the larger level; a block whose
  a is 0 stores a = 0 and the code of level 0;
* w_hat = float64(LEVELS_F16[code]) * float64(a); codes are packed in layout v1.
"""

import numpy as np
from scipy.stats import norm

from .quant import f64_to_f16

OFFSET = 0.9677083


def nf4_levels():
    """The 16 NF4 levels in ascending order, float64, from the quantile construction.

    Probability points: OFFSET - i (OFFSET - 1/2) / 8 for i = 0..7 give the positive
    levels, OFFSET - i (OFFSET - 1/2) / 7 for i = 0..6 the negative ones (mirrored);
    each level is the standard normal quantile of its point, then all are divided by
    the largest.
    """
    span = OFFSET - 0.5
    p_pos = np.array([OFFSET - i * span / 8.0 for i in range(8)])
    p_neg = np.array([OFFSET - i * span / 7.0 for i in range(7)])
    levels = [-norm.ppf(p) for p in p_neg] + [0.0] + [norm.ppf(p) for p in p_pos[::-1]]
    levels = np.array(levels, dtype=np.float64)  # ascending: most negative first
    return levels / norm.ppf(OFFSET)


LEVELS = nf4_levels()
LEVELS_F16 = f64_to_f16(LEVELS)
ZERO_CODE = int(np.flatnonzero(LEVELS == 0.0)[0])


def nf4_codes(v):
    """Index of the nearest fp16 NF4 level to each float64 value in [-1, 1] (ties upward)."""
    lv = LEVELS_F16.astype(np.float64)
    mids = (lv[:-1] + lv[1:]) / 2.0  # exact: fp16 values
    return np.searchsorted(mids, np.asarray(v, dtype=np.float64), side="right").astype(np.int64)


def quantize_nf4(W, s=None, block=64):
    """NF4 codes and float32 absmax of an nn.Linear weight (fp16 [N][K]).

    Returns (codes int64 [N][K], absmax float32 [N][K/block]).
    """
    W = np.asarray(W, dtype=np.float16)
    n, k = W.shape
    if k % block != 0:
        raise ValueError("K must be a multiple of the block size")
    w = W.astype(np.float64)
    if s is not None:
        w = w * np.asarray(s, dtype=np.float32).astype(np.float64)[None, :]
    wg = w.reshape(n, k // block, block)
    a = np.abs(wg).max(axis=2).astype(np.float32)
    a64 = a.astype(np.float64)
    safe = np.where(a64 == 0.0, 1.0, a64)
    codes = nf4_codes(wg / safe[:, :, None])
    codes = np.where((a64 == 0.0)[:, :, None], ZERO_CODE, codes)
    return codes.reshape(n, k), a


def quantize_pack_nf4(W, s=None, block=64):
    """NF4 codes packed in layout v1 and the float32 absmax per block."""
    from .layout import pack_codes

    codes, a = quantize_nf4(W, s, block)
    return pack_codes(codes), a


def dequantize_nf4(qweight, absmax, k, block=64):
    """w_hat = LEVELS_F16[code] * absmax, float64 [N][K]."""
    from .layout import unpack_codes

    codes = unpack_codes(qweight, k)
    n = codes.shape[0]
    a = np.asarray(absmax, dtype=np.float32).astype(np.float64)
    if a.shape != (n, k // block):
        raise ValueError("absmax must be [N][K/block]")
    lv = LEVELS_F16.astype(np.float64)[codes]
    return (lv.reshape(n, k // block, block) * a[:, :, None]).reshape(n, k)


def linear_nf4(x, qweight, absmax, block=64, rows=None):
    """y_ref = x @ w_hat^T and B = |x| @ |w_hat|^T (float64), as ``linear`` for NF4 weights."""
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    k = x64.shape[1]
    qweight = np.asarray(qweight, dtype=np.uint32)
    absmax = np.asarray(absmax, dtype=np.float32)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        qweight, absmax = qweight[rows], absmax[rows]
    w = dequantize_nf4(qweight, absmax, k, block)
    return x64 @ w.T, np.abs(x64) @ np.abs(w).T
