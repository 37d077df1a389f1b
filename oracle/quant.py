"""Oracle: AWQ scale, input fold, and group-wise RTN zero-point quantization.

Test infrastructure only; see the package docstring.

Sources (the pages are cited by title and section):

* "MIT 6.5940 L13 LLM Deployment" reading guide (quidproquo.cc), section on AWQ:
  salient input channels of W are multiplied by s > 1 and the matching input is
  divided by s, with 1/s foldable into the previous operator (slides 25-27);
  Q(w) = Delta * Round(w / Delta), round error expectation about 0.25
  (slides 26/28); s = s_X^alpha with s_X the mean activation magnitude, alpha
  chosen by search (slide 28). Its QServe table fixes the edge setting
  W4-A16-KV16 with 4-bit per-group weights, group 128.
* "MIT 6.5940 Lab 4 + Lab 5" guide, Lab 4 "starting point and setup": forward
  hooks record the mean absolute value of every linear layer's input on
  calibration blocks of 512 tokens; quantization is "pseudo quantization"
  (quantize to integers, immediately dequantize).
* "CMU 11-868 Model Quantization" guide, L19 "absmax and zero-point": the
  zero-point quantizer takes its scale from max - min, replaces a zero range
  by 1, adds an integer zero offset, rounds, and clips codes to the integer
  range. Its GPTQ setup section: asymmetric per-row min-max uniform
  quantization; AutoGPTQ example bits=4, group_size=128.
* "Quantization for LLMs" chapter 11, section 11.3: Y = X W^T =
  (X diag(s)^-1)(W diag(s))^T, alpha = 0.5 is the default strength.

Readings where the pages are silent or disagree (each one is also listed in
the design doc):

* R1 asymmetric min/max with unsigned codes in [0, 2^b - 1] (the L13 slide
  formula is the symmetric absmax one; the config and the zero-point slide
  code are asymmetric).
* R2 Round is round-half-to-even (``np.rint``).
* R3 q = clip(rint(w / Delta) + z, 0, 2^b - 1): round w/Delta first, then add
  the integer zero, so unclamped codes reproduce Delta * Round(w / Delta).
* R4 z = rint(-min / Delta) is not clamped; a zero offset is +0 (so a group
  whose minimum is +0 or -0 stores the same zero bits).
* R5 codes use the float64 Delta; the stored scale is f16(Delta).
* R6 a constant group (max == min) uses range 1.
* R7 w / Delta and -min / Delta are IEEE float64 divisions.
* R8 float64 -> float16 is a single round-to-nearest-even step.
* R9 s is computed in float64 and stored as float32; a channel whose mean
  magnitude is 0 gets s = 1; alpha = 0.5 uses the square root.
* R10 groups are consecutive input channels of one output row; K % group == 0.
"""

import numpy as np

# Rows handled per block, only to bound memory on large layers.
_ROW_BLOCK = 256


def f64_to_f16(a):
    """float64 -> float16, one round-to-nearest-even step (reading R8).

    NumPy converts double to half directly (no float32 intermediate). This is
    pinned against an exact-rational rounding in tests/test_oracle.py.
    """
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float64).astype(np.float16)


def channel_scale(x_cal, alpha=0.5):
    """AWQ per-input-channel scale s_k = (mean_t |x_cal[t, k]|) ** alpha.

    Follows the L13 guide's AWQ section (s = s_X^alpha, s_X = mean activation
    magnitude) and the Lab 4 setup (mean |input| per channel on calibration
    tokens). Readings R9: float64 arithmetic, float32 result, s = 1 where the
    mean is 0, square root for alpha = 0.5.

    x_cal: float16 [T][K]. Returns float32 [K].
    """
    x = np.asarray(x_cal, dtype=np.float16).astype(np.float64)
    t = x.shape[0]
    if t <= 0:
        raise ValueError("need at least one calibration token")
    mean = np.abs(x).sum(axis=0) / np.float64(t)
    if alpha == 0.5:
        s = np.sqrt(mean)
    else:
        s = np.power(mean, np.float64(alpha))
    s = np.where(mean == 0.0, 1.0, s)
    return s.astype(np.float32)


def scale_input(x, s):
    """The 1/s folded into the layer input: x_s = f16(x / s), float64 division.

    L13 guide, AWQ section (the input of a scaled channel is divided by s);
    chapter 11 section 11.3 (X diag(s)^-1). x: float16 [M][K]; s: float32 [K].
    """
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    return f64_to_f16(x64 / s64[None, :])


def quantize_groups(w, bits=4, group=128):
    """Round-to-nearest zero-point quantization of groups of `group` inputs.

    Steps, in order (CMU L19 zero-point quantizer; L13 AWQ slide formula
    Q(w) = Delta * Round(w / Delta); readings R1-R7, R10):

    1. per (row, group): mn = min w, mx = max w
    2. range = mx - mn, replaced by 1 when it is 0
    3. Delta = range / (2^b - 1)
    4. z = rint(-mn / Delta)             (not clamped; +0 when zero)
    5. q = clip(rint(w / Delta) + z, 0, 2^b - 1)

    w: float64 [N][K]. Returns (q int64 [N][K], delta float64 [N][K/g],
    z float64 [N][K/g]).
    """
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    if k % group != 0:
        raise ValueError("K must be a multiple of the group size")
    qmax = float(2 ** bits - 1)
    wg = w.reshape(n, k // group, group)
    mn = wg.min(axis=2)
    mx = wg.max(axis=2)
    rng = mx - mn
    rng = np.where(rng == 0.0, 1.0, rng)
    delta = rng / qmax
    z = np.rint(np.negative(mn) / delta) + 0.0  # the integer zero offset 0 has one encoding, +0
    q = np.clip(np.rint(wg / delta[:, :, None]) + z[:, :, None], 0.0, qmax)
    return q.astype(np.int64).reshape(n, k), delta, z


def pseudo_quantize(w, bits=4, group=128):
    """Q(w) = (q - z) * Delta in float64: quantize, then dequantize at once.

    The "pseudo quantization" of the Lab 4 setup; used for the invariant and
    statistical pins.
    """
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    q, delta, z = quantize_groups(w, bits, group)
    qg = q.reshape(n, k // group, group).astype(np.float64)
    return ((qg - z[:, :, None]) * delta[:, :, None]).reshape(n, k)


def quantize_pack(W, s=None, bits=4, group=128):
    """AWQ quantize-pack of one nn.Linear weight (fp16 [N][K], rows = outputs).

    w = float64(W) * float64(s) (exact: 11-bit times 24-bit significands), then
    ``quantize_groups``, then storage: scales = f16(Delta), zeros = f16(z),
    qweight = layout-v1 nibble words (bits = 4) or the 3-bit bit-plane words
    (bits = 3). Returns (qweight uint32 [N][K/8] or [N][3K/32], scales float16
    [N][K/g], zeros float16 [N][K/g]).
    """
    from .layout import pack_codes, pack_codes3

    W = np.asarray(W, dtype=np.float16)
    n, k = W.shape
    if bits not in (3, 4):
        raise ValueError("the packed layouts store 3-bit or 4-bit codes")
    if k % group != 0:
        raise ValueError("K must be a multiple of the group size")
    if bits == 3 and k % 32 != 0:
        raise ValueError("the 3-bit layout packs blocks of 32 inputs")
    pack = pack_codes if bits == 4 else pack_codes3
    s64 = None if s is None else np.asarray(s, dtype=np.float32).astype(np.float64)
    qweight = np.empty((n, k // 8 if bits == 4 else 3 * (k // 32)), dtype=np.uint32)
    scales = np.empty((n, k // group), dtype=np.float16)
    zeros = np.empty((n, k // group), dtype=np.float16)
    for r0 in range(0, n, _ROW_BLOCK):
        r1 = min(n, r0 + _ROW_BLOCK)
        w = W[r0:r1].astype(np.float64)
        if s64 is not None:
            w = w * s64[None, :]
        q, delta, z = quantize_groups(w, bits, group)
        qweight[r0:r1] = pack(q)
        scales[r0:r1] = f64_to_f16(delta)
        zeros[r0:r1] = f64_to_f16(z)
    return qweight, scales, zeros
