"""The AWQ scale search: the output-error loss over a grid of alpha (float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The "MIT 6.5940 L13 LLM Deployment" guide (AWQ section, slide 28) and chapter 11
(AWQ section) choose the scale by a grid search over alpha in [0, 1]:

    L(s) = || Q(W . s)(s^-1 . X) - W X ||,   s = s_X^alpha,   alpha* = argmin_alpha L(s_X^alpha),

with s_X the mean activation magnitude per input channel, measured on a small
calibration set, and the loss taken on the layer's *output*, not on the weights.

Reading R14 (where the pages leave the step open):
* the grid is alpha = i / 20, i = 0..20;
* the norm is the Frobenius norm, used squared (the argmin is the same);
* s^-1 . X is the input the kernel consumes, x_s = f16(x / s), and Q(W . s) is the
  dequantized weight built from the stored fp16 scale and zero (what the deployed
  layer computes); W X uses the fp16 weights as given;
* on equal losses the smallest alpha wins.
"""

import numpy as np

from .linear import dequantize
from .quant import channel_scale, quantize_pack, scale_input

GRID = tuple(i / 20 for i in range(21))


def alpha_loss(x_cal, W, alpha):
    """sum_{t,n} (y_q[t][n] - y[t][n])^2 in float64 for one alpha.

    x_cal: float16 [T][K] calibration activations; W: float16 [N][K].
    y_q = x_s . w_hat^T with s = channel_scale(x_cal, alpha), x_s = scale_input(x_cal, s),
    w_hat = dequantize(quantize_pack(W, s)); y = x_cal . W^T.
    """
    s = channel_scale(x_cal, alpha)
    xs = scale_input(x_cal, s).astype(np.float64)
    w_hat = dequantize(*quantize_pack(W, s), np.asarray(W).shape[1])
    x64 = np.asarray(x_cal, dtype=np.float16).astype(np.float64)
    w64 = np.asarray(W, dtype=np.float16).astype(np.float64)
    d = xs @ w_hat.T - x64 @ w64.T
    return float((d * d).sum())


def search_alpha(x_cal, W, grid=GRID):
    """Losses over the grid and the chosen alpha (first minimum)."""
    losses = np.array([alpha_loss(x_cal, W, a) for a in grid], dtype=np.float64)
    best = int(np.argmin(losses))  # the first index of the minimum
    return losses, grid[best]
