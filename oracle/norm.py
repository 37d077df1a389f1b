"""RMSNorm with the AWQ 1/s folded into it (the operator in front of the scaled layers).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fold the division by s into the operator that produces the layer's
input, so that inference runs no extra kernel: the Lab 4 + Lab 5 guide (AWQ
skeleton, part 2.3: the searched scales are merged into the preceding LayerNorm
or linear layer by ``scale_ln_fcs`` / ``scale_fc_fc``) and the chapter 11 AWQ
section (the division by s is merged into the LayerNorm in front). The decoder
blocks of the workloads are LLaMA-shaped, whose norm is RMSNorm; reading R13:
the folded operator is

    x_s[m][k] = f16( ((h[m][k] * r[m]) * gamma[k]) / s[k] ),
    r[m]      = 1 / sqrt( sum_k h[m][k]^2 / K + eps ),

every step in float64 in the order written (one rounding per operation, sqrt
and division correctly rounded), and one float64 -> float16 rounding at the
end. With s = 1 this is the plain RMSNorm output in fp16.
"""

import numpy as np

from .quant import f64_to_f16


def rms_factor(h, eps):
    """r[m] = 1 / sqrt(mean_k h[m][k]^2 + eps), float64. h: float16 [M][K]."""
    h64 = np.asarray(h, dtype=np.float16).astype(np.float64)
    if h64.ndim != 2 or h64.shape[1] == 0:
        raise ValueError("h must be [M][K] with K > 0")
    ms = (h64 * h64).sum(axis=1) / np.float64(h64.shape[1])
    return np.float64(1.0) / np.sqrt(ms + np.float64(eps))


def rmsnorm_fold(h, gamma, s, eps):
    """The RMSNorm output divided by the AWQ scale, as float16 (reading R13).

    h: float16 [M][K]; gamma: float16 [K]; s: float32 [K] or None (no fold).
    """
    h64 = np.asarray(h, dtype=np.float16).astype(np.float64)
    g64 = np.asarray(gamma, dtype=np.float16).astype(np.float64)
    r = rms_factor(h, eps)
    v = (h64 * r[:, None]) * g64[None, :]
    if s is not None:
        v = v / np.asarray(s, dtype=np.float32).astype(np.float64)[None, :]
    return f64_to_f16(v)
