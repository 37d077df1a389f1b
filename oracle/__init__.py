"""CPU oracle for the W4A16 group-quantized linear path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library, its
Python binding, the timed part of ``bench.py``) may import, call or link this
package. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.

It is a plain, slow, obviously-correct NumPy float64 restatement of what the
pages define, written step by step in the pages' order:

* ``channel_scale``   - the AWQ activation statistic s = s_X^alpha (mean |x| per
  input channel, gathered on calibration tokens).
* ``scale_input``     - the 1/s that the method folds into the layer input.
* ``quantize_groups`` - round-to-nearest, min/max zero-point quantization of
  groups of consecutive input channels.
* ``pack_codes`` / ``unpack_codes`` - the nibble layout (layout v1).
* ``quantize_pack``   - all of the above for one weight matrix.
* ``dequantize`` / ``linear`` - the fused dequantize-then-multiply, in float64.
* ``rmsnorm_fold``    - the RMSNorm in front of the scaled layers with the 1/s
  folded into it (the operator that produces x_s in a decoder block).
* ``alpha_loss`` / ``search_alpha`` - the AWQ output-error loss and its grid
  search over alpha.
* ``quantize_groups_sym`` / ``quantize_pack_sym`` - symmetric absmax codes (the
  same packed layouts, a fixed zero).
* ``nf4_levels`` / ``quantize_nf4`` / ``dequantize_nf4`` / ``linear_nf4`` - the
  NormalFloat-4 codebook and blockwise absmax NF4 quantization.

It shares no code, header, table or constant with the HIP path. The only module
both sides use is the seeded input generator ``synth``, which holds none of the
method's arithmetic.

Pins: every function is checked in ``tests/test_oracle*.py`` against closed
forms, brute force in exact rationals, worked words and invariants (see the
docstrings). No function here is "parity unpinned".
"""

from .quant import (
    channel_scale,
    scale_input,
    quantize_groups,
    pseudo_quantize,
    quantize_pack,
    f64_to_f16,
)
from .layout import pack_codes, unpack_codes, pack_codes3, unpack_codes3, LAYOUT_VERSION
from .linear import dequantize, linear, within_tolerance, TOL_REL, TOL_ABS
from .norm import rms_factor, rmsnorm_fold
from .search import GRID as ALPHA_GRID, alpha_loss, search_alpha
from .sym import quantize_groups_sym, quantize_pack_sym
from .nf4 import (
    LEVELS as NF4_LEVELS,
    LEVELS_F16 as NF4_LEVELS_F16,
    nf4_levels,
    nf4_codes,
    quantize_nf4,
    quantize_pack_nf4,
    dequantize_nf4,
    linear_nf4,
)

__all__ = [
    "channel_scale",
    "scale_input",
    "quantize_groups",
    "pseudo_quantize",
    "quantize_pack",
    "f64_to_f16",
    "pack_codes",
    "unpack_codes",
    "LAYOUT_VERSION",
    "dequantize",
    "linear",
    "within_tolerance",
    "TOL_REL",
    "TOL_ABS",
    "rms_factor",
    "rmsnorm_fold",
    "ALPHA_GRID",
    "alpha_loss",
    "search_alpha",
]
