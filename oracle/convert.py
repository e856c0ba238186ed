"""bf16 copies of float32 values (the optional gradient convert step).

Test infrastructure only (see the package docstring).

The pages give the attention inputs and outputs as bf16 ("bf16 I/O" of the
production guide's kernels) but keep no precision for gradients; here the
gradients are float32 and a caller that wants bf16 gets them rounded to the
nearest bf16, ties to even (the IEEE default rounding).  NaN stays NaN.
"""
from __future__ import annotations

import numpy as np


def round_to_bf16_bits(x) -> np.ndarray:
    """uint16 bf16 bit patterns of float32 values, round to nearest, ties to even.

    A bf16 value is the top 16 bits of a float32.  Dropping the low 16 bits
    rounds toward zero; adding 0x7FFF plus the lowest kept bit first rounds to
    nearest with ties to the even kept pattern, and carries into the exponent
    (up to infinity) exactly as value rounding does.  NaNs map to a quiet NaN
    of the same sign.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = a.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + keep_lsb) >> 16) & 0xFFFF
    nan = np.isnan(a)
    sign = (bits >> 16) & 0x8000
    out = np.where(nan, sign | 0x7FC0, rounded)
    return out.astype(np.uint16)
