"""Widening of stored element formats to float64 (oracle side).

The pages fix no precision; the two stored formats used by the workloads are
IEEE fp32 and bfloat16.  bfloat16 is held in NumPy as its raw 16-bit pattern
(uint16), which is the upper half of the fp32 pattern of the same value, so
widening is exact: shift the bits into the top of a 32-bit word, reinterpret
as fp32, then convert to float64.
"""

import numpy as np


def to_f64(x, dtype):
    """Return ``x`` as float64.

    ``dtype`` names how ``x`` is stored: ``"f32"`` (float32 array) or
    ``"bf16"`` (uint16 array holding bfloat16 bit patterns).  Both widenings
    are exact.
    """
    x = np.asarray(x)
    if dtype == "f32":
        if x.dtype != np.float32:
            raise TypeError(f"f32 data must be float32, got {x.dtype}")
        return x.astype(np.float64)
    if dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError(f"bf16 data must be uint16 bit patterns, got {x.dtype}")
        wide = x.astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
