"""Error measures the parity tolerances are stated in.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix no tolerance; these two readings are the ones the parity bar
is written against:

* fp32 inputs: floored maximum relative error
      max_i |g_i - o_i| / max(|o_i|, 1e-3 * max_j |o_j|)  <=  1e-4
  The floor keeps entries that cancel to almost zero from dominating.
* bf16 inputs: normwise relative error in fp64
      ||g - o||_2 / ||o||_2  <=  2e-2
  applied to y and to the final state separately.
"""
from __future__ import annotations

import numpy as np

FP32_MAX_REL = 1e-4
BF16_NORMWISE = 2e-2


def max_rel_err(got, ref, floor: float = 1e-3) -> float:
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    if o.size == 0:
        return 0.0
    scale = np.maximum(np.abs(o), floor * np.max(np.abs(o)))
    scale = np.where(scale == 0.0, 1.0, scale)
    return float(np.max(np.abs(g - o) / scale))


def normwise_err(got, ref) -> float:
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(o.ravel())
    num = np.linalg.norm((g - o).ravel())
    if den == 0.0:
        return float(num)
    return float(num / den)


def parity_error(got, ref, io_dtype: str) -> float:
    """Error in the measure that applies to ``io_dtype`` ('f32' or 'bf16')."""
    return max_rel_err(got, ref) if io_dtype == "f32" else normwise_err(got, ref)


def tolerance(io_dtype: str) -> float:
    return FP32_MAX_REL if io_dtype == "f32" else BF16_NORMWISE
