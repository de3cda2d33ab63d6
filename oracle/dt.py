"""fp64 time-step preprocessing of the Mamba-2 layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer does not feed its projected time step to the scan directly
(fla ``layers/mamba2.py``, ``Mamba2.torch_forward``, the single-token branch
and the chunked branch; the same arguments ``dt_bias``, ``dt_softplus=True``
and ``dt_limit`` that it passes to ``mamba_chunk_scan_combined``):

    dt = clamp(softplus(dt_raw + dt_bias_h), dt_min, dt_max)

with softplus(v) = log(1 + e^v), a per-head bias, and the clamp bounds of
``time_step_limit`` (by default 0 and +inf, which leave every softplus
output unchanged).  Without softplus the biased value is clamped directly.
This module evaluates that definition in IEEE double; the result then
enters the recurrence of ``serial``/``forms`` as the time step.
"""
from __future__ import annotations

import numpy as np


def softplus(v):
    """log(1 + e^v) in fp64, without overflow (``numpy.logaddexp``)."""
    return np.logaddexp(0.0, np.asarray(v, dtype=np.float64))


def process_dt(dt_raw, dt_bias=None, dt_softplus=False, dt_min=0.0, dt_max=np.inf):
    """The time step the recurrence uses, from the raw one.

    dt_raw: [..., H] (the head is the last axis, as in dt [b, L, H] and in
    the decode step's dt [b, H]); dt_bias: [H] or None.  Returns fp64.
    """
    v = np.asarray(dt_raw, dtype=np.float64)
    if dt_bias is not None:
        v = v + np.asarray(dt_bias, dtype=np.float64)
    if dt_softplus:
        v = softplus(v)
    return np.minimum(np.maximum(v, float(dt_min)), float(dt_max))
