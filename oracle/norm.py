"""fp64 gated RMS normalisation of the Mamba-2 layer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

fla ``layers/mamba2.py`` builds ``RMSNormGated(intermediate_size,
eps=norm_eps, norm_before_gate=False)`` and applies ``norm(y, gate)`` to the
scan output.  The pages name the module and its arguments but do not print
its body; the reading taken is the plain one those arguments describe, with
the mean over the whole row (no group size is passed):

    gate before the norm:  g = y * silu(z),  out = g / sqrt(mean(g^2) + eps) * w
    gate after the norm:   out = y / sqrt(mean(y^2) + eps) * w * silu(z)
    no gate:               out = y / sqrt(mean(y^2) + eps) * w
"""
from __future__ import annotations

import numpy as np

from .conv import silu


def gated_rmsnorm(y, z, weight, eps=1e-5, norm_before_gate=False):
    """y, z [..., dim] (z may be None), weight [dim] -> out [..., dim], fp64."""
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    g = y if (z is None or norm_before_gate) else y * silu(z)
    out = g / np.sqrt(np.mean(g * g, axis=-1, keepdims=True) + float(eps)) * w
    if z is not None and norm_before_gate:
        out = out * silu(z)
    return out
