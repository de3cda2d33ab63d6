"""The output gate and a per-channel D in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages' scan and decode kernels take ``D`` and ``z``; the lrnnx scan's
``selective_scan_ref`` spells out what they do to the output (its "Final
Output Processing"): the skip term is added, then the sum is multiplied by
SiLU of the gate.  The fla decode branch passes D expanded to [nheads,
headdim], so D may be per head or per (head, headdim column):

    y_t = (h_t C_t + D (*) x_t) * silu(z_t),     silu(v) = v / (1 + e^-v)

The state is the serial oracle's (the gate does not touch it).  SiLU is
scipy's logistic function ``expit`` times v.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit

from .serial import forward, state_update


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v * expit(v)


def skip(D, x):
    """D (*) x for D [H] or [H, P] and x [..., H, P] (0 for D None)."""
    x = np.asarray(x, dtype=np.float64)
    if D is None:
        return np.zeros_like(x)
    D = np.asarray(D, dtype=np.float64)
    return (D[:, None] if D.ndim == 1 else D) * x


def forward_gated(x, dt, A, B, C, D=None, z=None, initial_state=None):
    """(y [b,L,H,P], final [b,H,P,N]) in fp64 with the skip and the gate."""
    y, fin = forward(x, dt, A, B, C, None, initial_state)
    y = y + skip(D, x)
    if z is not None:
        y = y * silu(z)
    return y, fin


def forward_gated_abs(x, dt, A, B, C, D=None, z=None, initial_state=None):
    """The magnitude reference of forward_gated's y: every summed term in
    absolute value (the fp32 parity measure)."""
    ab = lambda a: None if a is None else np.abs(a)  # noqa: E731
    y, _ = forward(ab(x), dt, A, ab(B), ab(C), None, ab(initial_state))
    y = y + skip(ab(D), ab(x))
    if z is not None:
        y = y * np.abs(silu(z))
    return y


def state_update_gated(state, x, dt, A, B, C, D=None, z=None):
    """One decode token: (new state [b,H,P,N], gated y [b,H,P])."""
    fin, y = state_update(state, x, dt, A, B, C, None)
    y = y + skip(D, x)
    if z is not None:
        y = y * silu(z)
    return fin, y
