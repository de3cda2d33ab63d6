"""fp64 causal depthwise convolution of the Mamba-2 layer and its decode
update.

TEST INFRASTRUCTURE ONLY (see the package docstring).

fla ``layers/mamba2.py``, ``Mamba2.torch_forward``: the x | B | C channels
pass through ``nn.Conv1d(conv_dim, conv_dim, kernel_size=W, groups=conv_dim,
padding=W-1)``, whose output is cut to the first seqlen positions, and then
the activation (SiLU).  Written out per channel c, with x_t = 0 for t < 0:

    out_t[c] = act(bias[c] + sum_{k<W} w[c][k] x_{t-W+1+k}[c])

The cache of the single-token path holds the last W inputs per channel,
[b, conv_dim, W], zero-padded on the left (the layer's cache initialisation
pads the transposed inputs on the left to W); a decode step rolls it left by
one, puts the new input last and takes the same dot product.
"""
from __future__ import annotations

import numpy as np


def silu(v):
    """v * sigmoid(v) = v / (1 + e^-v), fp64."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def _act(v, activation):
    if activation in (None, "none"):
        return v
    if activation == "silu":
        return silu(v)
    raise ValueError(activation)


def causal_conv1d(x, weight, bias=None, activation="silu"):
    """x [b, L, D], weight [D, W], bias [D] or None -> out [b, L, D] (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    b, L, D = x.shape
    W = w.shape[1]
    xp = np.concatenate([np.zeros((b, W - 1, D)), x], axis=1)   # x_{t} at xp[t + W - 1]
    acc = np.zeros((b, L, D)) if bias is None else np.broadcast_to(
        np.asarray(bias, dtype=np.float64), (b, L, D)).copy()
    for k in range(W):
        acc += w[:, k] * xp[:, k:k + L, :]
    return _act(acc, activation)


def conv_state_after(x, width):
    """The cache after a sequence: [b, D, W] holding x_{L-W} .. x_{L-1},
    zeros before the first token."""
    x = np.asarray(x, dtype=np.float64)
    b, L, D = x.shape
    xp = np.concatenate([np.zeros((b, width, D)), x], axis=1)
    return np.ascontiguousarray(xp[:, -width:, :].transpose(0, 2, 1))


def conv_update(state, x, weight, bias=None, activation="silu"):
    """One decode token: state [b, D, W], x [b, D] -> (out [b, D], new state)."""
    s = np.asarray(state, dtype=np.float64)
    new = np.concatenate([s[:, :, 1:], np.asarray(x, dtype=np.float64)[:, :, None]], axis=2)
    acc = (new * np.asarray(weight, dtype=np.float64)[None]).sum(axis=2)
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float64)
    return _act(acc, activation), new
