"""Packed variable-length sequences on the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages' ``mamba_chunk_scan_combined`` takes ``seq_idx`` to pack several
sequences into one row: tokens of different sequences must not interact.
The reading: a token whose seq_idx differs from its predecessor's starts a
new sequence from a zero state; the row's initial state belongs to its first
sequence and the final state is that of its last token.  Evaluated here as
exactly that: the serial oracle run on every sequence separately.
"""
from __future__ import annotations

import numpy as np

from .serial import forward


def segments(seq_row):
    """[start, end) of each run of equal seq_idx values in one row."""
    s = np.asarray(seq_row)
    cuts = np.flatnonzero(s[1:] != s[:-1]) + 1
    bounds = np.concatenate([[0], cuts, [len(s)]])
    return list(zip(bounds[:-1], bounds[1:]))


def forward_varlen(x, dt, A, B, C, D, initial_state, seq_idx):
    """y [b, L, H, P] and the final state [b, H, P, N], fp64."""
    b, L, H, P = x.shape
    N = B.shape[3]
    y = np.zeros((b, L, H, P))
    fin = np.zeros((b, H, P, N))
    for r in range(b):
        for k, (s0, s1) in enumerate(segments(seq_idx[r])):
            init = None
            if k == 0 and initial_state is not None:
                init = initial_state[r:r + 1]
            yr, fr = forward(x[r:r + 1, s0:s1], dt[r:r + 1, s0:s1], A, B[r:r + 1, s0:s1],
                             C[r:r + 1, s0:s1], D, init)
            y[r, s0:s1] = yr[0]
            fin[r] = fr[0]
    return y, fin
