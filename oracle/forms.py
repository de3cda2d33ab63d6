"""Independent NumPy formulations of the SSD forward, used to pin the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Three ways of computing the same (y, final_state), all in float64:

``serial_numpy``  the per-token recurrence again, in NumPy instead of C.
``quadratic``     the quadratic "attention" form of the semiseparable matrix
                  (burn-mamba ``Mamba2SsdInput`` rustdoc, Step 1 applied with
                  one chunk covering the whole sequence), with every decay a
                  product of per-token factors computed by brute force and the
                  initial-state term written out explicitly.
``chunked``       the four-step chunked algorithm of the same rustdoc (Step 1
                  intra-chunk outputs, Step 2 chunk states (Eq. 20), Step 3
                  inter-chunk state passing (Eq. 22) done as one matrix product
                  with the segment-sum decay over chunks, Step 4 state-to-output
                  (Eq. 23), plus the D skip term), in the order and with the
                  zero padding of the naive branch of fla ``Mamba2.torch_forward``
                  and its ``segment_sum`` helper.

Shapes: x [b,L,H,P], dt [b,L,H] (already positive, i.e. after softplus),
A [H], B/C [b,L,G,N], D [H] or None, initial_state [b,H,P,N] or None.
Head h reads group h // (H/G).
"""
from __future__ import annotations

import numpy as np


def _expand_groups(M, nheads):
    """[b,L,G,N] -> [b,L,H,N] with head h reading group h // (H/G)."""
    G = M.shape[2]
    return np.repeat(M, nheads // G, axis=2)


def _prep(x, dt, A, B, C, D, initial_state):
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    H = x.shape[2]
    Bh = _expand_groups(np.asarray(B, dtype=np.float64), H)
    Ch = _expand_groups(np.asarray(C, dtype=np.float64), H)
    D = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    b, _, _, P = x.shape
    N = Bh.shape[3]
    S0 = np.zeros((b, H, P, N)) if initial_state is None else \
        np.asarray(initial_state, dtype=np.float64)
    return x, dt, A, Bh, Ch, D, S0


def serial_numpy(x, dt, A, B, C, D=None, initial_state=None):
    """Token-by-token recurrence, vectorised over (batch, head)."""
    x, dt, A, Bh, Ch, D, S = _prep(x, dt, A, B, C, D, initial_state)
    b, L, H, P = x.shape
    y = np.empty_like(x)
    S = S.copy()
    for t in range(L):
        alpha = np.exp(dt[:, t] * A[None, :])                       # [b,H]
        u = dt[:, t, :, None] * x[:, t]                             # [b,H,P]
        S = alpha[:, :, None, None] * S + u[:, :, :, None] * Bh[:, t, :, None, :]
        y[:, t] = np.einsum("bhpn,bhn->bhp", S, Ch[:, t]) + D[None, :, None] * x[:, t]
    return y, S


def decode_step_numpy(state, x, dt, A, B, C, D=None):
    """One token of the decode branch of fla ``Mamba2.torch_forward``:
    decay the cached state by exp(dt*A), add dt * B (outer) x, then read the
    output from the updated state with C and add the D skip term.

    state [b,H,P,N], x [b,H,P], dt [b,H], B/C [b,G,N].  Returns (state', y)."""
    state = np.asarray(state, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    H = x.shape[1]
    G = np.asarray(B).shape[1]
    Bh = np.repeat(np.asarray(B, dtype=np.float64), H // G, axis=1)     # [b,H,N]
    Ch = np.repeat(np.asarray(C, dtype=np.float64), H // G, axis=1)
    D = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    dA = np.exp(dt * np.asarray(A, dtype=np.float64)[None, :])           # [b,H]
    dBx = dt[:, :, None, None] * x[:, :, :, None] * Bh[:, :, None, :]
    new_state = state * dA[:, :, None, None] + dBx
    y = np.einsum("bhpn,bhn->bhp", new_state, Ch) + D[None, :, None] * x
    return new_state, y


def quadratic(x, dt, A, B, C, D=None, initial_state=None):
    """Brute-force masked quadratic form over the whole sequence.

    decay[t,s] = prod_{k=s+1..t} exp(dt_k A)   for s <= t, 0 above the diagonal
    M[t,s]     = (C_t . B_s) * decay[t,s] * dt_s
    y_t        = sum_s M[t,s] x_s + D x_t + prod_{k<=t} exp(dt_k A) * (S0 C_t)
    final      = sum_s decay[L-1,s] dt_s x_s (outer) B_s + prod_k exp(dt_k A) S0

    The products are accumulated one factor at a time (no cumulative sums),
    which is what makes this an independent check of the chunked path.
    """
    x, dt, A, Bh, Ch, D, S0 = _prep(x, dt, A, B, C, D, initial_state)
    b, L, H, P = x.shape
    alpha = np.exp(dt * A[None, None, :])                           # [b,L,H]
    decay = np.zeros((b, H, L, L))
    for t in range(L):
        run = np.ones((b, H))
        for s in range(t, -1, -1):
            decay[:, :, t, s] = run
            run = run * alpha[:, s, :]
    # full_decay[t] = prod_{k=0..t} alpha_k
    full_decay = np.empty((b, H, L))
    run = np.ones((b, H))
    for t in range(L):
        run = run * alpha[:, t, :]
        full_decay[:, :, t] = run
    CB = np.einsum("bthn,bshn->bhts", Ch, Bh)
    M = CB * decay * dt.transpose(0, 2, 1)[:, :, None, :]
    y = np.einsum("bhts,bshp->bthp", M, x)
    y += D[None, None, :, None] * x
    y += np.einsum("bht,bhpn,bthn->bthp", full_decay, S0, Ch)
    w = decay[:, :, L - 1, :] * dt.transpose(0, 2, 1)               # [b,H,L]
    final = np.einsum("bhs,bshp,bshn->bhpn", w, x, Bh)
    final += full_decay[:, :, L - 1, None, None] * S0
    return y, final


def segment_sum(a):
    """Stable segment sum over the last axis, as fla's ``segment_sum``:
    out[..., i, j] = sum_{k=j+1..i} a[..., k] for i >= j, -inf above the
    diagonal.  Built with a masked cumulative sum, never by subtracting two
    cumulative sums."""
    T = a.shape[-1]
    rep = np.repeat(a[..., None], T, axis=-1)          # rep[..., k, j] = a[..., k]
    strict = np.tril(np.ones((T, T), dtype=bool), k=-1)  # k > j
    rep = np.where(strict, rep, 0.0)
    seg = np.cumsum(rep, axis=-2)
    incl = np.tril(np.ones((T, T), dtype=bool), k=0)
    return np.where(incl, seg, -np.inf)


def chunked(x, dt, A, B, C, D=None, initial_state=None, chunk_len=64):
    """Four-step chunked SSD in float64 (zero-padded to a multiple of chunk_len)."""
    x, dt, A, Bh, Ch, D, S0 = _prep(x, dt, A, B, C, D, initial_state)
    b, L, H, P = x.shape
    N = Bh.shape[3]
    Q = int(chunk_len)
    pad = (Q - L % Q) % Q
    nc = (L + pad) // Q

    def padL(t):
        widths = [(0, 0)] * t.ndim
        widths[1] = (0, pad)
        return np.pad(t, widths)

    D_res = D[None, None, :, None] * padL(x)
    xdt = padL(x * dt[..., None])                                   # dt-weighted input
    a = padL(dt * A[None, None, :])                                  # [b,Lp,H]
    Bc = padL(Bh).reshape(b, nc, Q, H, N)
    Cc = padL(Ch).reshape(b, nc, Q, H, N)
    Xc = xdt.reshape(b, nc, Q, H, P)
    ac = a.reshape(b, nc, Q, H).transpose(0, 3, 1, 2)                # [b,H,c,Q]
    acum = np.cumsum(ac, axis=-1)

    # Step 1: intra-chunk outputs with zero incoming state.
    Lmask = np.exp(segment_sum(ac))                                  # [b,H,c,Q,Q]
    G = np.einsum("bclhn,bcshn->bclsh", Cc, Bc)
    Mm = G * Lmask.transpose(0, 2, 3, 4, 1)
    Y_diag = np.einsum("bclsh,bcshp->bclhp", Mm, Xc)

    # Step 2: state of every chunk from its own tokens only (Eq. 20).
    decay_states = np.exp(acum[..., -1:] - acum)                     # [b,H,c,Q]
    states = np.einsum("bclhn,bhcl,bclhp->bchpn", Bc, decay_states, Xc)

    # Step 3: inter-chunk recurrence (Eq. 22) as one product with the
    # segment-sum decay over chunk boundaries.
    states = np.concatenate([S0[:, None], states], axis=1)           # [b,c+1,H,P,N]
    chunk_ends = np.pad(acum[..., -1], [(0, 0), (0, 0), (1, 0)])     # [b,H,c+1]
    decay_chunk = np.exp(segment_sum(chunk_ends))                    # [b,H,c+1,c+1]
    new_states = np.einsum("bhzc,bchpn->bzhpn", decay_chunk, states)
    h_in, final = new_states[:, :-1], new_states[:, -1]

    # Step 4: contribution of each chunk's incoming state (Eq. 23).
    Y_off = np.einsum("bclhn,bchpn,bhcl->bclhp", Cc, h_in, np.exp(acum))

    y = (Y_diag + Y_off).reshape(b, nc * Q, H, P) + D_res
    return y[:, :L], final
