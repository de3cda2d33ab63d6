"""Independent NumPy formulations of the SSD forward, used to pin the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Three ways of computing the same (y, final_state), all in float64:

``serial_numpy``  the per-token recurrence again, in NumPy instead of C.
``serial_fp32``   the same loop with every operation rounded to float32: what
                  plain fp32 arithmetic scores under an error measure.
``quadratic``     the quadratic "attention" form of the semiseparable matrix
                  (burn-mamba ``Mamba2SsdInput`` rustdoc, Step 1 applied with
                  one chunk covering the whole sequence), with every decay a
                  product of per-token factors computed by brute force and the
                  initial-state term written out explicitly.
``chunked``       the four-step chunked algorithm of the same rustdoc (Step 1
                  intra-chunk outputs, Step 2 chunk states (Eq. 20), Step 3
                  inter-chunk state passing (Eq. 22), Step 4 state-to-output
                  (Eq. 23), plus the D skip term), chunk after chunk, with each
                  decay a product of per-token factors and the passing a
                  sequential loop over the chunks.

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


def serial_fp32(x, dt, A, B, C, D=None, initial_state=None):
    """The textbook evaluation of the recurrence in fp32: every operation of
    ``serial_numpy`` rounded to float32 (numpy float32 arithmetic), token by
    token.  Not a reference: it shows what plain fp32 arithmetic scores under
    an error measure, which sets the fp32 bars of the parity tests."""
    f = np.float32
    x = np.asarray(x, dtype=f)
    dt = np.asarray(dt, dtype=f)
    A = np.asarray(A, dtype=f)
    b, L, H, P = x.shape
    G = np.asarray(B).shape[2]
    Bh = np.repeat(np.asarray(B, dtype=f), H // G, axis=2)
    Ch = np.repeat(np.asarray(C, dtype=f), H // G, axis=2)
    D = np.zeros(H, dtype=f) if D is None else np.asarray(D, dtype=f)
    N = Bh.shape[3]
    S = np.zeros((b, H, P, N), dtype=f) if initial_state is None else \
        np.array(initial_state, dtype=f)
    y = np.empty_like(x)
    for t in range(L):
        al = np.exp(dt[:, t] * A[None, :]).astype(f)
        S = (al[:, :, None, None] * S + (dt[:, t, :, None] * x[:, t])[..., None]
             * Bh[:, t, :, None, :]).astype(f)
        y[:, t] = (np.einsum("bhpn,bhn->bhp", S, Ch[:, t]).astype(f)
                   + D[None, :, None] * x[:, t]).astype(f)
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


def chunked(x, dt, A, B, C, D=None, initial_state=None, chunk_len=64):
    """The four steps of the burn-mamba ``Mamba2SsdInput`` rustdoc, one chunk
    after the other, in float64.

    The sequence is cut into chunks of ``chunk_len`` tokens; a ragged last
    chunk is simply shorter (the zero padding of the rustdoc's layout adds
    nothing to any sum).  With alpha_k = exp(dt_k A) and h the state entering
    chunk [c0, c1), for tokens c0 <= s <= t < c1:

      decay(t, s) = alpha_{s+1} * ... * alpha_t          (1 when s = t)
      Step 1, intra-chunk output (L o C B^T) X:
          y_t  = sum_{s <= t} (C_t . B_s) decay(t, s) dt_s x_s
      Step 4, state to output (Eq. 23):
          y_t += (alpha_{c0} * ... * alpha_t) (h C_t)
      Step 2, the chunk's own state (Eq. 20):
          S    = sum_s decay(c1 - 1, s) dt_s x_s (outer) B_s
      Step 3, state passing (Eq. 22):
          h   <- (alpha_{c0} * ... * alpha_{c1-1}) h + S

    plus D x_t.  Every decay is a product accumulated one factor at a time,
    and the passing is a sequential loop over chunks, so this shares neither
    the per-token loop of the serial oracle nor the cumulative sums of the
    fused kernel."""
    x, dt, A, Bh, Ch, D, h = _prep(x, dt, A, B, C, D, initial_state)
    b, L, H, P = x.shape
    Q = int(chunk_len)
    y = np.empty_like(x)
    h = h.copy()
    for c0 in range(0, L, Q):
        c1 = min(c0 + Q, L)
        n = c1 - c0
        alpha = np.exp(dt[:, c0:c1] * A[None, None, :])            # [b,n,H]
        # decay[..., t, s] within the chunk, zero above the diagonal
        decay = np.zeros((b, H, n, n))
        for t in range(n):
            run = np.ones((b, H))
            for s in range(t, -1, -1):
                decay[:, :, t, s] = run
                run = run * alpha[:, s, :]
        # into[..., t] = alpha_{c0} * ... * alpha_t: the entering state's decay
        into = np.empty((b, H, n))
        run = np.ones((b, H))
        for t in range(n):
            run = run * alpha[:, t, :]
            into[:, :, t] = run
        xc, dtc = x[:, c0:c1], dt[:, c0:c1]                          # [b,n,H,P], [b,n,H]
        Bc, Cc = Bh[:, c0:c1], Ch[:, c0:c1]                          # [b,n,H,N]
        u = xc * dtc[..., None]                                       # dt_s x_s
        # Step 1
        cb = np.einsum("bthn,bshn->bhts", Cc, Bc)
        y_diag = np.einsum("bhts,bshp->bthp", cb * decay, u)
        # Step 4
        y_off = np.einsum("bht,bhpn,bthn->bthp", into, h, Cc)
        y[:, c0:c1] = y_diag + y_off + D[None, None, :, None] * xc
        # Step 2
        S = np.einsum("bhs,bshp,bshn->bhpn", decay[:, :, n - 1, :], u, Bc)
        # Step 3
        h = into[:, :, n - 1, None, None] * h + S
    return y, h
