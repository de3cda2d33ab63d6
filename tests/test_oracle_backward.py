"""Pins for the fp64 oracle's gradients (``oracle.backward``).

The backward oracle is reverse-mode differentiation of the serial loop,
written by hand in ``ssd_oracle.c``.  It is tied here to things other than
itself:
  * central finite differences of the forward oracle, on every element of
    every gradient of a small problem (with and without groups);
  * automatic differentiation (torch, fp64, CPU) of an independent
    formulation: the quadratic masked form, y = (L o C B^T o decay) (dt x)
    + D x + decay_from_start C init^T, and its final state;
  * closed forms at A = 0 (causal linear attention), where every gradient is
    a few library matrix products;
  * planted mistakes: copies of the adjoint loop with a plausible error each
    (written here in NumPy), which the finite differences reject.
"""
import numpy as np
import pytest

from state_space_sequence_amd.inputs import make_inputs

GRADS = ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit")
ARGS = ("x", "dt", "A", "B", "C", "D", "initial_state")


def _problem(b, L, H, P, N, G, seed, init=True):
    inp = make_inputs(b, L, H, P, N, G, io_dtype="f32", init_std=0.1 if init else 0.0,
                      seed=seed)
    a = {k: (None if inp[k] is None else inp[k].astype(np.float64)) for k in ARGS}
    rng = np.random.default_rng(seed + 100)
    dy = rng.standard_normal((b, L, H, P))
    dfin = rng.standard_normal((b, H, P, N))
    return a, dy, dfin


def _loss(oracle_mod, a, dy, dfin):
    y, f = oracle_mod.forward(*(a[k] for k in ARGS))
    return float((y * dy).sum() + (f * dfin).sum())


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


@pytest.mark.parametrize("G", [1, 2])
def test_backward_matches_finite_differences_everywhere(oracle_mod, G):
    """Every element of every gradient against a central difference of the
    loss <y, dy> + <final, dfinal> (step 1e-5: truncation ~1e-10, rounding
    ~1e-11 relative)."""
    a, dy, dfin = _problem(1, 9, 2, 3, 4, G, seed=11 + G)
    g = oracle_mod.backward(*(a[k] for k in ARGS), dy, dfin)
    eps = 1e-5
    for name, key in zip(ARGS, GRADS):
        base = a[name]
        fd = np.empty_like(base)
        for ix in np.ndindex(base.shape):
            p, m = base.copy(), base.copy()
            p[ix] += eps
            m[ix] -= eps
            fd[ix] = (_loss(oracle_mod, dict(a, **{name: p}), dy, dfin) -
                      _loss(oracle_mod, dict(a, **{name: m}), dy, dfin)) / (2 * eps)
        err = _rel(g[key], fd)
        assert err < 1e-7, "%s: %.3e" % (key, err)


def _quadratic_torch(x, dt, A, B, C, D, init):
    """The quadratic masked form in torch fp64 (autograd-able), written from
    the definition: decay(l, s) = exp(sum_{k=s+1..l} dt_k A) for s <= l."""
    import torch
    b, L, H, P = x.shape
    G = B.shape[2]
    hpg = H // G
    Bh = B.repeat_interleave(hpg, dim=2)            # [b, L, H, N]
    Ch = C.repeat_interleave(hpg, dim=2)
    a = dt * A                                      # [b, L, H]
    cum = torch.cumsum(a, dim=1)                    # sum_{k<=l} a_k
    diff = cum[:, :, None, :] - cum[:, None, :, :]  # [b, l, s, H] = sum_{k=s+1..l}
    mask = torch.tril(torch.ones(L, L, dtype=torch.bool))[None, :, :, None]
    decay = torch.where(mask, torch.exp(torch.where(mask, diff, torch.zeros_like(diff))),
                        torch.zeros_like(diff))
    cb = torch.einsum("blhn,bshn->blsh", Ch, Bh)
    M = cb * decay * dt[:, None, :, :]              # dt of the source token s
    y = torch.einsum("blsh,bshp->blhp", M, x) + D[None, None, :, None] * x
    # the initial state seen at token l, decayed by sum_{k<=l} a_k
    y = y + torch.exp(cum)[..., None] * torch.einsum("bhpn,blhn->blhp", init, Ch)
    tail = torch.exp(cum[:, -1:, :] - cum)          # decay from s to the end
    final = torch.einsum("bsh,bshp,bshn->bhpn", tail * dt, x, Bh) + \
        torch.exp(cum[:, -1, :])[..., None, None] * init
    return y, final


def test_backward_matches_autograd_of_the_quadratic_form(oracle_mod):
    import torch
    a, dy, dfin = _problem(2, 60, 4, 5, 6, 2, seed=21)
    g = oracle_mod.backward(*(a[k] for k in ARGS), dy, dfin)
    t = {k: torch.tensor(a[k], dtype=torch.float64, requires_grad=True) for k in ARGS}
    y, f = _quadratic_torch(*(t[k] for k in ARGS))
    loss = (y * torch.tensor(dy)).sum() + (f * torch.tensor(dfin)).sum()
    loss.backward()
    for name, key in zip(ARGS, GRADS):
        err = _rel(g[key], t[name].grad.numpy())
        assert err < 1e-11, "%s: %.3e" % (key, err)


def test_backward_closed_forms_at_zero_decay(oracle_mod):
    """A = 0: y = tril(C B^T) diag(dt) x + D x, final = x^T diag(dt) B (zero
    initial state), per head.  Then, with W = tril(C B^T):
      dx = diag(dt) W^T dy + D dy + diag(dt) B dfinal^T
      ddt_s = x_s . (W^T dy + B dfinal^T)_s
      dC = tril(dy (diag(dt) x)^T) B
      dB = tril(dy (diag(dt) x)^T)^T C + diag(dt) x dfinal
      dA = sum_l dy_l . sum_{s<=l} W[l,s] (T_l - T_s) dt_s x_s
           + sum_s (T_end - T_s) dt_s x_s^T dfinal B_s,  T = cumsum(dt)
      dD = sum dy . x;  dinit = sum_l C_l dy_l^T ... = dy^T C + dfinal."""
    a, dy, dfin = _problem(1, 23, 3, 4, 5, 3, seed=31, init=False)
    a["A"] = np.zeros_like(a["A"])
    g = oracle_mod.backward(*(a[k] for k in ARGS), dy, dfin)
    for h in range(3):
        x, dt = a["x"][0, :, h], a["dt"][0, :, h]
        B, C = a["B"][0, :, h], a["C"][0, :, h]
        Dh, dyh, V = a["D"][h], dy[0, :, h], dfin[0, h]
        W = np.tril(C @ B.T)
        xs = dt[:, None] * x
        T = np.cumsum(dt)
        np.testing.assert_allclose(g["dx"][0, :, h], dt[:, None] * (W.T @ dyh) + Dh * dyh +
                                   dt[:, None] * (B @ V.T), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["ddt"][0, :, h],
                                   np.sum(x * (W.T @ dyh + B @ V.T), axis=1), rtol=1e-12, atol=1e-12)
        Z = np.tril(dyh @ xs.T)
        np.testing.assert_allclose(g["dC"][0, :, h], Z @ B, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["dB"][0, :, h], Z.T @ C + xs @ V, rtol=1e-12, atol=1e-12)
        dA = np.sum(dyh * ((W * (T[:, None] - T[None, :])) @ xs)) + \
            np.sum(((T[-1] - T)[:, None] * xs) * (B @ V.T))
        np.testing.assert_allclose(g["dA"][h], dA, rtol=1e-12)
        np.testing.assert_allclose(g["dD"][h], np.sum(dyh * x), rtol=1e-12)
        np.testing.assert_allclose(g["dinit"][0, h], dyh.T @ C + V, rtol=1e-12, atol=1e-12)


def _adjoint_numpy(a, dy, dfin, mistake):
    """A NumPy copy of the adjoint loop for one batch entry and G = H, with
    one planted mistake."""
    x, dt, A, B, C, D = (a[k][0] if a[k].ndim > 1 else a[k] for k in ARGS[:6])
    init = a["initial_state"][0]
    L, H, P = x.shape
    out = {k: np.zeros_like(v) for k, v in (("dx", x), ("ddt", dt), ("dB", B), ("dC", C))}
    out["dA"], out["dD"], out["dinit"] = np.zeros(H), np.zeros(H), np.zeros_like(init)
    for h in range(H):
        S = [init[h].copy()]
        for t in range(L):
            S.append(np.exp(dt[t, h] * A[h]) * S[-1] + dt[t, h] * np.outer(x[t, h], B[t, h]))
        lam = dfin[0, h].copy()
        for t in range(L - 1, -1, -1):
            al = np.exp(dt[t, h] * A[h])
            lam = lam + np.outer(dy[0, t, h], C[t, h])
            out["dC"][t, h] += dy[0, t, h] @ S[t + 1]
            lb = lam @ B[t, h]
            out["dx"][t, h] = D[h] * dy[0, t, h] + dt[t, h] * lb
            out["dB"][t, h] += dt[t, h] * (x[t, h] @ lam)
            prev = S[t + 1] if mistake == "state_after" else S[t]
            e = np.sum(lam * al * prev)
            A_term = 0.0 if mistake == "no_decay_term" else A[h] * e
            out["ddt"][t, h] = x[t, h] @ lb + A_term
            out["dA"][h] += dt[t, h] * e
            out["dD"][h] += dy[0, t, h] @ x[t, h]
            lam = lam if mistake == "no_decay" else al * lam
        out["dinit"][h] = lam
    return out


@pytest.mark.parametrize("mistake", [None, "state_after", "no_decay_term", "no_decay"])
def test_planted_mistakes_are_caught(oracle_mod, mistake):
    """The finite-difference pin accepts the NumPy adjoint as written and
    rejects each planted mistake."""
    a, dy, dfin = _problem(1, 7, 2, 3, 4, 2, seed=41)
    g = _adjoint_numpy(a, dy, dfin, mistake)
    eps = 1e-5
    worst = 0.0
    for name, key in (("dt", "ddt"), ("A", "dA"), ("initial_state", "dinit"), ("x", "dx")):
        base = a[name]
        for ix in np.ndindex(base.shape):
            p, m = base.copy(), base.copy()
            p[ix] += eps
            m[ix] -= eps
            fd = (_loss(oracle_mod, dict(a, **{name: p}), dy, dfin) -
                  _loss(oracle_mod, dict(a, **{name: m}), dy, dfin)) / (2 * eps)
            got = g[key][ix[1:]] if key in ("dinit", "dx", "ddt") else g[key][ix]
            worst = max(worst, abs(got - fd) / max(abs(fd), 1e-3))
    if mistake is None:
        assert worst < 1e-6
        ref = oracle_mod.backward(*(a[k] for k in ARGS), dy, dfin)
        for key in GRADS:
            want = ref[key][0] if key in ("dx", "ddt", "dB", "dC", "dinit") else ref[key]
            np.testing.assert_allclose(g[key], want, rtol=1e-12, atol=1e-12)
    else:
        assert worst > 1e-3, mistake


def test_backward_long_sequence_uses_checkpoints(oracle_mod):
    """A sequence of several 64-token segments (and a ragged last one) agrees
    with the quadratic form's autograd: the segment replay is exact."""
    import torch
    a, dy, dfin = _problem(1, 150, 2, 3, 4, 1, seed=51)
    g = oracle_mod.backward(*(a[k] for k in ARGS), dy, dfin)
    t = {k: torch.tensor(a[k], dtype=torch.float64, requires_grad=True) for k in ARGS}
    y, f = _quadratic_torch(*(t[k] for k in ARGS))
    ((y * torch.tensor(dy)).sum() + (f * torch.tensor(dfin)).sum()).backward()
    for name, key in zip(ARGS, GRADS):
        assert _rel(g[key], t[name].grad.numpy()) < 1e-11, key
