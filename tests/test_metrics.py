"""The fp32 parity measure separates fp32 arithmetic from bf16 rounding and
from real mistakes (CPU only)."""
import numpy as np

from oracle import metrics
from state_space_sequence_amd.inputs import make_inputs, round_to_bf16


def _serial32(inp, round_state=None):
    x, dt, A, B, C, D, S = (inp[k].astype(np.float32) for k in
                            ("x", "dt", "A", "B", "C", "D", "initial_state"))
    b, L, H, P = x.shape
    G = B.shape[2]
    Bh, Ch = np.repeat(B, H // G, axis=2), np.repeat(C, H // G, axis=2)
    y = np.empty_like(x)
    for t in range(L):
        al = np.exp(dt[:, t] * A[None]).astype(np.float32)
        S = (al[:, :, None, None] * S + (dt[:, t, :, None] * x[:, t])[..., None]
             * Bh[:, t, :, None, :]).astype(np.float32)
        Sr = S if round_state is None else round_state(S)
        y[:, t] = np.einsum("bhpn,bhn->bhp", Sr, Ch[:, t]).astype(np.float32) \
            + D[None, :, None] * x[:, t]
    return y, S


def test_componentwise_measure_scores(oracle_mod):
    inp = make_inputs(1, 256, 2, 128, 256, 1, io_dtype="f32", init_std=0.1, seed=356)
    args = ("x", "dt", "A", "B", "C", "D", "initial_state")
    yr, fr = oracle_mod.forward(*(inp[k] for k in args))
    ia = metrics.abs_inputs(inp)
    ya, fa = oracle_mod.forward(*(ia[k] for k in args))
    # the fp32 recurrence passes with a wide margin
    y32, f32 = _serial32(inp)
    assert metrics.componentwise_err(y32, yr, ya) < 1e-6
    assert metrics.componentwise_err(f32, fr, fa) < 1e-5
    # reading the state through bf16 fails it
    yb, _ = _serial32(inp, round_state=lambda S: round_to_bf16(S))
    assert metrics.componentwise_err(yb, yr, ya) > 1e-4
    # a wrong sign on one output element fails it
    yw = y32.copy()
    yw[0, 100, 1, 7] *= -1
    assert metrics.componentwise_err(yw, yr, ya) > 1e-2
    # the magnitude reference bounds the result
    assert np.all(np.abs(yr) <= ya * (1 + 1e-12))


def test_componentwise_zero_reference_must_be_exact():
    assert metrics.componentwise_err([0.0, 1.0], [0.0, 1.0], [0.0, 2.0]) == 0.0
    assert metrics.componentwise_err([1e-30, 1.0], [0.0, 1.0], [0.0, 2.0]) == np.inf
