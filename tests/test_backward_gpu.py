"""GPU parity of the gradient pass (ssd_chunk_scan_bwd) against the fp64
oracle's reverse-mode loop, every element, through the C ABI.

Bar (normwise relative error of each gradient tensor, ||got - ref|| /
||ref||): fp32 runs 1e-4 (the forward's fp32 bar; fp32 accumulation and
fp32 operands leave about 1e-6), bf16 runs 2e-2 (the forward's bf16 bar:
the bf16 rounding of dx, dB and dC and of the products' operands is 2^-9
relative per term).  The same bars hold for dA: the kernels form its terms
without the large cancellation of the plain chunked form (a prefix sum over
the chunk of <dy, y - D x> - dt x . u loses about 1e-4 in fp32 and 3e-2 in
bf16 on these cases; the one difference they keep, of the strict row and
column sums of W, is summed in fp64).  Every gradient is also checked for
non-finite values.
"""
import numpy as np
import pytest

from state_space_sequence_amd.inputs import make_grad_inputs, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
KEYS = ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit")


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from state_space_sequence_amd import libssd
    libssd.load()
    return torch.device("cuda:0")


def _run(dev, inp, g, io, Q, D=True, init=True, dfinal=True):
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    t = to_torch(inp, io, dev)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    dy = torch.from_numpy(g["dy"]).to(tdt).to(dev)
    df = torch.from_numpy(g["dfinal"]).to(dev) if dfinal else None
    out = libssd.ssd_chunk_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"],
                                    t["D"] if D else None,
                                    t["initial_state"] if init else None, dy, df,
                                    chunk_len=Q)
    torch.cuda.synchronize()
    return {k: out[k].float().cpu().numpy().astype(np.float64) for k in KEYS}


def _ref(oracle_mod, inp, g, D=True, init=True, dfinal=True):
    return oracle_mod.backward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                               inp["D"] if D else None, inp["initial_state"] if init else None,
                               g["dy"], g["dfinal"] if dfinal else None)


def _check(got, ref, io, what):
    for k in KEYS:
        err = float(np.linalg.norm(got[k] - ref[k]) / max(np.linalg.norm(ref[k]), 1e-30))
        tol = TOL[io]
        _say("  %-40s %-5s err=%.3e tol=%.0e" % (what, k, err, tol))
        assert np.all(np.isfinite(got[k])), "%s %s has non-finite values" % (what, k)
        assert err <= tol, "%s %s: %.3e > %.0e" % (what, k, err, tol)


CASES = [
    # b, L, H, P, N, G, Q, io, init
    (1, 64, 2, 16, 16, 1, 16, "f32", True),
    (2, 77, 4, 32, 64, 2, 32, "f32", True),
    (1, 300, 4, 64, 128, 1, 64, "f32", True),
    (2, 513, 3, 48, 48, 3, 128, "f32", False),
    (1, 600, 2, 64, 128, 1, 256, "f32", True),
    (1, 256, 2, 128, 256, 1, 256, "f32", True),
    (1, 40, 2, 16, 32, 2, 16, "bf16", True),
    (1, 300, 4, 32, 64, 2, 64, "bf16", True),
    (2, 1000, 8, 64, 128, 8, 256, "bf16", True),
    (1, 257, 4, 96, 128, 4, 128, "bf16", True),
    (1, 512, 2, 128, 256, 1, 256, "bf16", False),
    (2, 333, 6, 64, 128, 1, 64, "bf16", True),
    # a multiple of 8 chunks: the dB / dC kernels place a chunk's row blocks
    # on one XCD (a different workgroup-to-tile map)
    (1, 1024, 4, 64, 128, 2, 128, "bf16", True),
    (1, 2048, 2, 32, 64, 1, 256, "f32", False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b%d_L%d_H%d_P%d_N%d_G%d_Q%d_%s%s" % (
    c[:8] + ("_init" if c[8] else "",)))
def test_backward_every_element(dev, oracle_mod, case):
    b, L, H, P, N, G, Q, io, init = case
    _say("case %s" % (case,))
    inp = make_inputs(b, L, H, P, N, G, io, init_std=0.1 if init else 0.0, seed=7 + L)
    g = make_grad_inputs(b, L, H, P, N, io, seed=11 + L)
    got = _run(dev, inp, g, io, Q)
    ref = _ref(oracle_mod, inp, g)
    _check(got, ref, io, "b%d L%d H%d P%d N%d G%d Q%d" % case[:7])


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_backward_optional_arguments(dev, oracle_mod, io):
    """No D, no initial state, no dfinal: the gradients at D = 0 and a zero
    initial state, with dLoss/dfinal = 0."""
    inp = make_inputs(1, 200, 4, 64, 128, 2, io, init_std=0.0, seed=3)
    g = make_grad_inputs(1, 200, 4, 64, 128, io, seed=4)
    got = _run(dev, inp, g, io, 64, D=False, init=False, dfinal=False)
    ref = _ref(oracle_mod, inp, g, D=False, init=False, dfinal=False)
    _check(got, ref, io, "no D / init / dfinal")


def test_backward_chunk_length_invariance(dev, oracle_mod):
    """The gradients do not depend on the chunk length beyond rounding."""
    inp = make_inputs(1, 300, 4, 64, 128, 1, "f32", init_std=0.1, seed=5)
    g = make_grad_inputs(1, 300, 4, 64, 128, "f32", seed=6)
    ref = _ref(oracle_mod, inp, g)
    for Q in (16, 32, 64, 128, 256):
        _check(_run(dev, inp, g, "f32", Q), ref, "f32", "Q=%d" % Q)


def test_backward_deterministic(dev):
    """Two calls give the same bits (dA and dD are summed in a fixed order)."""
    import torch
    inp = make_inputs(2, 500, 8, 64, 128, 2, "bf16", init_std=0.1, seed=8)
    g = make_grad_inputs(2, 500, 8, 64, 128, "bf16", seed=9)
    a = _run(dev, inp, g, "bf16", 256)
    b = _run(dev, inp, g, "bf16", 256)
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k
    torch.cuda.synchronize()


def test_backward_full_size_sampled_heads(dev, oracle_mod):
    """The 2.7B-shape layer (b4 L8192 H80 P64 N128 G1, Q256, bf16) in the
    launch configuration bench times, against the oracle on three sampled
    heads: their dx, ddt and dinit, and dA and dD (sums over the batch).  A
    head's gradients depend only on its own inputs and the shared B and C,
    so the oracle runs on those heads alone; dB and dC sum over all 80 heads
    of the group, which a sample does not give (they are checked every
    element on the smaller cases)."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import WORKLOADS, to_torch, workload_inputs
    w = WORKLOADS["mamba2_2p7b"]
    _say("workload %s, backward, sampled heads" % w.name)
    inp = workload_inputs(w)
    g = make_grad_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.io_dtype, seed=5)
    t = to_torch(inp, w.io_dtype, dev)
    dy = torch.from_numpy(g["dy"]).to(torch.bfloat16).to(dev)
    df = torch.from_numpy(g["dfinal"]).to(dev)
    out = libssd.ssd_chunk_scan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                    t["initial_state"], dy, df, chunk_len=w.chunk_len)
    torch.cuda.synchronize()
    heads = [0, 41, 79]
    hs = torch.tensor(heads, device=dev)
    got = {"dx": out["dx"].index_select(2, hs), "ddt": out["ddt"].index_select(2, hs),
           "dinit": out["dinit"].index_select(1, hs), "dA": out["dA"][hs], "dD": out["dD"][hs]}
    got = {k: v.float().cpu().numpy().astype(np.float64) for k, v in got.items()}
    del out, t, dy, df
    D, init = inp["D"], inp["initial_state"]   # (the workload has no initial state)
    ref = oracle_mod.backward(inp["x"][:, :, heads], inp["dt"][:, :, heads], inp["A"][heads],
                              inp["B"], inp["C"], None if D is None else D[heads],
                              None if init is None else init[:, heads], g["dy"][:, :, heads],
                              g["dfinal"][:, heads])
    for k in ("dx", "ddt", "dA", "dD", "dinit"):
        err = float(np.linalg.norm(got[k] - ref[k]) / max(np.linalg.norm(ref[k]), 1e-30))
        _say("  2.7B heads %s %-5s err=%.3e tol=%.0e" % (heads, k, err, TOL["bf16"]))
        assert np.all(np.isfinite(got[k])), k
        assert err <= TOL["bf16"], "%s: %.3e" % (k, err)
