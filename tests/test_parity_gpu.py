"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bar: fp32 inputs -> max componentwise relative error <= 1e-4, measured
against the magnitude of the summed terms (the oracle on absolute-valued
inputs), and the relative error floored at 1e-3 max|o| no worse than twice
the textbook fp32 recurrence's on the same inputs (never above 1e-4 where
that recurrence meets it); bf16 inputs -> normwise relative error <= 2e-2,
on y and on the final state separately, and on y also over every 32-token
block of every (batch, head) slice (oracle/metrics.py).  Small problems are
compared element by element on every output; the full-size workloads on
every (batch, head) slice as well.
"""
import sys

import numpy as np
import pytest

from oracle import metrics
from oracle.metrics import abs_inputs
from state_space_sequence_amd.inputs import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from state_space_sequence_amd import libssd
    libssd.load()
    return torch.device("cuda:0")


@pytest.fixture(params=["split", "fused"])
def path(request, monkeypatch):
    """Run the test through one forward path (the library reads
    SSD_FORWARD_PATH on every call): the split kernels or the fused pass."""
    monkeypatch.setenv("SSD_FORWARD_PATH", request.param)
    return request.param


def skip_if_path_unsupported(inp, io, Q):
    from state_space_sequence_amd import libssd
    b, L, H, P = inp["x"].shape
    G, N = inp["B"].shape[2], inp["B"].shape[3]
    try:
        libssd.ssd_chunk_scan_fwd_workspace_size(b, L, H, P, N, G, Q,
                                                 libssd.SSD_BF16 if io == "bf16" else libssd.SSD_F32)
    except libssd.SsdError as e:
        if e.status == libssd.SSD_ERR_UNSUPPORTED:
            pytest.skip("shape not covered by this forward path")
        raise


def gpu_forward(inp, io, Q, dev, init=True, final=True, D=True):
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    t = to_torch(inp, io, dev)
    y, fin = libssd.ssd_chunk_scan_fwd(
        t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"] if D else None,
        t["initial_state"] if init else None, chunk_len=Q, ngroups=t["B"].shape[2],
        return_final_state=final)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), (None if fin is None else fin.cpu().numpy())


def reference(oracle_mod, inp, want_abs=True):
    """(y, final, y_abs, final_abs) from the fp64 oracle."""
    args = ("x", "dt", "A", "B", "C", "D", "initial_state")
    yr, fr = oracle_mod.forward(*(inp[k] for k in args))
    if not want_abs:
        return yr, fr, None, None
    ia = abs_inputs(inp)
    ya, fa = oracle_mod.forward(*(ia[k] for k in args))
    return yr, fr, ya, fa


FWD_ARGS = ("x", "dt", "A", "B", "C", "D", "initial_state")


def textbook32(inp):
    """(y, final) of the textbook fp32 recurrence on these inputs (sets the
    floored fp32 bar)."""
    from oracle.forms import serial_fp32
    return serial_fp32(*(inp[k] for k in FWD_ARGS))


def check(got, ref, io, what, ref_abs=None, ref32=None, tok_axis=None):
    err = metrics.parity_error(got, ref, io, ref_abs)
    tol = metrics.tolerance(io)
    msg = "  %-28s err=%.3e tol=%.0e" % (what, err, tol)
    fl = bar = None
    if io == "f32":
        fl = metrics.max_rel_err(got, ref)
        msg += "  floored=%.3e" % fl
        if ref32 is not None:
            bar = metrics.fp32_floored_bar(metrics.max_rel_err(ref32, ref))
            msg += " (bar %.2e)" % bar
    blk = None
    if io == "bf16" and tok_axis is not None:
        blk, where = metrics.block_normwise_err(got, ref, tok_axis)
        msg += "  worst 32-token block %.3e at %s" % (blk, where)
    _say(msg)
    assert np.all(np.isfinite(got)), what + " has non-finite values"
    assert err <= tol, "%s: error %.3e > %.0e" % (what, err, tol)
    if bar is not None:
        assert fl <= bar, "%s: floored error %.3e > %.2e" % (what, fl, bar)
    if blk is not None:
        assert blk <= tol, "%s: 32-token block %s error %.3e > %.0e" % (what, where, blk, tol)


SMALL = [
    # b, L, H, P, N, G, Q, io, init
    (1, 1, 2, 16, 16, 1, 16, "f32", False),
    (2, 17, 4, 16, 32, 2, 16, "f32", True),
    (1, 300, 4, 32, 64, 2, 64, "bf16", True),
    (2, 513, 3, 48, 48, 3, 128, "f32", True),
    (1, 256, 2, 128, 256, 1, 256, "bf16", False),
    (1, 256, 2, 128, 256, 1, 256, "f32", True),
    (2, 1000, 8, 64, 128, 8, 256, "bf16", True),
    (1, 100, 2, 64, 128, 1, 32, "bf16", True),
    (1, 64, 2, 16, 16, 2, 64, "f32", True),
    (3, 700, 4, 64, 128, 1, 256, "f32", True),
    (2, 300, 4, 64, 128, 2, 64, "bf16", True),
    (1, 1000, 4, 32, 128, 1, 256, "bf16", True),
    (2, 777, 4, 64, 128, 2, 128, "f32", True),
    (1, 40, 2, 16, 128, 1, 32, "f32", True),
    (1, 33, 2, 32, 128, 2, 32, "bf16", False),
    (1, 512, 2, 128, 128, 1, 256, "bf16", True),
    (2, 257, 4, 96, 128, 4, 128, "bf16", True),
    # more 64-column workgroups than compute units: the fused path's
    # four-wave layout over two heads of one group (ragged tail)
    (2, 200, 132, 64, 128, 2, 64, "bf16", True),
    # more 32-column workgroups than compute units: the two-wave layout,
    # also with an odd head count
    (2, 300, 66, 64, 128, 1, 64, "bf16", True),
    (1, 130, 129, 64, 128, 1, 64, "bf16", False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b%d_L%d_H%d_P%d_N%d_G%d_Q%d_%s%s" % (
    c[:8] + ("_init" if c[8] else "",)))
def test_small_problems_every_element(dev, oracle_mod, path, case):
    b, L, H, P, N, G, Q, io, init = case
    _say("case %s path %s" % (case, path))
    inp = make_inputs(b, L, H, P, N, G, io_dtype=io, init_std=0.1 if init else 0.0,
                      seed=100 + L)
    skip_if_path_unsupported(inp, io, Q)
    y, fin = gpu_forward(inp, io, Q, dev)
    yr, finr, ya, fa = reference(oracle_mod, inp)
    y32, f32 = textbook32(inp) if io == "f32" else (None, None)
    check(y, yr, io, "y", ya, ref32=y32, tok_axis=1)
    check(fin, finr, io, "final_state", fa, ref32=f32)
    if io == "bf16":
        # bf16 inputs are checked normwise; also report the componentwise score
        _say("  componentwise y %.2e (informational)" % metrics.componentwise_err(y, yr, ya))


def decay_regime_inputs(io, seed, H=4):
    """Per-head decay profiles that cross every regime of the fused path in
    one sequence: weak decay, repeated rescaling of the tracked state scale
    (block decays of 20-40), blocks whose total decay exceeds exp(-60) (the
    exact per-element weights, dt A summed over 32 tokens down to -300), and
    factored blocks again after them; ragged length, initial state.  The
    four decay rates repeat over the heads."""
    L = 400
    inp = make_inputs(2, L, H, 64, 128, 1, io_dtype=io, init_std=0.1, seed=seed)
    t = np.arange(L)
    prof = np.where(t < 96, 0.01, np.where(t < 192, 0.25, np.where(t < 288, 0.08, 0.6)))
    rng = np.random.default_rng(seed)
    jitter = 1.0 + 0.2 * rng.standard_normal(size=(2, L, H))
    inp["A"] = np.resize(np.array([-16.0, -8.0, -2.0, -0.5], dtype=np.float32), H)
    inp["dt"] = (prof[None, :, None] * np.abs(jitter)).astype(np.float32)
    return inp


@pytest.mark.parametrize("io,H", [("bf16", 4), ("f32", 4), ("bf16", 66), ("bf16", 132)])
def test_decay_regimes(dev, oracle_mod, path, io, H):
    inp = decay_regime_inputs(io, seed=91, H=H)
    lam = inp["dt"][0, : 384].reshape(12, 32, H).sum(1) * inp["A"][None, :]
    _say("block decays per head: min %.1f max %.1f" % (-lam.max(), -lam.min()))
    assert (-lam > 60).any() and ((-lam > 20) & (-lam < 60)).any() and (-lam < 5).any()
    skip_if_path_unsupported(inp, io, 64)
    y, fin = gpu_forward(inp, io, 64, dev)
    yr, finr, ya, fa = reference(oracle_mod, inp)
    y32, f32 = textbook32(inp) if io == "f32" else (None, None)
    check(y, yr, io, "y", ya, ref32=y32, tok_axis=1)
    check(fin, finr, io, "final_state", fa, ref32=f32)


def test_tiny_workload(dev, oracle_mod):
    w = WORKLOADS["tiny_f32"]
    inp = workload_inputs(w)
    y, fin = gpu_forward(inp, w.io_dtype, w.chunk_len, dev)
    yr, finr, ya, fa = reference(oracle_mod, inp)
    y32, f32 = textbook32(inp)
    check(y, yr, "f32", "tiny y", ya, ref32=y32)
    check(fin, finr, "f32", "tiny final", fa, ref32=f32)


def _sample_slices(b, H, n, seed):
    rng = np.random.default_rng(seed)
    sl = {(0, 0), (b - 1, H - 1), (0, H - 1), (b - 1, 0)}
    while len(sl) < n:
        sl.add((int(rng.integers(b)), int(rng.integers(H))))
    return sorted(sl)


def check_every_slice(y, fin, yr, fr, io, what, ya=None, fa=None):
    """y and the final state against the oracle over the whole workload: the
    whole arrays, every (batch, head) slice's final state, and every 32-token
    block of every slice of y (fp32: every element, against the magnitude
    references ya and fa)."""
    check(y, yr, io, what + " y (every slice)", ya, tok_axis=1)
    check(fin, fr, io, what + " final (every slice)", fa)
    d = np.sqrt(((fin.astype(np.float64) - fr) ** 2).sum(axis=(-2, -1)))
    o = np.sqrt((fr ** 2).sum(axis=(-2, -1)))
    r = d / np.where(o > 0, o, 1.0)
    _say("  worst final-state slice %.3e at %s" % (r.max(), np.unravel_index(r.argmax(), r.shape)))
    assert r.max() <= metrics.tolerance(io)


@pytest.mark.parametrize("name", ["mamba2_130m", "mamba2_2p7b", "grouped_g8", "mamba2_130m_f32"])
def test_full_size_workloads_every_slice(dev, oracle_mod, path, name):
    w = WORKLOADS[name]
    _say("workload %s path %s" % (name, path))
    inp = workload_inputs(w)
    skip_if_path_unsupported(inp, w.io_dtype, w.chunk_len)
    y, fin = gpu_forward(inp, w.io_dtype, w.chunk_len, dev)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(fin))
    # every (batch, head) slice: the serial oracle over the whole workload
    yr, fr = oracle_mod.forward(*(inp[k] for k in FWD_ARGS))
    ya = fa = None
    if w.io_dtype == "f32":
        ia = abs_inputs(inp)
        ya, fa = oracle_mod.forward(*(ia[k] for k in FWD_ARGS))
    check_every_slice(y, fin, yr, fr, w.io_dtype, name, ya, fa)


def test_chunk_length_invariance_on_gpu(dev, oracle_mod):
    inp = make_inputs(2, 777, 4, 64, 128, 2, io_dtype="f32", init_std=0.1, seed=5)
    outs = {Q: gpu_forward(inp, "f32", Q, dev) for Q in (16, 32, 64, 128, 256)}
    yr, finr, ya, fa = reference(oracle_mod, inp)
    y32, f32 = textbook32(inp)
    for Q, (y, fin) in outs.items():
        check(y, yr, "f32", "Q=%d y" % Q, ya, ref32=y32)
        check(fin, finr, "f32", "Q=%d final" % Q, fa, ref32=f32)


@pytest.mark.parametrize("N", [32, 128])
def test_optional_arguments(dev, oracle_mod, N):
    inp = make_inputs(1, 200, 2, 32, N, 1, io_dtype="f32", init_std=0.1, seed=6)
    y, fin = gpu_forward(inp, "f32", 64, dev, init=False, final=False, D=False)
    assert fin is None
    inp0 = dict(inp, D=None, initial_state=None)
    yr, _, ya, _ = reference(oracle_mod, inp0)
    check(y, yr, "f32", "no D / no init / no final", ya, ref32=textbook32(inp0)[0])


def test_final_state_may_alias_initial_state(dev, oracle_mod, path):
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    inp = make_inputs(2, 300, 4, 64, 128, 1, io_dtype="bf16", init_std=0.1, seed=8)
    t = to_torch(inp, "bf16", dev)
    cache = t["initial_state"].clone()
    libssd.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], cache,
                              chunk_len=128, final_state=cache)
    torch.cuda.synchronize()
    _, finr = oracle_mod.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                                 inp["D"], inp["initial_state"])
    check(cache.cpu().numpy(), finr, "bf16", "aliased final")


def test_deterministic(dev, path):
    inp = make_inputs(2, 600, 8, 64, 128, 2, io_dtype="bf16", init_std=0.1, seed=9)
    y1, f1 = gpu_forward(inp, "bf16", 256, dev)
    y2, f2 = gpu_forward(inp, "bf16", 256, dev)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(f1, f2)


def test_timed_variant_matches_and_names_kernels(dev, path):
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    inp = make_inputs(1, 300, 4, 64, 128, 1, io_dtype="bf16", init_std=0.1, seed=10)
    t = to_torch(inp, "bf16", dev)
    hip = __import__("ctypes").CDLL("libamdhip64.so")
    evs = []
    for _ in range(libssd.max_kernels() + 1):
        e = __import__("ctypes").c_void_p()
        assert hip.hipEventCreate(__import__("ctypes").byref(e)) == 0
        evs.append(e.value)
    y1, f1 = libssd.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                       t["initial_state"], chunk_len=128)
    y2, f2, names = libssd.ssd_chunk_scan_fwd_timed(evs, t["x"], t["dt"], t["A"], t["B"],
                                                    t["C"], t["D"], t["initial_state"],
                                                    chunk_len=128)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(f1, f2)
    if path == "split":
        assert names == ["k1_dA_cumsum", "k2_chunk_cb", "k3_chunk_state", "k4_state_passing",
                         "k5_chunk_scan"]
    else:
        assert names == ["k_fused_ssd"]
    for e in evs:
        hip.hipEventDestroy(__import__("ctypes").c_void_p(e))


# ------------------------------------------------------------------ decode

def _decode_run(inp, io, dev, steps):
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    t = to_torch(inp, io, dev)
    state = t["initial_state"].clone()
    ys = []
    for s in range(steps):
        y = libssd.ssd_state_update(state, t["x"][:, s].contiguous(), t["dt"][:, s].contiguous(),
                                    t["A"], t["B"][:, s].contiguous(), t["C"][:, s].contiguous(),
                                    t["D"])
        ys.append(y)
    torch.cuda.synchronize()
    return torch.stack(ys, 1).float().cpu().numpy(), state.cpu().numpy(), t


# dstate 16, 32, 64, 80, 128 (workload), 256: 4, 8, 16, 32 (partly idle) and 64
# lanes per state row; headdim 112 leaves the last of eight row passes
# of a thread past the end (clamped loads, predicated stores)
@pytest.mark.parametrize("case", [(3, 5, 4, 16, 16, 2, "f32"), (2, 9, 6, 48, 80, 3, "bf16"),
                                  (2, 4, 2, 128, 256, 1, "f32"), (2, 3, 4, 32, 32, 1, "bf16"),
                                  (1, 3, 2, 112, 64, 2, "f32")])
def test_decode_small_every_element(dev, oracle_mod, case):
    b, steps, H, P, N, G, io = case
    inp = make_inputs(b, steps, H, P, N, G, io_dtype=io, init_std=0.1, seed=20 + P)
    y, state, _ = _decode_run(inp, io, dev, steps)
    yr, finr, ya, fa = reference(oracle_mod, inp)
    y32, f32 = textbook32(inp) if io == "f32" else (None, None)
    check(y, yr, io, "decode y", ya, ref32=y32, tok_axis=1)
    check(state, finr, io, "decode state", fa, ref32=f32)


def test_decode_workload_vs_serial_and_chunked(dev, oracle_mod, path):
    """64 decode steps of the b256 workload: against the serial oracle on
    sampled slices, and against the chunked forward over the same 64 tokens
    started from the same state (final state and every output)."""
    import torch
    from state_space_sequence_amd import libssd
    w = WORKLOADS["decode_b256"]
    _say("decode workload")
    inp = make_inputs(w.batch, w.decode_steps, w.nheads, w.headdim, w.dstate, w.ngroups,
                      io_dtype=w.io_dtype, init_std=w.init_std, seed=w.seed)
    y, state, t = _decode_run(inp, w.io_dtype, dev, w.decode_steps)
    # every (batch, head) slice against the serial oracle
    yr, fr = oracle_mod.forward(*(inp[k] for k in FWD_ARGS))
    check_every_slice(y, state, yr, fr, "bf16", "decode vs serial")
    yc, fc = libssd.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                       t["initial_state"], chunk_len=w.chunk_len)
    torch.cuda.synchronize()
    check(state, fc.cpu().numpy(), "bf16", "decode state vs chunked")
    check(y, yc.float().cpu().numpy(), "bf16", "decode y vs chunked")


# ------------------------------------------------------ time-step preprocessing

# (b, L, H, P, N, G, Q, io, softplus, dt_limit, bias shift or None for no bias)
DT_PROC = [
    # the layer's call: softplus(dt + dt_bias), limits (0, inf)
    (2, 300, 4, 64, 128, 1, 64, "bf16", True, None, 0.0),
    (2, 300, 4, 64, 128, 2, 64, "f32", True, None, 0.0),
    # both clamp bounds active
    (2, 333, 4, 64, 128, 2, 128, "bf16", True, (0.002, 0.05), 0.0),
    (1, 200, 3, 32, 128, 1, 32, "f32", True, (0.002, 0.05), 0.0),
    # no softplus: the biased value floored at 0 (bias shifted so that both
    # signs occur; large dt drives the exact per-element blocks)
    (1, 257, 4, 64, 128, 1, 64, "bf16", False, None, 5.0),
    # softplus of the raw value alone
    (1, 130, 2, 16, 32, 1, 64, "f32", True, None, None),
]


@pytest.mark.parametrize("case", DT_PROC, ids=lambda c: "b%d_L%d_H%d_P%d_N%d_G%d_Q%d_%s" % c[:8]
                         + ("_sp" if c[8] else "") + ("_lim" if c[9] else "")
                         + ("_nobias" if c[10] is None else ""))
def test_dt_preprocessing(dev, oracle_mod, path, case):
    """The `_ex` forward on the raw time step against the oracle run on the
    oracle's own preprocessing of it (oracle/dt.py)."""
    import torch
    from oracle.dt import process_dt
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    b, L, H, P, N, G, Q, io, sp, lim, shift = case
    _say("dt preprocessing case %s path %s" % (case, path))
    inp = make_inputs(b, L, H, P, N, G, io_dtype=io, init_std=0.1, seed=300 + L)
    skip_if_path_unsupported(inp, io, Q)
    bias = None if shift is None else (inp["dt_bias"] + np.float32(shift)).astype(np.float32)
    dtp = process_dt(inp["dt_raw"], bias, sp, *(lim or (0.0, np.inf)))
    if lim:
        assert (dtp == lim[0]).any() and (dtp == lim[1]).any()
    if not sp:
        assert (dtp == 0).any() and (dtp > 1).any()
    t = to_torch(inp, io, dev)
    tb = None if bias is None else torch.from_numpy(bias).to(dev)
    y, fin = libssd.ssd_chunk_scan_fwd(t["x"], t["dt_raw"], t["A"], t["B"], t["C"], t["D"],
                                       t["initial_state"], chunk_len=Q, ngroups=G, dt_bias=tb,
                                       dt_softplus=sp, dt_limit=lim)
    torch.cuda.synchronize()
    inp_p = dict(inp, dt=dtp)
    yr, finr, ya, fa = reference(oracle_mod, inp_p)
    y32, f32 = textbook32(inp_p) if io == "f32" else (None, None)
    check(y.float().cpu().numpy(), yr, io, "y", ya, ref32=y32, tok_axis=1)
    check(fin.cpu().numpy(), finr, io, "final_state", fa, ref32=f32)


def test_dt_preprocessing_identity_is_bit_exact(dev, path):
    """Preprocessing that is the identity on the (non-negative) processed dt:
    no bias, no softplus, limits (0, inf).  Same bits as the plain call."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    inp = make_inputs(2, 300, 4, 64, 128, 1, io_dtype="bf16", init_std=0.1, seed=17)
    skip_if_path_unsupported(inp, "bf16", 64)
    t = to_torch(inp, "bf16", dev)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["initial_state"])
    y1, f1 = libssd.ssd_chunk_scan_fwd(*args, chunk_len=64)
    y2, f2 = libssd.ssd_chunk_scan_fwd(*args, chunk_len=64, dt_limit=(0.0, float("inf")))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_decode_dt_preprocessing(dev, oracle_mod, io):
    """`ssd_state_update_ex` steps on the raw time step (bias, softplus, an
    active upper bound) against the serial oracle on the processed one."""
    import torch
    from oracle.dt import process_dt
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    b, steps, H, P, N, G = 3, 7, 4, 64, 128, 2
    inp = make_inputs(b, steps, H, P, N, G, io_dtype=io, init_std=0.1, seed=41)
    lim = (0.0, 0.08)
    dtp = process_dt(inp["dt_raw"], inp["dt_bias"], True, *lim)
    assert (dtp == lim[1]).any() and (dtp < lim[1]).any()
    t = to_torch(inp, io, dev)
    state = t["initial_state"].clone()
    ys = []
    for s in range(steps):
        ys.append(libssd.ssd_state_update(state, t["x"][:, s].contiguous(),
                                          t["dt_raw"][:, s].contiguous(), t["A"],
                                          t["B"][:, s].contiguous(), t["C"][:, s].contiguous(),
                                          t["D"], dt_bias=t["dt_bias"], dt_softplus=True,
                                          dt_limit=lim))
    torch.cuda.synchronize()
    y = torch.stack(ys, 1).float().cpu().numpy()
    inp_p = dict(inp, dt=dtp)
    yr, finr, ya, fa = reference(oracle_mod, inp_p)
    y32, f32 = textbook32(inp_p) if io == "f32" else (None, None)
    check(y, yr, io, "decode y", ya, ref32=y32, tok_axis=1)
    check(state.cpu().numpy(), finr, io, "decode state", fa, ref32=f32)


# ------------------------------------------------------ causal depthwise conv

# (b, L, dim, width, io, bias, activation)
CONV = [
    (2, 300, 96, 4, "bf16", True, "silu"),
    (1, 70, 40, 4, "f32", True, "silu"),        # ragged 64-token run
    (3, 3, 16, 4, "bf16", False, None),          # seqlen < width
    (2, 129, 2056, 3, "f32", True, "silu"),      # two 256-lane channel blocks, the second partial
    (1, 65, 8, 2, "bf16", True, "silu"),         # width 2, one channel group
    (2, 1, 24, 4, "f32", True, None),            # a single token
]


def _conv_ref(x, w, bias, act):
    from oracle.conv import causal_conv1d
    ref = causal_conv1d(x, w, bias, act)
    mag = causal_conv1d(np.abs(x), np.abs(w), None if bias is None else np.abs(bias), None)
    return ref, mag


@pytest.mark.parametrize("case", CONV, ids=lambda c: "b%d_L%d_D%d_W%d_%s" % c[:5]
                         + ("_bias" if c[5] else "") + ("_" + c[6] if c[6] else ""))
def test_causal_conv1d_every_element(dev, case):
    import torch
    from oracle.conv import conv_state_after
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_conv_inputs
    b, L, D, W, io, use_bias, act = case
    _say("conv case %s" % (case,))
    inp = make_conv_inputs(b, L, D, W, io_dtype=io, seed=500 + L + D)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    x = torch.from_numpy(inp["x"]).to(tdt).to(dev)
    w = torch.from_numpy(inp["weight"]).to(dev)
    bias = torch.from_numpy(inp["bias"]).to(dev) if use_bias else None
    out, state = libssd.ssd_causal_conv1d_fwd(x, w, bias, activation=act)
    torch.cuda.synchronize()
    ref, mag = _conv_ref(inp["x"], inp["weight"], inp["bias"] if use_bias else None, act)
    check(out.float().cpu().numpy(), ref, io, "conv out", mag)
    # the cache holds inputs (exact copies)
    np.testing.assert_array_equal(state.float().cpu().numpy(), conv_state_after(inp["x"], W))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_causal_conv1d_prefill_then_decode(dev, io):
    """The layer's sequence: a prefill over L tokens leaves the cache, then
    single-token updates continue from it; outputs against the oracle over
    the whole L + steps tokens."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_conv_inputs
    b, L, D, W, steps = 3, 37, 264, 4, 6
    inp = make_conv_inputs(b, L, D, W, io_dtype=io, seed=77, decode_steps=steps)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    x = torch.from_numpy(inp["x"]).to(tdt).to(dev)
    w = torch.from_numpy(inp["weight"]).to(dev)
    bias = torch.from_numpy(inp["bias"]).to(dev)
    out, state = libssd.ssd_causal_conv1d_fwd(x, w, bias, activation="silu")
    outs = []
    for s in range(steps):
        xs = torch.from_numpy(inp["x_dec"][s]).to(tdt).to(dev).contiguous()
        outs.append(libssd.ssd_causal_conv1d_update(state, xs, w, bias, activation="silu"))
    torch.cuda.synchronize()
    xall = np.concatenate([inp["x"], inp["x_dec"].transpose(1, 0, 2)], axis=1)
    ref, mag = _conv_ref(xall, inp["weight"], inp["bias"], "silu")
    check(out.float().cpu().numpy(), ref[:, :L], io, "prefill out", mag[:, :L])
    got = torch.stack(outs, 1).float().cpu().numpy()
    check(got, ref[:, L:], io, "decode out", mag[:, L:])


# (batch, dim, width, io, bias, activation, misalign): misalign shifts x and
# the cache by one element off their 16-byte alignment
CONV_UPD = [
    (256, 5376, 4, "bf16", True, "silu", False),  # the 2.7B layer's channels, b256
    (3, 264, 4, "f32", True, "silu", False),      # four channels per thread, fp32
    (1, 1032, 4, "f32", False, None, False),      # 258 threads: a partial second workgroup
    (2, 8, 4, "bf16", True, "silu", False),       # the smallest dim: two threads
    (2, 40, 3, "f32", False, None, False),        # width 3
    (5, 1032, 2, "bf16", True, "silu", False),    # width 2, a partial last workgroup
    (2, 264, 4, "bf16", True, "silu", True),      # misaligned x and cache: one channel per thread
]


@pytest.mark.parametrize("case", CONV_UPD, ids=lambda c: "b%d_dim%d_w%d_%s_%s_%s_%s" % c)
def test_causal_conv1d_update_every_element(dev, case):
    """One decode token of the conv from a full cache: out and the rolled
    cache against the oracle's update (the cache bit for bit: it holds
    inputs)."""
    import torch
    from oracle.conv import conv_state_after, conv_update
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_conv_inputs
    b, D, W, io, use_bias, act, mis = case
    _say("conv update case %s" % (case,))
    inp = make_conv_inputs(b, W, D, W, io_dtype=io, seed=700 + D + W, decode_steps=1)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    st0 = conv_state_after(inp["x"], W)           # [b, D, W], every slot filled
    x1 = inp["x_dec"][0]
    off = 1 if mis else 0

    def place(a):
        flat = torch.zeros(a.size + off, dtype=tdt, device=dev)
        flat[off:] = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).ravel()).to(tdt).to(dev)
        return flat[off:].view(*a.shape)
    state = place(st0)
    xs = place(x1)
    w = torch.from_numpy(inp["weight"]).to(dev)
    bias = torch.from_numpy(inp["bias"]).to(dev) if use_bias else None
    out = libssd.ssd_causal_conv1d_update(state, xs, w, bias, activation=act)
    torch.cuda.synchronize()
    ref, ref_state = conv_update(st0, x1, inp["weight"], inp["bias"] if use_bias else None, act)
    assert np.array_equal(state.float().cpu().numpy(), ref_state.astype(np.float32))
    check(out.float().cpu().numpy(), ref, io, "update out", np.abs(ref))


# ------------------------------------------------------ gated RMS normalisation

# (rows, dim, io, gate: "before" | "after" | None)
NORM = [
    # (8-value vectors per row -> threads x vectors per thread)
    (300, 512, "bf16", "before"),      # the layer's order; 64 -> 64 x 1
    (37, 5120, "bf16", "before"),      # the 2.7B layer's row; 640 -> 320 x 2
    (64, 1536, "f32", "before"),       # the 130M layer's row; 192 -> 192 x 1
    (5, 8192, "f32", "after"),         # the largest row; 1024 -> 512 x 2
    (9, 40, "bf16", None),             # shorter than a wave; 5 -> 64 x 1
    (130, 2056, "f32", None),          # 257 -> 192 x 2, the second partly clamped
]


@pytest.mark.parametrize("case", NORM, ids=lambda c: "rows%d_dim%d_%s_%s" % c)
def test_gated_rmsnorm_every_element(dev, case):
    import torch
    from oracle.norm import gated_rmsnorm
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_norm_inputs
    rows, dim, io, gate = case
    _say("norm case %s" % (case,))
    inp = make_norm_inputs(rows, dim, io_dtype=io, seed=600 + dim)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    y = torch.from_numpy(inp["y"]).to(tdt).to(dev)
    z = torch.from_numpy(inp["z"]).to(tdt).to(dev) if gate else None
    w = torch.from_numpy(inp["weight"]).to(dev)
    out = libssd.ssd_gated_rmsnorm_fwd(y, z, w, eps=1e-5, norm_before_gate=gate == "after")
    torch.cuda.synchronize()
    ref = gated_rmsnorm(inp["y"], inp["z"] if gate else None, inp["weight"], 1e-5,
                        norm_before_gate=gate == "after")
    # each output is a product of its inputs and the row's scale: no
    # cancellation, so the magnitude reference is the output itself
    check(out.float().cpu().numpy(), ref, io, "norm out", np.abs(ref))


def test_gated_rmsnorm_in_place(dev):
    import torch
    from oracle.norm import gated_rmsnorm
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_norm_inputs
    inp = make_norm_inputs(20, 1024, io_dtype="bf16", seed=9)
    y = torch.from_numpy(inp["y"]).to(torch.bfloat16).to(dev)
    z = torch.from_numpy(inp["z"]).to(torch.bfloat16).to(dev)
    w = torch.from_numpy(inp["weight"]).to(dev)
    libssd.ssd_gated_rmsnorm_fwd(y, z, w, out=y)
    torch.cuda.synchronize()
    check(y.float().cpu().numpy(), gated_rmsnorm(inp["y"], inp["z"], inp["weight"]), "bf16",
          "norm in place")


# ------------------------------------------------------ packed sequences

# (b, L, H, P, G, max sequence length, initial state, dt preprocessing);
# the head counts select the fused pass's three layouts (32, 64 and
# 128-column workgroups)
VARLEN = [
    # b, L, H, P, G, max sequence length, initial state, dt preprocessing, io, Q, N
    (2, 300, 4, 64, 1, 96, True, False, "bf16", 64, 128),
    (2, 333, 4, 64, 2, 8, True, False, "bf16", 64, 128),     # several starts per block
    (2, 200, 132, 64, 2, 70, True, False, "bf16", 64, 128),  # four-wave workgroups
    (2, 300, 66, 64, 1, 40, False, False, "bf16", 64, 128),  # two-wave workgroups
    (1, 257, 4, 64, 1, 96, True, True, "bf16", 64, 128),     # time-step preprocessing
    (2, 300, 4, 64, 1, 96, True, False, "f32", 64, 128),     # fp32: the split path
    (2, 333, 3, 32, 1, 8, True, True, "f32", 16, 64),        # starts in most 16-token chunks
    (2, 520, 4, 48, 2, 300, True, False, "f32", 256, 32),    # few starts, long chunks
    (1, 777, 2, 64, 1, 130, False, False, "bf16", 128, 96),  # dstate 96: the split path
]


def _varlen_check(oracle_mod, dev, inp, seq, dtp=False, io="bf16", Q=64):
    import torch
    from oracle.dt import process_dt
    from oracle.varlen import forward_varlen
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    t = to_torch(inp, io, dev)
    ts = torch.from_numpy(seq).to(dev)
    if dtp:
        y, fin = libssd.ssd_chunk_scan_fwd(t["x"], t["dt_raw"], t["A"], t["B"], t["C"], t["D"],
                                           t["initial_state"], chunk_len=Q, seq_idx=ts,
                                           dt_bias=t["dt_bias"], dt_softplus=True)
        dt_used = process_dt(inp["dt_raw"], inp["dt_bias"], True)
    else:
        y, fin = libssd.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                           t["initial_state"], chunk_len=Q, seq_idx=ts)
        dt_used = inp["dt"]
    torch.cuda.synchronize()
    yr, fr = forward_varlen(inp["x"], dt_used, inp["A"], inp["B"], inp["C"], inp["D"],
                            inp["initial_state"], seq)
    ya = fa = None
    if io == "f32":
        ia = abs_inputs(inp)
        ya, fa = forward_varlen(ia["x"], dt_used, inp["A"], ia["B"], ia["C"], ia["D"],
                                ia["initial_state"], seq)
    check(y.float().cpu().numpy(), yr, io, "varlen y", ya, tok_axis=1)
    check(fin.cpu().numpy(), fr, io, "varlen final", fa)
    # and every packed sequence on its own (a short one must not drown in the
    # norm of the others)
    from oracle.varlen import segments
    yg = y.float().cpu().numpy()
    for r in range(seq.shape[0]):
        for s0, s1 in segments(seq[r]):
            if io == "f32":
                e = metrics.componentwise_err(yg[r, s0:s1], yr[r, s0:s1], ya[r, s0:s1])
                assert e <= metrics.FP32_MAX_REL, (r, s0, e)
            else:
                e = metrics.normwise_err(yg[r, s0:s1], yr[r, s0:s1])
                assert e <= metrics.BF16_NORMWISE, (r, s0, e)


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: "b%d_L%d_H%d_P%d_G%d_max%d" % c[:6]
                         + ("_init" if c[6] else "") + ("_dtproc" if c[7] else "")
                         + "_%s_Q%d_N%d" % c[8:])
def test_varlen_packed_sequences(dev, oracle_mod, path, case):
    from state_space_sequence_amd.inputs import make_seq_idx
    b, L, H, P, G, mx, init, dtp, io, Q, N = case
    _say("varlen case %s path %s" % (case, path))
    inp = make_inputs(b, L, H, P, N, G, io_dtype=io, init_std=0.1 if init else 0.0,
                      seed=700 + L + H)
    skip_if_path_unsupported(inp, io, Q)
    seq = make_seq_idx(b, L, seed=800 + L, max_len=mx)
    _varlen_check(oracle_mod, dev, inp, seq, dtp, io, Q)


@pytest.mark.parametrize("Q", [64, 32, 16])
def test_varlen_placed_boundaries(dev, oracle_mod, path, Q):
    """Sequence starts at block starts (32, 64), a run of one-token sequences
    (100, 101, 102), at the last token, and none in the first block's tail;
    with 64-, 32- and 16-token chunks on the split path (starts at chunk
    starts, a chunk of one-token sequences)."""
    if path == "fused" and Q != 64:
        pytest.skip("the fused pass does not depend on the chunk length")
    L = 230
    inp = make_inputs(2, L, 4, 64, 128, 1, io_dtype="bf16", init_std=0.1, seed=61)
    seq = np.zeros((2, L), dtype=np.int32)
    for k, start in enumerate([32, 33, 64, 100, 101, 102, L - 1]):
        seq[:, start:] = k + 1
    seq[1, :] = np.minimum(seq[1], 3)      # row 1: starts at 32, 33 and 64 only
    _varlen_check(oracle_mod, dev, inp, seq, Q=Q)


@pytest.mark.parametrize("H", [4, 66, 132])
def test_varlen_through_decay_regimes(dev, oracle_mod, path, H):
    """Packed sequences on the decay-regime inputs: sequence starts inside
    weak-decay, rescaling and exact blocks, at block starts and at the last
    token, in the fused pass's three workgroup layouts; every sequence on its
    own against the per-sequence oracle."""
    inp = decay_regime_inputs("bf16", seed=93, H=H)
    L = inp["x"].shape[1]
    seq = np.zeros((2, L), dtype=np.int32)
    # row 0: weak (50), block start (64), rescale region (100, 150), block
    # start (192), exact region (300, 333, 350), the last token
    for k, start in enumerate([50, 64, 100, 150, 192, 230, 300, 333, 350, L - 1]):
        seq[0, start:] = k + 1
    # row 1: one start in the rescale region, one in the exact region
    seq[1, 150:] = 1
    seq[1, 300:] = 2
    _say("varlen decay regimes H=%d" % H)
    _varlen_check(oracle_mod, dev, inp, seq)


# ------------------------------------------ full-size checks of the layer steps

def test_causal_conv1d_full_size_sampled(dev):
    """The conv at the size bench.py times (the 2.7B layer's 5376 x | B | C
    channels, b4 L8192, width 4, SiLU), checked on sampled channels over
    every token, and the cache of all channels."""
    import torch
    from oracle.conv import causal_conv1d, conv_state_after
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_conv_inputs
    w = WORKLOADS["mamba2_2p7b"]
    D = w.nheads * w.headdim + 2 * w.ngroups * w.dstate
    inp = make_conv_inputs(w.batch, w.seqlen, D, 4, io_dtype="bf16", seed=w.seed)
    x = torch.from_numpy(inp["x"]).to(torch.bfloat16).to(dev)
    wt = torch.from_numpy(inp["weight"]).to(dev)
    bias = torch.from_numpy(inp["bias"]).to(dev)
    out, state = libssd.ssd_causal_conv1d_fwd(x, wt, bias, "silu")
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    ch = np.unique(np.concatenate([[0, 7, 8, D - 8, D - 1], rng.integers(0, D, 59)]))
    ref = causal_conv1d(inp["x"][:, :, ch], inp["weight"][ch], inp["bias"][ch], "silu")
    got = out[:, :, torch.from_numpy(ch).to(dev)].float().cpu().numpy()
    check(got, ref, "bf16", "conv full size (sampled channels)")
    np.testing.assert_array_equal(state.float().cpu().numpy(), conv_state_after(inp["x"], 4))


def test_gated_rmsnorm_full_size_sampled(dev):
    """The gated norm at the size bench.py times (32768 rows x 5120), on
    sampled rows."""
    import torch
    from oracle.norm import gated_rmsnorm
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_norm_inputs
    w = WORKLOADS["mamba2_2p7b"]
    rows, dim = w.batch * w.seqlen, w.nheads * w.headdim
    inp = make_norm_inputs(rows, dim, io_dtype="bf16", seed=w.seed)
    y = torch.from_numpy(inp["y"]).to(torch.bfloat16).to(dev)
    z = torch.from_numpy(inp["z"]).to(torch.bfloat16).to(dev)
    wt = torch.from_numpy(inp["weight"]).to(dev)
    out = libssd.ssd_gated_rmsnorm_fwd(y, z, wt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rs = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 254)]))
    ref = gated_rmsnorm(inp["y"][rs], inp["z"][rs], inp["weight"])
    got = out[torch.from_numpy(rs).to(dev)].float().cpu().numpy()
    check(got, ref, "bf16", "norm full size (sampled rows)")
    for i in range(len(rs)):
        assert metrics.normwise_err(got[i], ref[i]) <= metrics.BF16_NORMWISE, rs[i]


def test_varlen_full_size_every_slice(dev, oracle_mod):
    """The 2.7B-shape forward with packed sequences as bench.py times it,
    checked on every head of every row against the per-sequence oracle."""
    import torch
    from oracle.varlen import forward_varlen
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_seq_idx, to_torch
    w = WORKLOADS["mamba2_2p7b"]
    inp = workload_inputs(w)
    seq = make_seq_idx(w.batch, w.seqlen, seed=w.seed, max_len=2048)
    t = to_torch(inp, w.io_dtype, dev)
    y, fin = libssd.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                       t["initial_state"], chunk_len=w.chunk_len,
                                       seq_idx=torch.from_numpy(seq).to(dev))
    torch.cuda.synchronize()
    # every head of every row against the per-sequence oracle
    yr, fr = forward_varlen(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                            inp["initial_state"], seq)
    check_every_slice(y.float().cpu().numpy(), fin.cpu().numpy(), yr, fr, "bf16",
                      "varlen full size")


def test_dt_preprocessing_full_size_every_slice(dev, oracle_mod):
    """The 2.7B-shape forward on the raw time step (softplus(dt + dt_bias) in
    the kernels) as bench.py times it, checked on every (batch, head) slice
    against the oracle run on the processed time step."""
    import torch
    from oracle.dt import process_dt
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    w = WORKLOADS["mamba2_2p7b"]
    inp = workload_inputs(w)
    t = to_torch(inp, w.io_dtype, dev)
    _say("dt preprocessing full size %s" % w.name)
    y, fin = libssd.ssd_chunk_scan_fwd(t["x"], t["dt_raw"], t["A"], t["B"], t["C"], t["D"],
                                       t["initial_state"], chunk_len=w.chunk_len,
                                       dt_bias=t["dt_bias"], dt_softplus=True)
    torch.cuda.synchronize()
    dt_used = process_dt(inp["dt_raw"], inp["dt_bias"], True)
    yr, fr = oracle_mod.forward(*(dict(inp, dt=dt_used)[k] for k in FWD_ARGS))
    check_every_slice(y.float().cpu().numpy(), fin.cpu().numpy(), yr, fr, "bf16",
                      "dt_proc full size")


@pytest.mark.parametrize("io", ["bf16", "f32", "bf16_segmented"])
def test_forward_and_decode_replay_in_a_graph(dev, monkeypatch, io):
    """The library allocates nothing and sets no memory from the host, so a
    forward and a decode step can be captured in one HIP graph.  Each replay
    (after eager resets and synchronisations) equals the eager calls bit for
    bit.  bf16 runs the fused kernel, fp32 the split kernels, and the
    segmented fused forward forks its state-only pass onto the library's
    auxiliary stream and joins it back inside the capture."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    b, L, H, P, N, G, Q = 2, 1000, 8, 64, 128, 2, 256
    if io == "bf16_segmented":
        io = "bf16"
        monkeypatch.setenv("SSD_FORWARD_PATH", "fused")
        monkeypatch.setenv("SSD_FUSED_SEGMENTS", "4")
    inp = make_inputs(b, L, H, P, N, G, io_dtype=io, init_std=0.1, seed=31)
    t = to_torch(inp, io, dev)
    code = libssd.SSD_BF16 if io == "bf16" else libssd.SSD_F32
    y = torch.empty_like(t["x"])
    fin = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(libssd.ssd_chunk_scan_fwd_workspace_size(b, L, H, P, N, G, Q, code), 1),
                     dtype=torch.uint8, device=dev)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["initial_state"])
    kw = dict(chunk_len=Q, y=y, final_state=fin, workspace=ws)
    xd, dtd = t["x"][:, 0].contiguous(), t["dt"][:, 0].contiguous()
    Bd, Cd = t["B"][:, 0].contiguous(), t["C"][:, 0].contiguous()
    yd = torch.empty_like(xd)
    _say("graph replay case %s" % io)
    libssd.ssd_chunk_scan_fwd(*args, **kw)
    torch.cuda.synchronize()
    y_ref, fin_ref = y.clone(), fin.clone()
    state0 = fin_ref.clone()
    state = state0.clone()
    libssd.ssd_state_update(state, xd, dtd, t["A"], Bd, Cd, t["D"], y=yd)
    torch.cuda.synchronize()
    yd_ref, st_ref = yd.clone(), state.clone()

    state.copy_(state0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        libssd.ssd_chunk_scan_fwd(*args, **kw)
        libssd.ssd_state_update(state, xd, dtd, t["A"], Bd, Cd, t["D"], y=yd)
    for rep in range(3):
        y.zero_()
        fin.zero_()
        yd.zero_()
        state.copy_(state0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), rep
        assert torch.equal(fin, fin_ref), rep
        assert torch.equal(yd, yd_ref), rep
        assert torch.equal(state, st_ref), rep
    del graph


# ------------------------------------------------------ opt-in non-finite check

@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_nonfinite_check_forward(dev, monkeypatch, path, io):
    """With SSD_CHECK_FINITE set: clean inputs pass, a NaN in x, an infinity
    in dt or in the initial state, and an output that overflows each return
    SSD_ERR_NONFINITE; with the check off the same NaN goes through silently
    (the status is OK and y holds NaNs)."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    inp = make_inputs(2, 300, 4, 64, 128, 2, io_dtype=io, init_std=0.1, seed=51)
    skip_if_path_unsupported(inp, io, 64)
    t = to_torch(inp, io, dev)

    def run(**over):
        a = dict(t, **over)
        return libssd.ssd_chunk_scan_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"],
                                         a["initial_state"], chunk_len=64)

    monkeypatch.setenv("SSD_CHECK_FINITE", "1")
    y, fin = run()
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.isfinite(fin).all()
    xn = t["x"].clone()
    xn[1, 123, 2, 7] = float("nan")
    dtn = t["dt"].clone()
    dtn[0, 299, 3] = float("inf")
    sn = t["initial_state"].clone()
    sn[1, 0, 5, 100] = float("-inf")
    big = torch.full_like(t["x"], 3.0e38 if io == "f32" else 3.0e38)
    for what, over in (("x NaN", dict(x=xn)), ("dt inf", dict(dt=dtn)),
                       ("initial state -inf", dict(initial_state=sn)),
                       ("y overflow", dict(x=big))):
        with pytest.raises(libssd.SsdError) as ei:
            run(**over)
        assert ei.value.status == libssd.SSD_ERR_NONFINITE, what
        _say("  %s -> SSD_ERR_NONFINITE" % what)
    monkeypatch.setenv("SSD_CHECK_FINITE", "0")
    y, _ = run(x=xn)
    torch.cuda.synchronize()
    assert torch.isnan(y).any()


def test_nonfinite_check_decode_conv_norm(dev, monkeypatch):
    """The check on the decode step (a NaN in the cached state), the
    convolution (an infinity in x, misaligned by one element in the update)
    and the gated norm (a NaN in the gate)."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_conv_inputs, make_norm_inputs, to_torch
    monkeypatch.setenv("SSD_CHECK_FINITE", "1")
    inp = make_inputs(2, 1, 4, 64, 128, 1, io_dtype="bf16", init_std=0.1, seed=52)
    t = to_torch(inp, "bf16", dev)
    state = t["initial_state"].clone()
    args = (t["x"][:, 0].contiguous(), t["dt"][:, 0].contiguous(), t["A"],
            t["B"][:, 0].contiguous(), t["C"][:, 0].contiguous(), t["D"])
    libssd.ssd_state_update(state, *args)
    state[0, 3, 63, 127] = float("nan")
    with pytest.raises(libssd.SsdError) as ei:
        libssd.ssd_state_update(state, *args)
    assert ei.value.status == libssd.SSD_ERR_NONFINITE

    cin = make_conv_inputs(2, 40, 64, 4, io_dtype="bf16", seed=53, decode_steps=1)
    x = torch.from_numpy(cin["x"]).to(torch.bfloat16).to(dev)
    w = torch.from_numpy(cin["weight"]).to(dev)
    out, cs = libssd.ssd_causal_conv1d_fwd(x, w, None, "silu")
    x[1, 39, 63] = float("inf")
    with pytest.raises(libssd.SsdError) as ei:
        libssd.ssd_causal_conv1d_fwd(x, w, None, "silu")
    assert ei.value.status == libssd.SSD_ERR_NONFINITE
    # the update on 2-byte aligned operands: the odd first element checked on its own
    flat = torch.zeros(2 * 64 + 1, dtype=torch.bfloat16, device=dev)
    xd = flat[1:].view(2, 64)
    xd.copy_(torch.from_numpy(cin["x_dec"][0]).to(torch.bfloat16))
    libssd.ssd_causal_conv1d_update(cs, xd, w, None, "silu")
    xd[0, 0] = float("nan")
    with pytest.raises(libssd.SsdError) as ei:
        libssd.ssd_causal_conv1d_update(cs, xd, w, None, "silu")
    assert ei.value.status == libssd.SSD_ERR_NONFINITE

    nin = make_norm_inputs(8, 256, io_dtype="bf16", seed=54)
    y = torch.from_numpy(nin["y"]).to(torch.bfloat16).to(dev)
    z = torch.from_numpy(nin["z"]).to(torch.bfloat16).to(dev)
    wn = torch.from_numpy(nin["weight"]).to(dev)
    libssd.ssd_gated_rmsnorm_fwd(y, z, wn)
    z[7, 255] = float("nan")
    with pytest.raises(libssd.SsdError) as ei:
        libssd.ssd_gated_rmsnorm_fwd(y, z, wn)
    assert ei.value.status == libssd.SSD_ERR_NONFINITE
    torch.cuda.synchronize()


# ------------------------------------------------ output gate, per-channel D

# (b, L, H, P, N, G, Q, io, z, per-channel D, extra); the head counts select
# the fused pass's three workgroup layouts (32, 64, 128 columns)
GATED = [
    (2, 300, 4, 64, 128, 2, 64, "bf16", True, True, None),
    (2, 300, 4, 64, 128, 2, 64, "f32", True, True, None),
    (2, 333, 4, 64, 128, 1, 128, "bf16", True, False, None),
    (2, 333, 4, 64, 128, 1, 128, "f32", False, True, None),
    (2, 200, 132, 64, 128, 2, 64, "bf16", True, True, None),
    (2, 300, 66, 64, 128, 1, 64, "bf16", True, False, None),
    (2, 257, 3, 32, 64, 1, 64, "f32", True, True, None),
    (1, 257, 4, 64, 128, 1, 64, "bf16", True, True, "dtproc"),
    (2, 300, 4, 64, 128, 1, 64, "bf16", True, True, "varlen"),
    (2, 200, 132, 64, 128, 2, 64, "bf16", True, True, "varlen"),
    (2, 400, 4, 64, 128, 1, 64, "bf16", True, True, "decay"),
    (2, 400, 4, 64, 128, 1, 64, "f32", False, True, "decay"),
    (2, 400, 132, 64, 128, 1, 64, "bf16", False, True, "decay"),
    (2, 400, 66, 64, 128, 1, 64, "bf16", True, True, "decay"),
]


@pytest.mark.parametrize("case", GATED, ids=lambda c: "b%d_L%d_H%d_P%d_N%d_G%d_Q%d_%s" % c[:8]
                         + ("_z" if c[8] else "") + ("_Dhp" if c[9] else "")
                         + ("_" + c[10] if c[10] else ""))
def test_gate_and_per_channel_D(dev, oracle_mod, path, case):
    """y = (C h + D (*) x) silu(z) with D per head or per (head, column),
    against the gate oracle (oracle/gate.py): the gate alone, the per-column
    D alone and both, with the time-step preprocessing, with packed
    sequences (the fused pass), and through the exact and rescaled blocks of
    the decay-regime inputs (where a per-head D rides on the diagonal
    weights and a per-column one cannot)."""
    import torch
    from oracle.dt import process_dt
    from oracle.gate import forward_gated, forward_gated_abs, silu, skip
    from oracle.varlen import forward_varlen
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_gate_inputs, make_seq_idx, to_torch
    b, L, H, P, N, G, Q, io, use_z, dhp, extra = case
    _say("gate case %s path %s" % (case, path))
    if extra == "decay":
        inp = decay_regime_inputs(io, seed=95, H=H)
    else:
        inp = make_inputs(b, L, H, P, N, G, io_dtype=io, init_std=0.1, seed=900 + L + H)
    skip_if_path_unsupported(inp, io, Q)
    g = make_gate_inputs(b, L, H, P, io_dtype=io, seed=901 + L)
    z = g["z"] if use_z else None
    D = g["D_hp"] if dhp else inp["D"]
    t = to_torch(inp, io, dev)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    tz = None if z is None else torch.from_numpy(z).to(tdt).to(dev)
    tD = torch.from_numpy(D).to(dev)
    kw = dict(chunk_len=Q, z=tz)
    dt_used, dt_arg = inp["dt"], t["dt"]
    if extra == "dtproc":
        kw.update(dt_bias=t["dt_bias"], dt_softplus=True)
        dt_used, dt_arg = process_dt(inp["dt_raw"], inp["dt_bias"], True), t["dt_raw"]
    seq = None
    if extra == "varlen":
        seq = make_seq_idx(b, L, seed=902 + L, max_len=60)
        kw["seq_idx"] = torch.from_numpy(seq).to(dev)
    y, fin = libssd.ssd_chunk_scan_fwd(t["x"], dt_arg, t["A"], t["B"], t["C"], tD,
                                       t["initial_state"], **kw)
    torch.cuda.synchronize()
    args = (inp["x"], dt_used, inp["A"], inp["B"], inp["C"], D, z, inp["initial_state"])
    if seq is not None:
        core, fr = forward_varlen(inp["x"], dt_used, inp["A"], inp["B"], inp["C"], None,
                                  inp["initial_state"], seq)
        yr = core + skip(D, inp["x"])
        if z is not None:
            yr = yr * silu(z)
    else:
        yr, fr = forward_gated(*args)
    ya = forward_gated_abs(*args) if io == "f32" else None
    check(y.float().cpu().numpy(), yr, io, "gated y", ya, tok_axis=1)
    # the state is not gated: the plain bar on the final state
    _, _, _, fa = reference(oracle_mod, dict(inp, dt=dt_used)) if io == "f32" else (0, 0, 0, None)
    check(fin.cpu().numpy(), fr, io, "final_state", fa)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_gated_decode_every_element(dev, oracle_mod, io):
    """ssd_state_update with the gate and a per-column D, step by step,
    against the gate oracle's decode step."""
    import torch
    from oracle.gate import state_update_gated
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_gate_inputs, to_torch
    b, steps, H, P, N, G = 3, 5, 4, 64, 128, 2
    inp = make_inputs(b, steps, H, P, N, G, io_dtype=io, init_std=0.1, seed=81)
    t = to_torch(inp, io, dev)
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    Dhp = make_gate_inputs(b, 0, H, P, io_dtype=io, seed=82)["D_hp"]
    zs = [make_gate_inputs(b, 0, H, P, io_dtype=io, seed=83 + s)["z"] for s in range(steps)]
    tD = torch.from_numpy(Dhp).to(dev)
    state = t["initial_state"].clone()
    st_ref = inp["initial_state"].astype(np.float64)
    for s in range(steps):
        tz = torch.from_numpy(zs[s]).to(tdt).to(dev)
        y = libssd.ssd_state_update(state, t["x"][:, s].contiguous(), t["dt"][:, s].contiguous(),
                                    t["A"], t["B"][:, s].contiguous(), t["C"][:, s].contiguous(),
                                    tD, z=tz)
        torch.cuda.synchronize()
        st_ref, yr = state_update_gated(st_ref, inp["x"][:, s], inp["dt"][:, s], inp["A"],
                                        inp["B"][:, s], inp["C"][:, s], Dhp, zs[s])
        err = metrics.normwise_err(y.float().cpu().numpy(), yr)
        _say("  step %d gated y normwise %.3e" % (s, err))
        assert err <= (2e-5 if io == "f32" else metrics.BF16_NORMWISE)
    assert metrics.normwise_err(state.cpu().numpy(), st_ref) <= (2e-6 if io == "f32" else 2e-2)


def test_gated_full_size_every_slice(dev, oracle_mod):
    """The 2.7B-shape forward with the gate and a per-column D, on every
    (batch, head) slice."""
    import torch
    from oracle.gate import forward_gated
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_gate_inputs, to_torch
    w = WORKLOADS["mamba2_2p7b"]
    inp = workload_inputs(w)
    g = make_gate_inputs(w.batch, w.seqlen, w.nheads, w.headdim, io_dtype="bf16", seed=w.seed)
    t = to_torch(inp, "bf16", dev)
    y, fin = libssd.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"],
                                       torch.from_numpy(g["D_hp"]).to(dev), t["initial_state"],
                                       chunk_len=w.chunk_len,
                                       z=torch.from_numpy(g["z"]).to(torch.bfloat16).to(dev))
    torch.cuda.synchronize()
    yr, fr = forward_gated(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], g["D_hp"], g["z"],
                           inp["initial_state"])
    check_every_slice(y.float().cpu().numpy(), fin.cpu().numpy(), yr, fr, "bf16",
                      "gated full size")


# bf16 cases of the gate test (the fused pass is bf16) that cross the
# windows below: plain, gated, per-column D, two- and four-wave workgroups,
# packed sequences, the time-step preprocessing and the decay regimes
WINDOW_CASES = [c for i, c in enumerate(GATED) if i in (0, 2, 4, 5, 7, 8, 9, 10, 12)]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "b%d_L%d_H%d_Q%d" % (c[0], c[1], c[2], c[6])
                         + ("_z" if c[8] else "") + ("_Dhp" if c[9] else "")
                         + ("_" + c[10] if c[10] else ""))
def test_fused_resources_rebased_every_four_blocks(dev, oracle_mod, monkeypatch, case):
    """The fused pass's loader addresses each stream (x, B, C, dt, y, z,
    sequence labels) with 32-bit offsets from a buffer resource that it moves
    forward every window of blocks.  Forcing the window down to 4 blocks
    (128 tokens) makes these 200-400-token problems cross one to three window
    boundaries, with the prefetches three blocks ahead and the y stores one
    behind in different windows; every element against the oracle."""
    monkeypatch.setenv("SSD_FUSED_WINDOW_SHIFT", "2")
    monkeypatch.setenv("SSD_FORWARD_PATH", "fused")
    test_gate_and_per_channel_D(dev, oracle_mod, "fused", case)


def test_long_sequence_fused_sampled_heads(dev, oracle_mod, monkeypatch):
    """One 262,144-token sequence at the 2.7B layer shape (80 heads of 64
    columns, one group of 128 states, chunk 256, bf16, an initial state).
    A row of x is 2.7 GB, past what a 32-bit buffer offset reaches, so the
    fused pass's loader moves its resources forward three times along the
    row (every 2048 blocks).  Sixteen head slices, the first and last heads
    among them, against the serial oracle: every 32-token block of y and the
    final states."""
    import torch
    monkeypatch.setenv("SSD_FORWARD_PATH", "fused")
    L, H, P, N = 262144, 80, 64, 128
    _say("long sequence b1 L%d H%d: drawing inputs" % (L, H))
    inp = make_inputs(1, L, H, P, N, 1, io_dtype="bf16", init_std=0.1, seed=1239)
    assert L * H * P * 2 > 2 ** 31
    _say("  forward on the fused pass")
    y, fin = gpu_forward(inp, "bf16", 256, dev)
    rng = np.random.default_rng(1240)
    hs = sorted({0, 1, 39, 40, H - 2, H - 1} | set(int(v) for v in rng.choice(H, 10, replace=False)))
    while len(hs) < 16:
        hs = sorted(set(hs) | {int(rng.integers(H))})
    _say("  oracle on heads %s" % hs)
    yr, fr = oracle_mod.forward(inp["x"][:, :, hs], inp["dt"][:, :, hs], inp["A"][hs],
                                inp["B"], inp["C"], inp["D"][hs], inp["initial_state"][:, hs])
    yg = np.ascontiguousarray(y[:, :, hs])
    del y
    check(yg, yr, "bf16", "long y (16 heads)", tok_axis=1)
    check(fin[:, hs], fr, "bf16", "long final (16 heads)")
    # the last window's blocks and the tail on their own
    check(yg[:, -2048:], yr[:, -2048:], "bf16", "long y, last 2048 tokens", tok_axis=1)


@pytest.mark.parametrize("shift", [None, "2"], ids=["natural_window", "four_block_window"])
def test_fused_reads_and_writes_nothing_past_the_end(dev, oracle_mod, monkeypatch, shift):
    """A ragged one-row problem (300 tokens: 9 blocks and 12 tokens) whose
    inputs x, dt, B, C, z and the sequence labels are each the head of a
    buffer 256 tokens longer, the rest NaN (labels: a new sequence on every
    token), and whose y is the head of one whose rest holds a sentinel.  The
    fused pass's loader prefetches up to three blocks past the last one and
    stores the last block whole: the resources' ranges must turn those rows
    into zeros and dropped stores.  A NaN read would reach the final state;
    a stray store would change the sentinel."""
    import torch
    from oracle.gate import silu, skip
    from oracle.varlen import forward_varlen
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_gate_inputs, make_seq_idx, to_torch
    monkeypatch.setenv("SSD_FORWARD_PATH", "fused")
    if shift:
        monkeypatch.setenv("SSD_FUSED_WINDOW_SHIFT", shift)
    L, H, P, N, pad = 300, 4, 64, 128, 256
    inp = make_inputs(1, L, H, P, N, 1, io_dtype="bf16", init_std=0.1, seed=1301)
    g = make_gate_inputs(1, L, H, P, io_dtype="bf16", seed=1302)
    seq = make_seq_idx(1, L, seed=1303, max_len=90)
    t = to_torch(inp, "bf16", dev)

    def guarded(v, fill):
        full = torch.full((v.shape[0], L + pad) + tuple(v.shape[2:]), fill, dtype=v.dtype,
                          device=dev)
        full[:, :L] = v
        view = full[:, :L]
        assert view.is_contiguous()
        return full, view

    _, xv = guarded(t["x"], float("nan"))
    _, dtv = guarded(t["dt"], float("nan"))
    _, bv = guarded(t["B"], float("nan"))
    _, cv = guarded(t["C"], float("nan"))
    _, zv = guarded(torch.from_numpy(g["z"]).to(torch.bfloat16).to(dev), float("nan"))
    sfull = torch.arange(L + pad, dtype=torch.int32, device=dev)[None] + 1000
    sfull[:, :L] = torch.from_numpy(seq).to(dev)
    sv = sfull[:, :L]
    yfull = torch.full((1, L + pad, H, P), 7.0, dtype=torch.bfloat16, device=dev)
    y, fin = libssd.ssd_chunk_scan_fwd(xv, dtv, t["A"], bv, cv, t["D"], t["initial_state"],
                                       chunk_len=64, y=yfull[:, :L], seq_idx=sv, z=zv)
    torch.cuda.synchronize()
    assert y.data_ptr() == yfull.data_ptr()
    assert bool((yfull[:, L:] == 7.0).all()), "a store landed past the end of y"
    core, fr = forward_varlen(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], None,
                              inp["initial_state"], seq)
    yr = (core + skip(inp["D"], inp["x"])) * silu(g["z"])
    check(y.float().cpu().numpy(), yr, "bf16", "guarded y", tok_axis=1)
    check(fin.cpu().numpy(), fr, "bf16", "guarded final state")


# ------------------------------------------ the segmented fused forward

SEGMENTED = [
    # b, L, H, G, init, segments
    (2, 1000, 4, 1, True, 4),      # 32 blocks: 8 per segment
    (2, 1000, 4, 2, False, 7),     # uneven: 5 blocks per segment, the last 2
    (1, 777, 6, 3, True, 3),       # ragged tail in the last segment
    (2, 300, 132, 2, True, 2),     # four-wave workgroups, two heads of a group each
]


@pytest.mark.parametrize("seg0_pct", [30, 80, 150])
@pytest.mark.parametrize("case", SEGMENTED, ids=lambda c: "b%d_L%d_H%d_G%d%s_seg%d" % (
    c[0], c[1], c[2], c[3], "_init" if c[4] else "", c[5]))
def test_fused_segments_every_element(dev, oracle_mod, monkeypatch, case, seg0_pct):
    """The fused forward with the sequence cut into segments (the main pass
    over segment 0 beside the state-only pass over segments 1 .. n - 2, then
    the main pass over the rest, chaining the segments' states), forced onto
    small problems with segment 0 at 30%, 80% and 150% of the others' length:
    every element of y and the final state against the oracle."""
    b, L, H, G, init, nseg = case
    monkeypatch.setenv("SSD_FORWARD_PATH", "fused")
    monkeypatch.setenv("SSD_FUSED_SEGMENTS", str(nseg))
    monkeypatch.setenv("SSD_FUSED_SEG0_PCT", str(seg0_pct))
    _say("segmented case %s" % (case,))
    inp = make_inputs(b, L, H, 64, 128, G, io_dtype="bf16", init_std=0.1 if init else 0.0,
                      seed=1400 + L + H)
    y, fin = gpu_forward(inp, "bf16", 64, dev)
    yr, fr, _, _ = reference(oracle_mod, inp, want_abs=False)
    check(y, yr, "bf16", "segmented y", tok_axis=1)
    check(fin, fr, "bf16", "segmented final")


SEGMENTED_GATED = [c for i, c in enumerate(GATED) if i in (0, 4, 7, 8, 9, 10, 12, 13)]


@pytest.mark.parametrize("nseg", [2, 3])
@pytest.mark.parametrize("case", SEGMENTED_GATED, ids=lambda c: "b%d_L%d_H%d" % (c[0], c[1], c[2])
                         + ("_z" if c[8] else "") + ("_Dhp" if c[9] else "")
                         + ("_" + c[10] if c[10] else ""))
def test_fused_segments_with_every_option(dev, oracle_mod, monkeypatch, case, nseg):
    """Segments with the gate, per-column D, the time-step preprocessing,
    packed sequences (a start in one segment cuts the decay of the state
    handed on) and the decay regimes (rescaled and exact blocks on either
    side of a segment boundary)."""
    monkeypatch.setenv("SSD_FUSED_SEGMENTS", str(nseg))
    monkeypatch.setenv("SSD_FORWARD_PATH", "fused")
    test_gate_and_per_channel_D(dev, oracle_mod, "fused", case)


@pytest.mark.parametrize("nseg", [2, 4])
def test_fused_segments_sequence_starts_at_boundaries(dev, oracle_mod, monkeypatch, nseg):
    """Packed sequences whose starts fall on a segment's first token, on its
    last token, and a segment with no start between two with starts."""
    monkeypatch.setenv("SSD_FUSED_SEGMENTS", str(nseg))
    monkeypatch.setenv("SSD_FORWARD_PATH", "fused")
    L = 1024                       # 32 blocks: segments of 16 (nseg 2) or 8 blocks
    seg_tokens = L // nseg
    inp = make_inputs(2, L, 4, 64, 128, 1, io_dtype="bf16", init_std=0.1, seed=1501)
    seq = np.zeros((2, L), dtype=np.int32)
    starts = [seg_tokens, 2 * seg_tokens - 1, seg_tokens + 5] if nseg == 2 else \
        [seg_tokens, 2 * seg_tokens - 1, 3 * seg_tokens + 17]
    for k, st in enumerate(sorted(starts)):
        seq[0, st:] = k + 1
    seq[1, seg_tokens:] = 1          # row 1: one start, at the first segment boundary
    _say("segments %d, starts %s" % (nseg, sorted(starts)))
    _varlen_check(oracle_mod, dev, inp, seq)


def test_fused_segments_timed_names_two_kernels(dev, monkeypatch):
    """The timed forward of a segmented problem names its two phases (the
    first runs two kernels on two streams) and matches the untimed one bit
    for bit."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    monkeypatch.setenv("SSD_FORWARD_PATH", "fused")
    monkeypatch.setenv("SSD_FUSED_SEGMENTS", "3")
    inp = make_inputs(2, 1000, 4, 64, 128, 1, io_dtype="bf16", init_std=0.1, seed=1502)
    t = to_torch(inp, "bf16", dev)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["initial_state"])
    y0, f0 = libssd.ssd_chunk_scan_fwd(*args, chunk_len=64)
    import bench
    ev = bench.HipEvents()
    evs = [ev.create() for _ in range(libssd.max_kernels() + 1)]
    y1, f1, names = libssd.ssd_chunk_scan_fwd_timed(evs, *args, chunk_len=64)
    torch.cuda.synchronize()
    for e in evs:
        ev.destroy(e)
    _say("kernels %s" % names)
    assert names == ["k_fused_ssd_state+seg0", "k_fused_ssd"]
    assert torch.equal(y0, y1) and torch.equal(f0, f1)


# ------------------------------------------ the NaN-poisoned workspace

POISON = [
    # path, io, b, L, H, P, N, G, Q, segments (fused), packed sequences
    ("split", "f32", 2, 777, 4, 64, 128, 2, 128, 0, False),
    ("split", "f32", 2, 333, 3, 32, 64, 1, 16, 0, True),
    ("split", "bf16", 2, 520, 4, 48, 32, 2, 256, 0, False),
    ("split", "bf16", 1, 300, 66, 64, 128, 1, 64, 0, True),
    ("fused", "bf16", 2, 1000, 4, 64, 128, 2, 64, 4, False),
    ("fused", "bf16", 2, 1000, 4, 64, 128, 1, 64, 3, True),
]


@pytest.mark.parametrize("case", POISON, ids=lambda c: "%s_%s_b%d_L%d_H%d_P%d_N%d_G%d_Q%d_seg%d" % (
    c[:10]) + ("_varlen" if c[10] else ""))
def test_workspace_poisoned_with_nan(dev, oracle_mod, monkeypatch, case):
    """SSD_POISON_WORKSPACE fills the workspace with NaN before the call:
    every intermediate a kernel reads must have been written by an earlier
    kernel of the same call (with the non-finite check on, the call must
    return SSD_OK), and the result is unchanged bit for bit."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_seq_idx, to_torch
    path, io, b, L, H, P, N, G, Q, nseg, varlen = case
    monkeypatch.setenv("SSD_FORWARD_PATH", path)
    if nseg:
        monkeypatch.setenv("SSD_FUSED_SEGMENTS", str(nseg))
    inp = make_inputs(b, L, H, P, N, G, io_dtype=io, init_std=0.1, seed=1600 + L)
    t = to_torch(inp, io, dev)
    kw = dict(chunk_len=Q)
    if varlen:
        kw["seq_idx"] = torch.from_numpy(make_seq_idx(b, L, seed=1601, max_len=50)).to(dev)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["initial_state"])
    y0, f0 = libssd.ssd_chunk_scan_fwd(*args, **kw)
    monkeypatch.setenv("SSD_POISON_WORKSPACE", "1")
    monkeypatch.setenv("SSD_CHECK_FINITE", "1")
    need = libssd.ssd_chunk_scan_fwd_workspace_size(b, L, H, P, N, G, Q,
                                                    libssd.SSD_BF16 if io == "bf16" else libssd.SSD_F32)
    assert need > 0
    y1, f1 = libssd.ssd_chunk_scan_fwd(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
