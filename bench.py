"""Benchmark of the libssd chunked SSD forward on one MI355X.

One step = one ``ssd_chunk_scan_fwd`` over the Mamba-2 2.7B-shape SSD layer
(batch 4, seqlen 8192, 80 heads, headdim 64, d_state 128, 1 group, chunk 256;
bf16 x/B/C, fp32 dt/A/D/state), every kernel of the chunked algorithm, on
synthetic seeded inputs already resident in HBM: `warmup` untimed calls,
then exactly `steps` calls with HIP events on the launch stream between them
(the host time of one call, ``host_dispatch_ms``, about 17 us, is reported on
its own; the forward takes far longer on the GPU, so the queue never drains).
Calls shorter than their host time (the tiny forward, the conv update) are
timed as replays of a HIP graph holding many of them.  Prints one JSON line.

Also reported (not part of ``value``):
  * ``measured_peaks``: a 1 GiB device copy and an 8192^3 bf16 GEMM, the
    measured counterparts of the spec peaks (run first; they also bring the
    clocks to a steady state);
  * per-kernel GPU time from HIP events recorded between the kernels of each
    call (``ssd_chunk_scan_fwd_timed`` on the same stream);
  * ``roofline`` for the dominant kernel and ``path_roofline`` for the whole
    call against algorithmic bytes (x, B, C, dt, A, D read once; y and the
    final state written once; no intermediates);
  * the other workloads, timed before the headline: the tiny fp32, 130M and
    8-group forwards, the decode state update (b256 / 80 heads), the
    headline forward on the raw time step with the preprocessing (bias,
    softplus) inside the kernels, with packed variable-length sequences, and
    with the output gate and a per-column D,
    the causal depthwise conv before the scan and its single-token update,
    and the gated RMS normalisation after it;
  * ``per_workload``: for each of the five workloads, tokens/s, TFLOP/s, GB/s
    and the roofline fractions against the spec and the measured peaks, next
    to the oracle's tokens/s on the host cores;
  * ``cpu_baseline``: the fp64 serial oracle on the host cores over a bounded
    sample of (batch, head) slices of the headline workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # fp32 MFMA / vector
METRIC = "SSD fwd tokens/sec per layer + achieved TFLOP/s & HBM GB/s vs MI355X peak"


# ------------------------------------------------------------------ HIP events

class HipEvents:
    """Minimal ctypes access to hipEvent_* of the HIP runtime torch loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventCreate.restype = ctypes.c_int
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventRecord.restype = ctypes.c_int
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventSynchronize.restype = ctypes.c_int
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.restype = ctypes.c_int
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.restype = ctypes.c_int
        self.lib.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                            ctypes.c_int, ctypes.c_void_p]
        self.lib.hipMemcpyAsync.restype = ctypes.c_int

    def memcpy_d2d(self, dst, src, nbytes, stream_handle):
        # hipMemcpyDeviceToDevice = 3
        rc = self.lib.hipMemcpyAsync(ctypes.c_void_p(dst), ctypes.c_void_p(src),
                                     ctypes.c_size_t(nbytes), 3, ctypes.c_void_p(stream_handle))
        if rc != 0:
            raise RuntimeError("hipMemcpyAsync failed (%d)" % rc)

    def create(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError("hipEventCreate failed (%d)" % rc)
        return e.value

    def record(self, e, stream_handle):
        rc = self.lib.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream_handle))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def ms(self, a, b):
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a),
                                          ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return float(out.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))


# ------------------------------------------------------------------ accounting

def alg_bytes_forward(w, es):
    """Algorithmic HBM bytes of one forward: inputs read once, outputs once."""
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    x = b * L * H * P * es
    bc = 2 * b * L * G * N * es
    dt = b * L * H * 4
    small = 2 * H * 4
    init = b * H * P * N * 4 if w.init_std > 0 else 0
    final = b * H * P * N * 4
    y = b * L * H * P * es
    return x + bc + dt + small + init + final + y


def alg_flops_forward(w):
    """Flops of the chunked SSD forward (the pages' four steps), with each
    causal triangle counted once: the C B^T blocks (Q(Q+1)/2 entries of N
    products per chunk and group), the chunk states (P Q N per chunk and
    head), the output (the off-diagonal P Q N and the diagonal Q(Q+1)/2 P per
    chunk and head) and the passing of the states (P N per chunk and head),
    two flops per multiply-add.  The serial recurrence's 4 P N per token and
    head, and the dense L x L quadratic form, are not counted."""
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len
    nc = -(-L // Q)
    cb = 2 * (Q * (Q + 1) // 2) * N * b * nc * G
    state = 2 * P * Q * N * b * nc * H
    out = (2 * Q * N * P + Q * (Q + 1) * P) * b * nc * H
    passing = 2 * P * N * b * nc * H
    return cb + state + out + passing


def kernel_alg_bytes(name, w, es):
    """Algorithmic bytes of one launch of a kernel.

    k_fused_ssd performs the whole SSD forward except the prefix sums and
    the C B^T diagonal blocks, so its algorithmic bytes are those of the
    forward itself (inputs read once, outputs written once).  The helper
    kernels and the five kernels of the split path count what each must
    read and write given its own inputs and outputs.  (A segmented fused
    forward's two passes are taken together, as the forward.)"""
    b, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len
    if name == "k_fused_ssd":
        return alg_bytes_forward(w, es)
    if name == "k1_dA_cumsum":
        # dt in; prefix hi, lo and dt per chunk out (the padded chunk length)
        return b * L * H * 4 + 3 * b * H * (-(-L // Q)) * Q * 4
    nc = -(-L // Q)
    per_chunk_vec = b * H * nc * Q * 4          # acum or dtT
    states = b * nc * H * P * N * 4
    ntl = Q // 16
    cb = b * nc * G * (ntl * (ntl + 1) // 2) * 256 * 4
    x = b * L * H * P * es
    bc1 = b * L * G * N * es
    if name == "k2_chunk_cb":
        return 2 * bc1 + cb
    if name == "k3_chunk_state":
        return x + bc1 + 2 * per_chunk_vec + states
    if name == "k4_state_passing":
        init = b * H * P * N * 4 if w.init_std > 0 else 0
        return 2 * states + b * H * nc * 4 + init + b * H * P * N * 4
    if name == "k5_chunk_scan":
        return x + bc1 + cb + states + 2 * per_chunk_vec + x
    return None


# ------------------------------------------------------------------ runs

def time_graph(fn, ev, reps, warmup=0, per_graph=1, dist=None):
    """GPU time of one call of ``fn``, in ms: ``per_graph`` calls captured in
    one HIP graph (torch.cuda.CUDAGraph), ``warmup`` untimed replays, then
    ``reps`` replays between a pair of HIP events on the replay stream, with a
    device synchronisation on both sides.  A call from Python costs the host
    about as much time as the forward costs the GPU, so timing plain calls
    would measure the host; the replays time the kernels."""
    import torch
    fn()                       # eager once: the library validates, nothing is cached
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            fn()
    for _ in range(warmup):
        graph.replay()
    sh = torch.cuda.current_stream().cuda_stream
    # an event before every replay and after the last: the whole region and
    # the spread of single replays from the same run
    evs = [ev.create() for _ in range(reps + 1)]
    torch.cuda.synchronize()
    for k in range(reps):
        ev.record(evs[k], sh)
        graph.replay()
    ev.record(evs[reps], sh)
    torch.cuda.synchronize()
    ms = ev.ms(evs[0], evs[reps]) / (reps * per_graph)
    if dist is not None:
        one = sorted(ev.ms(evs[k], evs[k + 1]) / per_graph for k in range(reps))
        for q, f in (("min", 0.0), ("p10", 0.1), ("p50", 0.5), ("p90", 0.9), ("max", 1.0)):
            dist[q] = one[min(len(one) - 1, int(round(f * (len(one) - 1))))]
    for e in evs:
        ev.destroy(e)
    del graph
    return ms


def time_plain(fn, ev, reps, warmup=0, dist=None, warm_ms=40.0):
    """GPU time of one call of ``fn``, in ms: ``warmup`` untimed calls (after
    ``warm_ms`` of calls that bring the clocks up, when warmup > 0), a
    device synchronisation, then exactly ``reps`` calls with a HIP event on
    the launch stream before each and after the last, and a synchronisation.
    For calls whose GPU time exceeds their host time (tens of microseconds
    here) the queue never drains, so the region holds the kernels back to
    back.  (A HIP graph holding a single forward costs about 10 us more per
    replay than a plain call on this runtime, so graphs are kept for calls
    shorter than their host time, several calls per graph.)"""
    if warmup > 0 and warm_ms > 0:
        warm(fn, warm_ms)
    import torch
    for _ in range(warmup):
        fn()
    sh = torch.cuda.current_stream().cuda_stream
    evs = [ev.create() for _ in range(reps + 1)]
    torch.cuda.synchronize()
    for k in range(reps):
        ev.record(evs[k], sh)
        fn()
    ev.record(evs[reps], sh)
    torch.cuda.synchronize()
    ms = ev.ms(evs[0], evs[reps]) / reps
    if dist is not None:
        one = sorted(ev.ms(evs[k], evs[k + 1]) for k in range(reps))
        for q, f in (("min", 0.0), ("p10", 0.1), ("p50", 0.5), ("p90", 0.9), ("max", 1.0)):
            dist[q] = one[min(len(one) - 1, int(round(f * (len(one) - 1))))]
    for e in evs:
        ev.destroy(e)
    return ms


def warm(fn, ms=40.0):
    """Calls ``fn`` back to back for at least ``ms`` of wall time: after the
    seconds it takes to draw a workload's inputs the GPU clocks have dropped,
    and a few warmup calls of a sub-millisecond forward do not bring them
    back up."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def host_dispatch_ms(fn, n=50):
    """Host wall time of one plain call (argument checks, ctypes, launch), in
    ms, measured on calls that queue behind each other on the stream."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    return (t1 - t0) * 1e3 / n


def setup(w, dev):
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch, workload_inputs
    inp = workload_inputs(w)
    t = to_torch(inp, w.io_dtype, dev)
    y = torch.empty_like(t["x"])
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32,
                      device=dev)
    io = libssd.SSD_BF16 if w.io_dtype == "bf16" else libssd.SSD_F32
    need = libssd.ssd_chunk_scan_fwd_workspace_size(w.batch, w.seqlen, w.nheads, w.headdim,
                                                    w.dstate, w.ngroups, w.chunk_len, io)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    return inp, t, y, fin, ws


def per_kernel_split(call_timed, ev, steps):
    """Per-kernel GPU time (ms) from ``ssd_chunk_scan_fwd_timed``: HIP events
    recorded on the launch stream between the kernels of each call."""
    import torch
    from state_space_sequence_amd import libssd
    nev = libssd.max_kernels() + 1
    events = [[ev.create() for _ in range(nev)] for _ in range(steps)]
    names = None
    for k in range(steps):
        names = call_timed(events[k])
    torch.cuda.synchronize()
    nk = len(names)
    per_kernel = [sum(ev.ms(events[k][i], events[k][i + 1]) for k in range(steps)) / steps
                  for i in range(nk)]
    for row in events:
        for e in row:
            ev.destroy(e)
    return dict(zip(names, per_kernel))


def time_forward(w, dev, steps, warmup, ev, per_graph=1, prepared=None, warm_ms=40.0):
    """The forward of workload ``w``: ms per call (exactly ``steps`` timed
    calls after ``warmup``; plain calls, or with ``per_graph`` > 1 replays of
    a graph holding that many calls), the spread of single calls, the
    per-kernel split, and the host time of a plain call.  ``prepared`` is the
    result of setup() when the inputs were made beforehand."""
    from state_space_sequence_amd import libssd
    inp, t, y, fin, ws = prepared if prepared is not None else setup(w, dev)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["initial_state"])
    kw = dict(chunk_len=w.chunk_len, y=y, final_state=fin, workspace=ws)

    def call():
        libssd.ssd_chunk_scan_fwd(*args, **kw)

    def call_timed(events):
        return libssd.ssd_chunk_scan_fwd_timed(events, *args, **kw)[2]

    dist = {}
    if per_graph > 1:
        gpu_ms = time_graph(call, ev, steps, warmup, per_graph, dist)
    else:
        gpu_ms = time_plain(call, ev, steps, warmup, dist, warm_ms)
    split = per_kernel_split(call_timed, ev, min(steps, 50))
    host_ms = host_dispatch_ms(call)
    del t, y, fin, ws
    return dict(gpu_ms=gpu_ms, per_kernel_ms=split, host_dispatch_ms=host_ms, inputs=inp,
                dist=dist)


def time_forward_varlen(w, dev, ev, steps=100, warmup=20, max_len=2048):
    """ms per forward with each row packed with sequences of lengths drawn
    from 1 .. max_len (ssd_chunk_scan_fwd_varlen), from graph replays."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_seq_idx
    inp, t, y, fin, ws = setup(w, dev)
    seq = make_seq_idx(w.batch, w.seqlen, seed=w.seed, max_len=max_len)
    nseq = int(sum(len(set(r.tolist())) for r in seq))
    ts = torch.from_numpy(seq).to(dev)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["initial_state"])
    kw = dict(chunk_len=w.chunk_len, y=y, final_state=fin, workspace=ws, seq_idx=ts)
    ms = time_plain(lambda: libssd.ssd_chunk_scan_fwd(*args, **kw), ev, steps, warmup)
    del t, y, fin, ws
    return ms, nseq


def time_forward_dt_proc(w, dev, ev, steps=100, warmup=20):
    """ms per forward with the time-step preprocessing inside the kernels:
    the raw dt with the per-head bias and softplus, limits (0, inf), as the
    Mamba-2 layer calls the scan (ssd_chunk_scan_fwd_ex), from graph replays."""
    from state_space_sequence_amd import libssd
    inp, t, y, fin, ws = setup(w, dev)
    args = (t["x"], t["dt_raw"], t["A"], t["B"], t["C"], t["D"], t["initial_state"])
    kw = dict(chunk_len=w.chunk_len, y=y, final_state=fin, workspace=ws,
              dt_bias=t["dt_bias"], dt_softplus=True)
    ms = time_plain(lambda: libssd.ssd_chunk_scan_fwd(*args, **kw), ev, steps, warmup)
    del t, y, fin, ws
    return ms


def time_forward_gated(w, dev, ev, steps=100, warmup=20):
    """ms per forward with the output gate and a per-(head, column) D, y =
    (C h + D (*) x) silu(z) (ssd_chunk_scan_fwd_full)."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_gate_inputs
    inp, t, y, fin, ws = setup(w, dev)
    g = make_gate_inputs(w.batch, w.seqlen, w.nheads, w.headdim, io_dtype=w.io_dtype,
                         seed=w.seed)
    tdt = torch.bfloat16 if w.io_dtype == "bf16" else torch.float32
    z = torch.from_numpy(g["z"]).to(tdt).to(dev)
    Dhp = torch.from_numpy(g["D_hp"]).to(dev)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], Dhp, t["initial_state"])
    kw = dict(chunk_len=w.chunk_len, y=y, final_state=fin, workspace=ws, z=z)
    ms = time_plain(lambda: libssd.ssd_chunk_scan_fwd(*args, **kw), ev, steps, warmup)
    del t, y, fin, ws, z
    return ms


def alg_flops_backward(w):
    """Dense-product FLOPs of one gradient pass as the kernels form it, per
    (batch, chunk, head): the adjoint chunk product G_c and the recomputed
    chunk state (2 QPN each), u's state and causal parts (2 QNP + Q(Q+1)P),
    and dB's and dC's state parts, causal scores and causal products (2 QPN +
    Q(Q+1)P + Q(Q+1)N each); plus the recomputed C B^T, Q(Q+1)N per (batch,
    chunk, group).  Causal blocks count their lower triangle."""
    Q, P, N = w.chunk_len, w.headdim, w.dstate
    nc = -(-w.seqlen // Q)
    per_head = 10 * Q * P * N + 3 * Q * (Q + 1) * P + 2 * Q * (Q + 1) * N
    return w.batch * nc * (w.nheads * per_head + w.ngroups * Q * (Q + 1) * N)


def time_backward(w, dev, ev, steps=10, warmup=2):
    """ms per gradient pass (ssd_chunk_scan_bwd) on this workload with seeded
    dy and dfinal, its kernels' times (per-kernel events, separate calls),
    and its dense-product rate against the MFMA peak of its operand type."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_grad_inputs
    inp, t, y, fin, ws = setup(w, dev)
    del y, fin, ws
    g = make_grad_inputs(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.io_dtype,
                         seed=w.seed + 1)
    tdt = torch.bfloat16 if w.io_dtype == "bf16" else torch.float32
    dy = torch.from_numpy(g["dy"]).to(tdt).to(dev)
    dfin = torch.from_numpy(g["dfinal"]).to(dev)
    args = (t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["initial_state"], dy, dfin)
    io = libssd.SSD_BF16 if w.io_dtype == "bf16" else libssd.SSD_F32
    wsb = torch.empty(libssd.ssd_chunk_scan_bwd_workspace_size(
        w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len, io),
        dtype=torch.uint8, device=dev)
    out = libssd.ssd_chunk_scan_bwd(*args, chunk_len=w.chunk_len, workspace=wsb)
    ms = time_plain(lambda: libssd.ssd_chunk_scan_bwd(*args, chunk_len=w.chunk_len, out=out,
                                                      workspace=wsb), ev, steps, warmup)
    evs = [ev.create() for _ in range(libssd.bwd_max_kernels() + 1)]
    per = {}
    for _ in range(max(1, steps // 2)):
        o = libssd.ssd_chunk_scan_bwd(*args, chunk_len=w.chunk_len, out=out, workspace=wsb,
                                      events=evs)
        torch.cuda.synchronize()
        for i, n in enumerate(o["kernel_names"]):
            per.setdefault(n, []).append(ev.ms(evs[i], evs[i + 1]))
    for e in evs:
        ev.destroy(e)
    flops = alg_flops_backward(w)
    peak = BF16_PEAK_TFLOPS if w.io_dtype == "bf16" else FP32_PEAK_TFLOPS
    tf = flops / (ms * 1e-3) / 1e12
    del t, dy, dfin, wsb, out
    return {"what": "gradients of (y, final_state) with respect to every input "
                    "(ssd_chunk_scan_bwd, recomputing the forward's chunk states)",
            "ms_per_step": round(ms, 4),
            "tokens_per_s": round(w.batch * w.seqlen / (ms * 1e-3), 1),
            "alg_flops": flops, "tflops": round(tf, 2),
            "frac_mfma": round(tf / peak, 4),
            "per_kernel_ms": {k: round(sum(v) / len(v), 4) for k, v in per.items()}}


def time_conv(w, dev, ev, steps=50, warmup=10, decode_batch=256):
    """The causal depthwise conv that precedes the scan, on this layer's
    x | B | C channels (dim = H P + 2 G N, width 4, SiLU, bias): the
    sequence forward and the single-token update at batch decode_batch,
    each against the HBM roofline of its algorithmic bytes (graph replays)."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_conv_inputs
    D, W = w.nheads * w.headdim + 2 * w.ngroups * w.dstate, 4
    es = 2 if w.io_dtype == "bf16" else 4
    tdt = torch.bfloat16 if w.io_dtype == "bf16" else torch.float32
    inp = make_conv_inputs(w.batch, w.seqlen, D, W, io_dtype=w.io_dtype, seed=w.seed)
    x = torch.from_numpy(inp["x"]).to(tdt).to(dev)
    wt = torch.from_numpy(inp["weight"]).to(dev)
    bias = torch.from_numpy(inp["bias"]).to(dev)
    out = torch.empty_like(x)
    state = torch.empty((w.batch, D, W), dtype=tdt, device=dev)
    ms = time_plain(lambda: libssd.ssd_causal_conv1d_fwd(x, wt, bias, "silu", out=out,
                                                         conv_state=state), ev, steps, warmup)
    alg = 2 * w.batch * w.seqlen * D * es + D * (W + 1) * 4 + w.batch * D * W * es
    gbs = alg / (ms * 1e-3) / 1e9
    res = {"workload": "causal conv1d b%d L%d dim %d width %d, SiLU, %s"
                       % (w.batch, w.seqlen, D, W, w.io_dtype),
           "ms_per_step": round(ms, 4),
           "tokens_per_s": round(w.batch * w.seqlen / (ms * 1e-3), 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "alg_bytes_per_launch": alg}}
    bd = decode_batch
    cs = torch.zeros((bd, D, W), dtype=tdt, device=dev)
    xd = torch.randn((bd, D), device=dev).to(tdt)
    od = torch.empty_like(xd)
    per_graph, reps = 50, 8
    msd = time_graph(lambda: libssd.ssd_causal_conv1d_update(cs, xd, wt, bias, "silu", out=od),
                     ev, reps, 1, per_graph)
    # the replays ran: after W or more updates with the same token, every
    # slot of the cache holds it
    if not torch.equal(cs, xd[:, :, None].expand(bd, D, W)):
        raise RuntimeError("conv update graph replays did not update the cache")
    algd = 2 * bd * D * W * es + 2 * bd * D * es + D * (W + 1) * 4
    gbd = algd / (msd * 1e-3) / 1e9
    res_d = {"workload": "causal conv1d update b%d dim %d width %d, SiLU, %s"
                         % (bd, D, W, w.io_dtype),
             "us_per_step": round(msd * 1e3, 2),
             "timing": "%d updates captured in one graph, %d replays" % (per_graph, reps),
             "roofline": {"bound": "hbm", "achieved": round(gbd, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(gbd / HBM_PEAK_GBS, 4),
                          "alg_bytes_per_launch": algd}}
    del x, out, state, cs, xd, od
    return res, res_d


def time_norm(w, dev, ev, steps=50, warmup=10):
    """The gated RMS normalisation after the scan on this layer's output
    (rows = b L, dim = H P, gate before the norm, eps 1e-5), against the HBM
    roofline of its algorithmic bytes (y and z read, out written once)."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_norm_inputs
    rows, dim = w.batch * w.seqlen, w.nheads * w.headdim
    es = 2 if w.io_dtype == "bf16" else 4
    tdt = torch.bfloat16 if w.io_dtype == "bf16" else torch.float32
    inp = make_norm_inputs(rows, dim, io_dtype=w.io_dtype, seed=w.seed)
    y = torch.from_numpy(inp["y"]).to(tdt).to(dev)
    z = torch.from_numpy(inp["z"]).to(tdt).to(dev)
    wt = torch.from_numpy(inp["weight"]).to(dev)
    out = torch.empty_like(y)
    ms = time_plain(lambda: libssd.ssd_gated_rmsnorm_fwd(y, z, wt, out=out), ev, steps, warmup)
    alg = 3 * rows * dim * es + dim * 4
    gbs = alg / (ms * 1e-3) / 1e9
    del y, z, out
    return {"workload": "gated RMSNorm rows %d dim %d, %s" % (rows, dim, w.io_dtype),
            "ms_per_step": round(ms, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "alg_bytes_per_launch": alg}}


def decode_alg_bytes(w):
    es = 2 if w.io_dtype == "bf16" else 4
    b, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    return 2 * b * H * P * N * 4 + b * H * P * es * 2 + 2 * b * G * N * es + b * H * 4 + 2 * H * 4


def decode_alg_flops(w):
    """Per step and (batch, head): the state decay and update (3 P N) and
    the output product (2 P N), plus D x (2 P)."""
    b, H, P, N = w.batch, w.nheads, w.headdim, w.dstate
    return b * H * (5 * P * N + 2 * P)


def time_decode(w, dev, ev, reps=3):
    """The decode workload's steps of ssd_state_update, all captured in one
    graph (one step per captured call), timed from replays."""
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import make_inputs, to_torch
    inp = make_inputs(w.batch, w.decode_steps, w.nheads, w.headdim, w.dstate, w.ngroups,
                      io_dtype=w.io_dtype, init_std=w.init_std, seed=w.seed)
    t = to_torch(inp, w.io_dtype, dev)
    xs = [t["x"][:, s].contiguous() for s in range(w.decode_steps)]
    dts = [t["dt"][:, s].contiguous() for s in range(w.decode_steps)]
    Bs = [t["B"][:, s].contiguous() for s in range(w.decode_steps)]
    Cs = [t["C"][:, s].contiguous() for s in range(w.decode_steps)]
    state = t["initial_state"].clone()
    ys = [torch.empty_like(xs[0]) for _ in range(w.decode_steps)]
    step = [0]

    def one():
        s = step[0] % w.decode_steps
        step[0] += 1
        libssd.ssd_state_update(state, xs[s], dts[s], t["A"], Bs[s], Cs[s], t["D"], y=ys[s])

    ms = time_plain(one, ev, reps * w.decode_steps, w.decode_steps)
    alg = decode_alg_bytes(w)
    gbs = alg / (ms * 1e-3) / 1e9
    b, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    return {"workload": "decode b%d H%d P%d N%d G%d, %d steps, fp32 state, %s x/B/C"
                        % (b, H, P, N, G, w.decode_steps, w.io_dtype),
            "us_per_step": round(ms * 1e3, 2),
            "ms_per_step": round(ms, 5),
            "tokens_per_s": round(b / (ms * 1e-3), 1),
            "timing": "%d passes over the %d steps, plain calls" % (reps, w.decode_steps),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "alg_bytes_per_launch": alg}}


def measure_peaks(dev, ev):
    """Measured counterparts of the spec peaks: a device-to-device copy of
    1 GiB (torch's copy kernel; read + write bytes) and a 8192^3 bf16 GEMM
    (torch.matmul, hipBLASLt).  These also bring the clocks to their steady
    state before the timed workloads."""
    import torch
    n = 1 << 30
    copies = {}
    sh = torch.cuda.current_stream().cuda_stream
    for dt_ in (torch.float32, torch.int64):
        src = torch.empty(n // torch.tensor([], dtype=dt_).element_size(), dtype=dt_,
                          device=dev).fill_(1)
        dst = torch.empty_like(src)
        copies["torch copy_ " + str(dt_).split(".")[-1]] = time_plain(lambda: dst.copy_(src),
                                                                      ev, 10, 2)
        if dt_ == torch.int64:
            copies["hipMemcpyAsync"] = time_plain(
                lambda: ev.memcpy_d2d(dst.data_ptr(), src.data_ptr(), n, sh), ev, 10, 2)
        del src, dst
    best = min(copies, key=copies.get)
    ms_copy = copies[best]
    m = 8192
    a = torch.randn((m, m), device=dev, dtype=torch.bfloat16)
    bm = torch.randn((m, m), device=dev, dtype=torch.bfloat16)
    c = torch.empty((m, m), device=dev, dtype=torch.bfloat16)
    sh = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        torch.matmul(a, bm, out=c)
    e0, e1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    ev.record(e0, sh)
    reps = 20
    for _ in range(reps):
        torch.matmul(a, bm, out=c)
    ev.record(e1, sh)
    torch.cuda.synchronize()
    ms_mm = ev.ms(e0, e1) / reps
    ev.destroy(e0)
    ev.destroy(e1)
    del a, bm, c
    return {"copy_gbs": round(2 * n / (ms_copy * 1e-3) / 1e9, 1),
            "copy_what": "device-to-device copy of 1 GiB (read + write bytes), the fastest of "
                         + ", ".join("%s %.1f GB/s" % (k, 2 * n / (v * 1e-3) / 1e9)
                                     for k, v in copies.items()),
            "bf16_gemm_tflops": round(2 * m ** 3 / (ms_mm * 1e-3) / 1e12, 1),
            "gemm_what": "8192 x 8192 x 8192 bf16 torch.matmul (hipBLASLt)"}


def _cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, inp, target_s=12.0):
    """The fp64 serial oracle on the host cores, on a bounded sample of the
    workload's (batch, head) slices over the full sequence; tokens/s scaled to
    the whole workload by the fraction of slices computed."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    threads = oracle.max_threads()
    nsl = w.batch * w.nheads
    order = [(b, h) for b in range(w.batch) for h in range(w.nheads)]

    def run(k):
        sl = order[:k]
        t0 = time.perf_counter()
        # slices are independent: one call per batch row keeps the arrays whole
        done = 0
        for b in sorted({s[0] for s in sl}):
            hs = [h for bb, h in sl if bb == b]
            x = inp["x"][b:b + 1][:, :, hs]
            dt = inp["dt"][b:b + 1][:, :, hs]
            g = np.array(hs) // (w.nheads // w.ngroups)
            if w.ngroups == 1:
                Bm, Cm = inp["B"][b:b + 1], inp["C"][b:b + 1]
                init = None if inp["initial_state"] is None else inp["initial_state"][b:b + 1][:, hs]
                oracle.forward(x, dt, inp["A"][hs], Bm, Cm, inp["D"][hs], init)
            else:
                oracle.forward_slices(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                                      inp["D"], inp["initial_state"], w.ngroups,
                                      [(b, h) for h in hs])
            done += len(hs)
            del g
        return time.perf_counter() - t0, done

    cal_k = min(nsl, max(4, threads))
    t_cal, _ = run(cal_k)
    per_slice = t_cal / cal_k
    k = int(min(nsl, max(cal_k, target_s / max(per_slice, 1e-9))))
    if k > cal_k:
        t_run, k = run(k)
    else:
        t_run, k = t_cal, cal_k
    # a workload that the oracle finishes in well under the target time is
    # run whole several times and the time averaged
    reps = 1
    if k == nsl and t_run < 0.2 * target_s:
        reps = int(min(1000, max(1, 0.2 * target_s / max(t_run, 1e-6))))
        t0 = time.perf_counter()
        for _ in range(reps):
            run(k)
        t_run = (time.perf_counter() - t0) / reps
    tokens_equiv = w.batch * w.seqlen * (k / nsl)
    return {"value": round(tokens_equiv / t_run, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": _cpu_model(),
            "sample": "%d of %d (batch, head) slices, all %d tokens each, fp64 serial "
                      "recurrence (C, OpenMP over slices), %.3g s per pass%s; tokens/s scaled by "
                      "the slice fraction" % (k, nsl, w.seqlen, t_run,
                                              " (mean of %d passes)" % reps if reps > 1 else "")}


COPY_CAL_BYTES = 256 << 20


def _code_only(text):
    """C++ source with comments removed and whitespace collapsed (string
    literals in these files hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(read=None):
    """sha256 of the code (comments and layout aside) of the kernel sources
    the fused path is built from; a stored traffic measurement is reported
    only while it matches."""
    import hashlib
    hsh = hashlib.sha256()
    for name in ("ssd_fused_kernels.hip", "ssd_device.hpp", "ssd_kernels.hpp"):
        path = os.path.join("state_space_sequence_amd", "csrc", name)
        if read is None:
            with open(os.path.join(ROOT, path)) as f:
                text = f.read()
        else:
            text = read(path)
        hsh.update(_code_only(text).encode())
    return hsh.hexdigest()


def describe(w):
    if w.decode_steps:
        return "decode b%d H%d P%d N%d G%d, %d steps, fp32 state, %s x/B/C" % (
            w.batch, w.nheads, w.headdim, w.dstate, w.ngroups, w.decode_steps, w.io_dtype)
    return "b%d L%d H%d P%d N%d G%d Q%d, %s x/B/C%s" % (
        w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len, w.io_dtype,
        ", initial state" if w.init_std > 0 else "")


def config_row(w, ms, peaks, oracle_rate):
    """One row of the per-workload table: GPU rate and roofline fractions
    against the spec and the measured peaks, next to the oracle's rate."""
    es = 2 if w.io_dtype == "bf16" else 4
    if w.decode_steps:
        tokens, flops, abytes = w.batch, decode_alg_flops(w), decode_alg_bytes(w)
    else:
        tokens, flops, abytes = w.batch * w.seqlen, alg_flops_forward(w), alg_bytes_forward(w, es)
    gbs = abytes / (ms * 1e-3) / 1e9
    tfl = flops / (ms * 1e-3) / 1e12
    mfma_peak = BF16_PEAK_TFLOPS if w.io_dtype == "bf16" else FP32_PEAK_TFLOPS
    t_hbm, t_mfma = abytes / (HBM_PEAK_GBS * 1e9), flops / (mfma_peak * 1e12)
    row = {"workload": describe(w), "gpu_ms": round(ms, 5),
           "tokens_per_s": round(tokens / (ms * 1e-3), 1),
           "tflops": round(tfl, 2), "gbs": round(gbs, 1),
           "bound": "hbm" if t_hbm >= t_mfma else "mfma",
           "roofline_us": round(max(t_hbm, t_mfma) * 1e6, 2),
           "frac_hbm_spec": round(gbs / HBM_PEAK_GBS, 4),
           "frac_hbm_measured": round(gbs / peaks["copy_gbs"], 4),
           "frac_mfma_spec": round(tfl / mfma_peak, 4),
           "frac_mfma_measured": (round(tfl / peaks["bf16_gemm_tflops"], 4)
                                  if w.io_dtype == "bf16" else None),
           "alg_bytes": abytes, "alg_flops": flops}
    if oracle_rate is not None:
        row["oracle_tokens_per_s"] = oracle_rate["value"]
        row["oracle_cores"] = oracle_rate["cores"]
        row["gpu_over_oracle"] = round(row["tokens_per_s"] / oracle_rate["value"], 1)
    return row


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mamba2_2p7b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra-steps", type=int, default=100,
                    help="timed calls per other workload (counter runs use a few)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads and the decode timing")
    ap.add_argument("--backward-only", action="store_true",
                    help="of the other workloads, time only the gradient passes "
                         "(for kernel traces and counters of the backward)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM traffic per launch of the dominant kernel "
                         "(from rocprofv3 FETCH_SIZE/WRITE_SIZE runs), if present")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one device-to-device copy of 256 MiB, the known-size "
                         "kernel the FETCH_SIZE / WRITE_SIZE counters are scaled by")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: libssd has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import WORKLOADS, make_inputs
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    libssd.load()
    dev = torch.device("cuda:0")
    ev = HipEvents()

    w = WORKLOADS[args.workload]
    es = 2 if w.io_dtype == "bf16" else 4
    if args.copy_calibration:
        src = torch.empty(COPY_CAL_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # the headline's inputs are made first (drawing them keeps the host busy
    # for seconds, long enough for the GPU clocks to drop), then the measured
    # peaks (their copy and GEMM loops also bring the clocks to a steady
    # state), the other workloads, and the timed headline right after them
    prepared = setup(w, dev)
    peaks = measure_peaks(dev, ev)
    extra, fwd_ms = {}, {}
    if not args.no_extra and not args.backward_only:
        for name in ("tiny_f32", "mamba2_130m", "mamba2_130m_f32", "grouped_g8"):
            wx = WORKLOADS[name]
            # the tiny forward takes microseconds: 50 per captured graph
            reps, per_graph = ((max(1, args.extra_steps // 5), 50) if name == "tiny_f32"
                               else (args.extra_steps, 1))
            rx = time_forward(wx, dev, reps, 5, ev, per_graph)
            fwd_ms[name] = rx["gpu_ms"]
            esx = 2 if wx.io_dtype == "bf16" else 4
            gb = alg_bytes_forward(wx, esx) / (rx["gpu_ms"] * 1e-3) / 1e9
            extra[name] = {"ms_per_step": round(rx["gpu_ms"], 5),
                           "tokens_per_s": round(wx.batch * wx.seqlen / (rx["gpu_ms"] * 1e-3), 1),
                           "path_frac_hbm": round(gb / HBM_PEAK_GBS, 4),
                           "per_kernel_ms": {k: round(v, 4) for k, v in rx["per_kernel_ms"].items()},
                           "host_dispatch_ms": round(rx["host_dispatch_ms"], 4)}
            del rx
        extra["decode_b256"] = time_decode(WORKLOADS["decode_b256"], dev, ev,
                                           reps=max(1, min(3, args.extra_steps // 30)))
        fwd_ms["decode_b256"] = extra["decode_b256"]["ms_per_step"]
        xs = args.extra_steps
        msd = time_forward_dt_proc(w, dev, ev, steps=xs, warmup=min(20, xs))
        extra[w.name + "_dt_proc"] = {
            "what": "the same forward on the raw time step: softplus(dt + dt_bias) in the kernels",
            "ms_per_step": round(msd, 4),
            "tokens_per_s": round(w.batch * w.seqlen / (msd * 1e-3), 1)}
        msv, nseq = time_forward_varlen(w, dev, ev, steps=xs, warmup=min(20, xs))
        extra[w.name + "_varlen"] = {
            "what": "the same forward with %d packed sequences (lengths 1..2048) in its %d rows"
                    % (nseq, w.batch),
            "ms_per_step": round(msv, 4),
            "tokens_per_s": round(w.batch * w.seqlen / (msv * 1e-3), 1)}
        msg = time_forward_gated(w, dev, ev, steps=xs, warmup=min(20, xs))
        extra[w.name + "_gated"] = {
            "what": "the same forward with the output gate and a per-(head, column) D: "
                    "y = (C h + D x) silu(z), z read like x",
            "ms_per_step": round(msg, 4),
            "tokens_per_s": round(w.batch * w.seqlen / (msg * 1e-3), 1),
            "alg_bytes": alg_bytes_forward(w, es) + w.batch * w.seqlen * w.nheads * w.headdim * es,
            "frac_hbm": round((alg_bytes_forward(w, es) + w.batch * w.seqlen * w.nheads * w.headdim
                               * es) / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        extra["conv1d_" + w.name], extra["conv1d_update_b256"] = time_conv(
            w, dev, ev, steps=max(1, xs // 2), warmup=min(10, xs))
        extra["gated_rmsnorm_" + w.name] = time_norm(w, dev, ev, steps=max(1, xs // 2),
                                                     warmup=min(10, xs))
    if not args.no_extra:
        xs = args.extra_steps
        for name in ("mamba2_130m", "mamba2_130m_f32", w.name):
            extra["backward_" + name] = time_backward(WORKLOADS[name], dev, ev,
                                                      steps=max(2, min(10, xs // 10)),
                                                      warmup=min(2, xs))

    # the headline: exactly `steps` timed graph replays of one forward each
    # (exactly `warmup` untimed calls: the other workloads and the measured
    # peaks have just brought the clocks up)
    r = time_forward(w, dev, args.steps, args.warmup, ev, prepared=prepared, warm_ms=0.0)
    del prepared
    ms_step = r["gpu_ms"]
    fwd_ms[w.name] = ms_step
    tokens = w.batch * w.seqlen
    value = tokens / (ms_step * 1e-3)
    flops = alg_flops_forward(w)
    abytes = alg_bytes_forward(w, es)
    per = r["per_kernel_ms"]
    dom = max(per, key=per.get)
    # one kernel per forward: its average launch is the timed replays' time
    dom_ms = ms_step if len(per) == 1 else per[dom]
    dom_bytes = kernel_alg_bytes(dom, w, es)
    if "k_fused_ssd_state" in per:
        # a segmented fused forward: its two passes together do the
        # forward's work, so the roofline is taken over both
        dom = "k_fused_ssd_state + k_fused_ssd"
        dom_ms = sum(per.values())
        dom_bytes = alg_bytes_forward(w, es)
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            # counters taken on this kernel, this workload, this source only
            if (tj.get("kernel") == dom and tj.get("workload") == w.name
                    and tj.get("source_sha256") == kernel_source_hash()):
                traffic = tj.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None
    path_gbs = abytes / (ms_step * 1e-3) / 1e9
    path_tflops = flops / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.io_dtype == "bf16" else "f32",
        "data": "synthetic (seeded; distributions of the Mamba-2 layer initialisation)",
        "config": {"workload": "Mamba-2 2.7B-shape SSD layer forward" if w.name == "mamba2_2p7b"
                   else w.name,
                   "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk_len": w.chunk_len, "io_dtype": w.io_dtype,
                   "state_dtype": "f32", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "alg_bytes_per_launch": dom_bytes, "avg_launch_ms": round(dom_ms, 4),
                     "measured_peak": peaks["copy_gbs"],
                     "frac_measured_peak": round(dom_gbs / peaks["copy_gbs"], 4)},
        "path_roofline": {"bound": "hbm", "alg_bytes": abytes, "alg_flops": flops,
                          "achieved_gbs": round(path_gbs, 1),
                          "achieved_tflops": round(path_tflops, 2),
                          "frac_hbm": round(path_gbs / HBM_PEAK_GBS, 4),
                          "frac_mfma_bf16": round(path_tflops / BF16_PEAK_TFLOPS, 4),
                          "roofline_us": round(max(abytes / (HBM_PEAK_GBS * 1e9),
                                                   flops / (BF16_PEAK_TFLOPS * 1e12)) * 1e6, 2)},
        "timing": "exactly `steps` plain calls after `warmup`, a HIP event on the launch "
                  "stream before each and after the last; the host time of a call "
                  "(host_dispatch_ms) is a small fraction of the forward, so the queue never "
                  "drains",
        "step_ms_dist": {k: round(v, 4) for k, v in r["dist"].items()},
        "per_kernel_ms": {k: round(v, 4) for k, v in per.items()},
        "host_dispatch_ms": round(r["host_dispatch_ms"], 4),
        "measured_peaks": peaks,
    }
    if extra:
        out["other_workloads"] = extra
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, r["inputs"])
    # per-workload table (every workload timed in this run)
    table = {}
    for name in ("tiny_f32", "mamba2_130m", "mamba2_130m_f32", "mamba2_2p7b", "grouped_g8",
                 "decode_b256"):
        if name not in fwd_ms:
            continue
        wx = WORKLOADS[name]
        rate = None
        if not args.no_cpu_baseline:
            if name == w.name:
                rate = out["cpu_baseline"]
            else:
                if wx.decode_steps:
                    inp = make_inputs(wx.batch, wx.decode_steps, wx.nheads, wx.headdim, wx.dstate,
                                      wx.ngroups, io_dtype=wx.io_dtype, init_std=wx.init_std,
                                      seed=wx.seed)
                else:
                    from state_space_sequence_amd.inputs import workload_inputs
                    inp = workload_inputs(wx)
                rate = cpu_baseline(wx, inp, target_s=3.0)
        table[name] = config_row(wx, fwd_ms[name], peaks, rate)
    out["per_workload"] = table
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
