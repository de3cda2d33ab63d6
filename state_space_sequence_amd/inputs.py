"""Seeded synthetic inputs for the SSD forward and the decode state update.

This module draws random numbers and nothing else: it holds none of the
SSD arithmetic, so both the HIP path (through the tests and the benchmark)
and the fp64 oracle can consume what it produces without sharing code.

Distributions (one reading of the Mamba-2 layer's initialisation in fla
``modeling_mamba2.py``, ``Mamba2PreTrainedModel._init_weights``, which draws a
time step log-uniformly in [time_step_min, time_step_max] = [1e-3, 1e-1] and
stores its inverse softplus as ``dt_bias``; A is the negative exponential of a
log-uniform draw, as ``A = -exp(A_log)``):

    A_h       = -exp(U(0, ln 16))                         fp32 [H]
    dt_bias_h = u + log(-expm1(-u)),  u = exp(U(ln 1e-3, ln 1e-1))
    D_h       ~ U(0, 1)                                   fp32 [H]
    x         ~ N(0, 1)                                   [b,L,H,P]
    dt        = softplus(0.5 * N(0, 1) + dt_bias_h)       fp32 [b,L,H]
    B, C      ~ N(0, 1)                                   [b,L,G,N]
    init      = 0, or N(0, 0.1^2)                         fp32 [b,H,P,N]

Draw order: A, dt_bias, D, x, dt-noise, B, C, init, from
``numpy.random.Generator(PCG64(seed))``.  x, B and C are rounded to bf16
(round to nearest even) when the workload is bf16; every array is returned
as float32 holding exactly the values the GPU receives.

The same draw also yields the layer's raw time step, for callers that let
the library apply the time-step preprocessing itself:

    dt_raw    = 0.5 * N(0, 1)  (the same noise)            fp32 [b,L,H]
    dt_bias   = dt_bias_h                                  fp32 [H]
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_len: int
    io_dtype: str            # 'f32' or 'bf16' for x, B, C and y
    init_std: float = 0.0    # 0 -> zero initial state
    seed: int = 1234
    decode_steps: int = 0    # >0: a decode workload of that many tokens
    notes: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


# The workloads.  Shapes of the "130M" and "2.7B" entries are the SSD
# layer shapes of those Mamba-2 sizes (d_inner = 2 * d_model, headdim 64,
# d_state 128); no weights are involved.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 128, 2, 16, 16, 1, 32, "f32", seed=1234),
    "mamba2_130m": Workload("mamba2_130m", 8, 2048, 24, 64, 128, 1, 256, "bf16",
                            seed=1235),
    "mamba2_2p7b": Workload("mamba2_2p7b", 4, 8192, 80, 64, 128, 1, 256, "bf16",
                            seed=1236),
    "grouped_g8": Workload("grouped_g8", 2, 16380, 64, 64, 128, 8, 256, "bf16",
                           init_std=0.1, seed=1237),
    "decode_b256": Workload("decode_b256", 256, 64, 80, 64, 128, 1, 256, "bf16",
                            init_std=0.1, seed=1238, decode_steps=64),
    # the 130M layer shape with fp32 x, B, C and y (the split path)
    "mamba2_130m_f32": Workload("mamba2_130m_f32", 8, 2048, 24, 64, 128, 1, 256, "f32",
                                seed=1239),
}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), returned as
    float32.  Finite inputs only."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _softplus(v):
    # log(1 + e^v) without overflow for large v
    return np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))


def make_inputs(batch, seqlen, nheads, headdim, dstate, ngroups,
                io_dtype="bf16", init_std=0.0, seed=1234):
    """Draw one problem.  Returns a dict of float32 numpy arrays
    x, dt, A, B, C, D, initial_state (None when init_std == 0), and the raw
    time step dt_raw with its per-head bias dt_bias."""
    rng = np.random.Generator(np.random.PCG64(seed))
    H, P, N, G = nheads, headdim, dstate, ngroups
    A = -np.exp(rng.uniform(0.0, np.log(16.0), size=H))
    u = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=H))
    dt_bias = u + np.log(-np.expm1(-u))
    D = rng.uniform(0.0, 1.0, size=H)
    x = rng.standard_normal(size=(batch, seqlen, H, P), dtype=np.float32)
    noise = rng.standard_normal(size=(batch, seqlen, H), dtype=np.float32)
    dt = _softplus(0.5 * noise.astype(np.float64) + dt_bias[None, None, :])
    Bm = rng.standard_normal(size=(batch, seqlen, G, N), dtype=np.float32)
    Cm = rng.standard_normal(size=(batch, seqlen, G, N), dtype=np.float32)
    init = None
    if init_std > 0:
        init = (init_std * rng.standard_normal(size=(batch, H, P, N),
                                               dtype=np.float32)).astype(np.float32)
    if io_dtype == "bf16":
        x, Bm, Cm = round_to_bf16(x), round_to_bf16(Bm), round_to_bf16(Cm)
    elif io_dtype != "f32":
        raise ValueError("io_dtype must be 'f32' or 'bf16'")
    return {
        "x": np.ascontiguousarray(x, dtype=np.float32),
        "dt": dt.astype(np.float32),
        "A": A.astype(np.float32),
        "B": np.ascontiguousarray(Bm, dtype=np.float32),
        "C": np.ascontiguousarray(Cm, dtype=np.float32),
        "D": D.astype(np.float32),
        "initial_state": init,
        "dt_raw": (0.5 * noise.astype(np.float64)).astype(np.float32),
        "dt_bias": dt_bias.astype(np.float32),
    }


def workload_inputs(w: Workload, seqlen: int | None = None, batch: int | None = None):
    """Inputs for a named workload, optionally with a shorter sequence or
    batch (same seed and distributions)."""
    return make_inputs(batch or w.batch, seqlen or w.seqlen, w.nheads, w.headdim,
                       w.dstate, w.ngroups, w.io_dtype, w.init_std, w.seed)


def to_torch(inp: dict, io_dtype: str, device):
    """Move a ``make_inputs`` dict to torch tensors on ``device``: x, B, C in
    ``io_dtype``, everything else float32."""
    import torch
    tdt = torch.bfloat16 if io_dtype == "bf16" else torch.float32
    out = {}
    for k, v in inp.items():
        if v is None:
            out[k] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k in ("x", "B", "C"):
            t = t.to(tdt)
        out[k] = t.to(device).contiguous()
    return out


def make_conv_inputs(batch, seqlen, dim, width, io_dtype="bf16", seed=1234, decode_steps=0):
    """Inputs of the causal depthwise convolution before the scan.

    x ~ N(0, 1) [batch, seqlen, dim] (the projected x | B | C channels),
    rounded to bf16 for a bf16 problem; weight [dim, width] and bias [dim]
    ~ U(-1/sqrt(width), 1/sqrt(width)), the default initialisation of a
    depthwise ``nn.Conv1d`` (fan-in = width); fp32.  With decode_steps > 0,
    also x_dec [decode_steps, batch, dim], the tokens that follow.  Draw
    order: weight, bias, x, x_dec."""
    rng = np.random.Generator(np.random.PCG64(seed))
    bound = 1.0 / np.sqrt(width)
    w = rng.uniform(-bound, bound, size=(dim, width)).astype(np.float32)
    bias = rng.uniform(-bound, bound, size=dim).astype(np.float32)
    x = rng.standard_normal(size=(batch, seqlen, dim), dtype=np.float32)
    xd = rng.standard_normal(size=(decode_steps, batch, dim), dtype=np.float32)
    if io_dtype == "bf16":
        x, xd = round_to_bf16(x), round_to_bf16(xd)
    elif io_dtype != "f32":
        raise ValueError("io_dtype must be 'f32' or 'bf16'")
    return {"x": np.ascontiguousarray(x), "weight": w, "bias": bias,
            "x_dec": np.ascontiguousarray(xd)}


def make_norm_inputs(rows, dim, io_dtype="bf16", seed=1234):
    """Inputs of the gated RMS normalisation after the scan: y, z ~ N(0, 1)
    [rows, dim] (the scan output and the gate channels), rounded to bf16 for
    a bf16 problem; weight [dim] fp32 = 1 + 0.1 N(0, 1) (the module starts at
    ones; a spread exercises the per-channel scale).  Draw order: y, z,
    weight."""
    rng = np.random.Generator(np.random.PCG64(seed))
    y = rng.standard_normal(size=(rows, dim), dtype=np.float32)
    z = rng.standard_normal(size=(rows, dim), dtype=np.float32)
    w = (1.0 + 0.1 * rng.standard_normal(size=dim)).astype(np.float32)
    if io_dtype == "bf16":
        y, z = round_to_bf16(y), round_to_bf16(z)
    elif io_dtype != "f32":
        raise ValueError("io_dtype must be 'f32' or 'bf16'")
    return {"y": np.ascontiguousarray(y), "z": np.ascontiguousarray(z), "weight": w}


def make_grad_inputs(batch, seqlen, nheads, headdim, dstate, io_dtype="bf16", seed=0):
    """The gradients a backward call receives: dy ~ N(0, 1) [b, L, H, P]
    (rounded to bf16 for a bf16 problem) and dfinal ~ N(0, 1) [b, H, P, N]
    fp32, drawn in that order from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dy = rng.standard_normal(size=(batch, seqlen, nheads, headdim), dtype=np.float32)
    dfin = rng.standard_normal(size=(batch, nheads, headdim, dstate), dtype=np.float32)
    if io_dtype == "bf16":
        dy = round_to_bf16(dy)
    elif io_dtype != "f32":
        raise ValueError("io_dtype must be 'f32' or 'bf16'")
    return {"dy": np.ascontiguousarray(dy), "dfinal": dfin}


def make_seq_idx(batch, seqlen, seed=1234, max_len=96):
    """Packed-sequence labels [batch, seqlen] int32: each row is cut into
    sequences of lengths drawn uniformly from 1 .. max_len, labelled 0, 1, 2,
    ... in order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.zeros((batch, seqlen), dtype=np.int32)
    for r in range(batch):
        t, k = 0, 0
        while t < seqlen:
            n = int(rng.integers(1, max_len + 1))
            out[r, t:t + n] = k
            t, k = t + n, k + 1
    return out


def make_gate_inputs(batch, seqlen, nheads, headdim, io_dtype="bf16", seed=0):
    """The output gate z ~ N(0, 1) ([b, L, H, P], rounded to the I/O dtype;
    seqlen 0 gives the decode shape [b, H, P]) and a per-(head, column) D ~
    U(0, 1) ([H, P] fp32), drawn in that order from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (batch, nheads, headdim) if seqlen == 0 else (batch, seqlen, nheads, headdim)
    z = rng.standard_normal(size=shape).astype(np.float32)
    if io_dtype == "bf16":
        z = round_to_bf16(z)
    Dhp = rng.uniform(0.0, 1.0, size=(nheads, headdim)).astype(np.float32)
    return {"z": z, "D_hp": Dhp}
