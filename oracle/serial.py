"""ctypes front end of the C serial-recurrence oracle (``ssd_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The recurrence (per batch b, head h, group g = h // (H/G)):
    alpha_t = exp(dt_t * A_h)
    S_t     = alpha_t * S_{t-1} + dt_t * x_t^T (outer) B_t        (P x N)
    y_t     = S_t C_t + D_h * x_t
This is the "mamba" discretisation of the lrnnx ``selective_scan_ref``
sequential loop with a per-head scalar A, and the single-token branch of
fla ``Mamba2.torch_forward`` run once per token.  Everything is fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libssd_oracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile ``ssd_oracle.c`` into ``_build/libssd_oracle.so`` with gcc.

    ``-ffp-contract=off`` keeps every multiply and add a separately rounded
    double operation (no fused multiply-add), so the oracle is the plain
    definition evaluated in IEEE double.
    """
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-std=c99", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            path = build(force=False)
            lib = ctypes.CDLL(path)
            lib.ssd_oracle_forward.restype = ctypes.c_int
            lib.ssd_oracle_forward.argtypes = [ctypes.c_int] * 6 + [_dp] * 9 + [ctypes.c_int]
            lib.ssd_oracle_backward.restype = ctypes.c_int
            lib.ssd_oracle_backward.argtypes = [ctypes.c_int] * 6 + [_dp] * 16 + [ctypes.c_int]
            lib.ssd_oracle_max_threads.restype = ctypes.c_int
            lib.ssd_oracle_max_threads.argtypes = []
            _lib = lib
    return _lib


def max_threads() -> int:
    """Threads the OpenMP loop uses when ``nthreads`` is not given."""
    return _load().ssd_oracle_max_threads()


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def forward(x, dt, A, B, C, D=None, initial_state=None, ngroups=None,
            nthreads: int = 0, want_final: bool = True):
    """Serial fp64 SSD forward.

    x [b,L,H,P], dt [b,L,H], A [H], B/C [b,L,G,N], D [H] or None,
    initial_state [b,H,P,N] or None (zeros).  Returns (y [b,L,H,P],
    final_state [b,H,P,N] or None), both float64.
    """
    x, dt, A, B, C = (_f64(v) for v in (x, dt, A, B, C))
    D = None if D is None else _f64(D)
    init = None if initial_state is None else _f64(initial_state)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if ngroups is not None and ngroups != G:
        raise ValueError("ngroups does not match B's group dimension")
    if dt.shape != (b, L, H) or A.shape != (H,) or B.shape != (b, L, G, N) \
            or C.shape != B.shape:
        raise ValueError("inconsistent input shapes")
    if D is not None and D.shape != (H,):
        raise ValueError("D must have shape [nheads]")
    if init is not None and init.shape != (b, H, P, N):
        raise ValueError("initial_state must have shape [b,H,P,N]")
    y = np.empty((b, L, H, P), dtype=np.float64)
    final = np.empty((b, H, P, N), dtype=np.float64) if want_final else None
    rc = _load().ssd_oracle_forward(b, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A),
                                    _ptr(B), _ptr(C), _ptr(D), _ptr(init),
                                    _ptr(y), _ptr(final), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem (code %d)" % rc)
    return y, final


def backward(x, dt, A, B, C, D, initial_state, dy, dfinal=None, nthreads: int = 0):
    """Gradients of the serial fp64 forward, by reverse-mode differentiation
    of its loop (``ssd_oracle_backward`` in ``ssd_oracle.c``).

    dy [b,L,H,P] is the gradient of the loss with respect to y, dfinal
    [b,H,P,N] (or None = 0) with respect to the final state.  Returns a dict
    of float64 arrays: dx [b,L,H,P], ddt [b,L,H], dA [H], dB and dC
    [b,L,G,N], dD [H] and dinit [b,H,P,N] (the gradients with respect to D
    and the initial state also when those are None, i.e. at D = 0 and a
    zero initial state).
    """
    x, dt, A, B, C, dy = (_f64(v) for v in (x, dt, A, B, C, dy))
    D = None if D is None else _f64(D)
    init = None if initial_state is None else _f64(initial_state)
    dfin = None if dfinal is None else _f64(dfinal)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if dt.shape != (b, L, H) or A.shape != (H,) or B.shape != (b, L, G, N) \
            or C.shape != B.shape or dy.shape != x.shape:
        raise ValueError("inconsistent input shapes")
    if D is not None and D.shape != (H,):
        raise ValueError("D must have shape [nheads]")
    for v in (init, dfin):
        if v is not None and v.shape != (b, H, P, N):
            raise ValueError("states must have shape [b,H,P,N]")
    out = {"dx": np.empty_like(x), "ddt": np.empty_like(dt), "dA": np.empty(H),
           "dB": np.empty_like(B), "dC": np.empty_like(C), "dD": np.empty(H),
           "dinit": np.empty((b, H, P, N))}
    rc = _load().ssd_oracle_backward(
        b, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init),
        _ptr(dy), _ptr(dfin), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]),
        _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dinit"]), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the problem (code %d)" % rc)
    return out


def forward_slices(x, dt, A, B, C, D, initial_state, ngroups, slices,
                   nthreads: int = 0):
    """Serial fp64 forward for a subset of (batch, head) slices only.

    Slices of the recurrence are independent, so each listed (b, h) is
    gathered into a problem of its own with one head and one group; the
    result is exactly that slice of the full problem.  ``x`` etc. may be
    float32 arrays holding the exact values the GPU sees.  Returns
    (y [n, L, P], final [n, P, N]) in float64.
    """
    H = x.shape[2]
    G = B.shape[2]
    hpg = H // ngroups
    assert G == ngroups
    bs = np.array([s[0] for s in slices])
    hs = np.array([s[1] for s in slices])
    gs = hs // hpg
    xs = x[bs, :, hs, :][:, :, None, :]           # [n, L, 1, P]
    dts = dt[bs, :, hs][:, :, None]                # [n, L, 1]
    Bs = B[bs, :, gs, :][:, :, None, :]            # [n, L, 1, N]
    Cs = C[bs, :, gs, :][:, :, None, :]
    As = np.asarray(A)[hs]
    Ds = None if D is None else np.asarray(D)[hs]
    inits = None if initial_state is None else initial_state[bs, hs][:, None]
    n = len(slices)
    # Each gathered slice becomes one batch entry with one head: A and D are
    # per head, so run the slices one by one to keep A[h] per slice.
    ys, finals = [], []
    for i in range(n):
        yi, fi = forward(xs[i:i + 1], dts[i:i + 1], As[i:i + 1], Bs[i:i + 1],
                         Cs[i:i + 1], None if Ds is None else Ds[i:i + 1],
                         None if inits is None else inits[i:i + 1],
                         nthreads=nthreads)
        ys.append(yi[0, :, 0, :])
        finals.append(fi[0, 0])
    return np.stack(ys), np.stack(finals)


def state_update(state, x, dt, A, B, C, D=None, ngroups=None):
    """One decode step: the serial recurrence applied to a single token.

    state [b,H,P,N], x [b,H,P], dt [b,H], B/C [b,G,N].  Returns
    (new_state, y [b,H,P]) in float64; ``state`` is not modified.
    """
    x = np.asarray(x)
    y, final = forward(x[:, None], np.asarray(dt)[:, None], A,
                       np.asarray(B)[:, None], np.asarray(C)[:, None], D,
                       state, ngroups)
    return final, y[:, 0]
