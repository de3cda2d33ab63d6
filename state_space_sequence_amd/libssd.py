"""ctypes binding of libssd.so (C ABI in include/ssd.h).

Argument marshalling only: every step of the SSD runs in the HIP kernels of
libssd.so.  PyTorch supplies device memory and the current stream.  There is
no fallback: if libssd.so is missing or cannot be loaded, every call raises.

Python names mirror the C entry points:
    ssd_chunk_scan_fwd_workspace_size(...)       -> int bytes
    ssd_chunk_scan_fwd(x, dt, A, B, C, ...)      -> (y, final_state)
    ssd_chunk_scan_fwd_timed(events, x, ...)     -> (y, final_state, kernel names)
    ssd_state_update(state, x, dt, A, B, C, ...) -> y   (state updated in place)
    ssd_chunk_scan_bwd(x, ..., dy, dfinal_state)  -> dict of gradients
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libssd.so")

SSD_OK = 0
SSD_ERR_INVALID_ARGUMENT = 1
SSD_ERR_UNSUPPORTED = 2
SSD_ERR_WORKSPACE = 3
SSD_ERR_HIP = 4
SSD_ERR_NONFINITE = 5  # opt-in check: SSD_CHECK_FINITE set in the environment

SSD_F32 = 0
SSD_BF16 = 1

_lock = threading.Lock()
_lib = None


class SsdError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = load().ssd_status_string(status).decode()
        super().__init__("%s failed: %s (status %d)" % (where, msg, status))


_i = ctypes.c_int
_p = ctypes.c_void_p
_sz = ctypes.c_size_t

_FWD_ARGS = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _sz, _p]
# x dt A B C D init dy dfinal, chunk_len ngroups b L H P N io, dx ddt dA dB dC dD dinit, ws bytes stream
_BWD_ARGS = [_p] * 9 + [_i] * 8 + [_p] * 7 + [_p, _sz, _p]


class DtProc(ctypes.Structure):
    """``ssd_dt_proc`` of include/ssd.h: the time-step preprocessing the
    ``_ex`` entry points apply, min(max(f(dt + dt_bias), dt_min), dt_max)."""
    _fields_ = [("dt_bias", ctypes.c_void_p), ("dt_softplus", ctypes.c_int),
                ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float)]


class Gate(ctypes.Structure):
    """``ssd_gate`` of include/ssd.h: the output gate z (nullable) and
    whether D is per (head, headdim column)."""
    _fields_ = [("z", ctypes.c_void_p), ("D_per_channel", ctypes.c_int)]


def load():
    """Load libssd.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libssd.so not found at %s; build it with "
                "`python -m state_space_sequence_amd.build_lib`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        lib.ssd_abi_version.restype = _i
        lib.ssd_abi_version.argtypes = []
        lib.ssd_status_string.restype = ctypes.c_char_p
        lib.ssd_status_string.argtypes = [_i]
        lib.ssd_chunk_scan_fwd_workspace_size.restype = _i
        lib.ssd_chunk_scan_fwd_workspace_size.argtypes = [_i] * 8 + [ctypes.POINTER(_sz)]
        lib.ssd_chunk_scan_fwd.restype = _i
        lib.ssd_chunk_scan_fwd.argtypes = _FWD_ARGS
        lib.ssd_chunk_scan_fwd_max_kernels.restype = _i
        lib.ssd_chunk_scan_fwd_max_kernels.argtypes = []
        lib.ssd_chunk_scan_fwd_timed.restype = _i
        lib.ssd_chunk_scan_fwd_timed.argtypes = _FWD_ARGS + [
            ctypes.POINTER(_p), _i, ctypes.POINTER(_i), ctypes.POINTER(ctypes.c_char_p)]
        lib.ssd_state_update.restype = _i
        lib.ssd_state_update.argtypes = [_p] * 7 + [_i] * 6 + [_p, _p]
        lib.ssd_chunk_scan_bwd_workspace_size.restype = _i
        lib.ssd_chunk_scan_bwd_workspace_size.argtypes = [_i] * 8 + [ctypes.POINTER(_sz)]
        lib.ssd_chunk_scan_bwd.restype = _i
        lib.ssd_chunk_scan_bwd.argtypes = _BWD_ARGS
        lib.ssd_chunk_scan_bwd_max_kernels.restype = _i
        lib.ssd_chunk_scan_bwd_max_kernels.argtypes = []
        lib.ssd_chunk_scan_bwd_timed.restype = _i
        lib.ssd_chunk_scan_bwd_timed.argtypes = _BWD_ARGS + [_p, _i, ctypes.POINTER(_i), _p]
        lib.ssd_chunk_scan_fwd_noalloc.restype = _i
        lib.ssd_chunk_scan_fwd_noalloc.argtypes = _FWD_ARGS[:17] + [_p]
        lib.ssd_chunk_scan_fwd_ex.restype = _i
        lib.ssd_chunk_scan_fwd_ex.argtypes = _FWD_ARGS + [ctypes.POINTER(DtProc)]
        lib.ssd_chunk_scan_fwd_varlen.restype = _i
        lib.ssd_chunk_scan_fwd_varlen.argtypes = _FWD_ARGS + [_p, ctypes.POINTER(DtProc)]
        lib.ssd_chunk_scan_fwd_full.restype = _i
        lib.ssd_chunk_scan_fwd_full.argtypes = _FWD_ARGS + [_p, ctypes.POINTER(DtProc),
                                                             ctypes.POINTER(Gate)]
        lib.ssd_state_update_full.restype = _i
        lib.ssd_state_update_full.argtypes = [_p] * 7 + [_i] * 6 + [_p, _p, ctypes.POINTER(DtProc),
                                                                    ctypes.POINTER(Gate)]
        lib.ssd_state_update_ex.restype = _i
        lib.ssd_state_update_ex.argtypes = [_p] * 7 + [_i] * 6 + [_p, _p, ctypes.POINTER(DtProc)]
        lib.ssd_causal_conv1d_fwd.restype = _i
        lib.ssd_causal_conv1d_fwd.argtypes = [_p, _p, _p] + [_i] * 6 + [_p, _p, _p]
        lib.ssd_causal_conv1d_update.restype = _i
        lib.ssd_causal_conv1d_update.argtypes = [_p, _p, _p, _p] + [_i] * 5 + [_p, _p]
        lib.ssd_gated_rmsnorm_fwd.restype = _i
        lib.ssd_gated_rmsnorm_fwd.argtypes = [_p, _p, _p, _i, _i, ctypes.c_float, _i, _i, _p, _p]
        _lib = lib
    return _lib


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise TypeError("x/B/C must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(name, t, dtype=None, device=None):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def max_kernels() -> int:
    return load().ssd_chunk_scan_fwd_max_kernels()


def ssd_chunk_scan_fwd_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups,
                                      chunk_len, io_dtype) -> int:
    out = _sz(0)
    st = load().ssd_chunk_scan_fwd_workspace_size(batch, seqlen, nheads, headdim, dstate,
                                                  ngroups, chunk_len, io_dtype,
                                                  ctypes.byref(out))
    if st != SSD_OK:
        raise SsdError(st, "ssd_chunk_scan_fwd_workspace_size")
    return out.value


def _dt_proc(dt_bias, dt_softplus, dt_limit, H, dev):
    """The ssd_dt_proc struct for these options, or None when none is set
    (then dt is used as given)."""
    import torch
    if dt_bias is None and not dt_softplus and dt_limit is None:
        return None
    if dt_bias is not None:
        _check_dev("dt_bias", dt_bias, torch.float32, dev)
        if tuple(dt_bias.shape) != (H,):
            raise ValueError("dt_bias must be [H]")
    lo, hi = (0.0, float("inf")) if dt_limit is None else (float(dt_limit[0]), float(dt_limit[1]))
    return DtProc(None if dt_bias is None else dt_bias.data_ptr(), 1 if dt_softplus else 0,
                  lo, hi)


def _gate(z, D, like, H, P, dev):
    """The ssd_gate struct for a gate z (shaped like ``like``) and a D of
    shape [H] or [H, P], or None when neither is used."""
    d2 = D is not None and D.dim() == 2
    if D is not None and tuple(D.shape) not in ((H,), (H, P)):
        raise ValueError("D must be [H] or [H, P]")
    if z is None and not d2:
        return None
    if z is not None:
        _check_dev("z", z, like.dtype, dev)
        if tuple(z.shape) != tuple(like.shape):
            raise ValueError("z must have x's shape")
    return Gate(None if z is None else z.data_ptr(), 1 if d2 else 0)


def _forward(timed_events, x, dt, A, B, C, D, initial_state, chunk_len, ngroups, y,
             final_state, workspace, return_final_state, stream, dtp=None, seq_idx=None,
             z=None):
    import torch
    lib = load()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    io = _dtype_code(x)
    _check_dev("x", x, None, dev)
    for n, t in (("B", B), ("C", C)):
        _check_dev(n, t, x.dtype, dev)
    for n, t in (("dt", dt), ("A", A), ("D", D), ("initial_state", initial_state)):
        _check_dev(n, t, torch.float32, dev)
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [b,L,H,P] and B/C [b,L,G,N]")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if ngroups is not None and ngroups != G:
        raise ValueError("ngroups=%d but B has %d groups" % (ngroups, G))
    if tuple(dt.shape) != (b, L, H) or tuple(A.shape) != (H,) or \
            tuple(B.shape) != (b, L, G, N) or tuple(C.shape) != (b, L, G, N):
        raise ValueError("inconsistent shapes x%s dt%s A%s B%s C%s" % (
            tuple(x.shape), tuple(dt.shape), tuple(A.shape), tuple(B.shape), tuple(C.shape)))
    gate = _gate(z, D, x, H, P, dev)
    if initial_state is not None and tuple(initial_state.shape) != (b, H, P, N):
        raise ValueError("initial_state must be [b,H,P,N]")
    if y is None:
        y = torch.empty_like(x)
    _check_dev("y", y, x.dtype, dev)
    if tuple(y.shape) != tuple(x.shape):
        raise ValueError("y must have x's shape")
    if final_state is None and return_final_state:
        final_state = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    _check_dev("final_state", final_state, torch.float32, dev)
    need = ssd_chunk_scan_fwd_workspace_size(b, L, H, P, N, G, chunk_len, io)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_dev("workspace", workspace, torch.uint8, dev)
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(initial_state),
            int(chunk_len), G, b, L, H, P, N, io, _ptr(y), _ptr(final_state),
            _ptr(workspace), _sz(workspace.numel()), _stream_handle(stream))
    if gate is not None:
        if timed_events is not None:
            raise ValueError("the timed forward takes no gate")
        if seq_idx is not None:
            _check_dev("seq_idx", seq_idx, torch.int32, dev)
            if tuple(seq_idx.shape) != (b, L):
                raise ValueError("seq_idx must be [b, L] int32")
        st = lib.ssd_chunk_scan_fwd_full(*args, _ptr(seq_idx),
                                         None if dtp is None else ctypes.byref(dtp),
                                         ctypes.byref(gate))
        where = "ssd_chunk_scan_fwd_full"
    elif seq_idx is not None:
        if timed_events is not None:
            raise ValueError("the timed forward takes unpacked rows only")
        _check_dev("seq_idx", seq_idx, torch.int32, dev)
        if tuple(seq_idx.shape) != (b, L):
            raise ValueError("seq_idx must be [b, L] int32")
        st = lib.ssd_chunk_scan_fwd_varlen(*args, _ptr(seq_idx),
                                           None if dtp is None else ctypes.byref(dtp))
        where = "ssd_chunk_scan_fwd_varlen"
    elif dtp is not None:
        if timed_events is not None:
            raise ValueError("the timed forward takes processed dt only")
        st = lib.ssd_chunk_scan_fwd_ex(*args, ctypes.byref(dtp))
        where = "ssd_chunk_scan_fwd_ex"
    elif timed_events is None:
        st = lib.ssd_chunk_scan_fwd(*args)
        where = "ssd_chunk_scan_fwd"
    else:
        arr = (ctypes.c_void_p * len(timed_events))(*[ctypes.c_void_p(e) for e in timed_events])
        nk = _i(0)
        names = (ctypes.c_char_p * max_kernels())()
        st = lib.ssd_chunk_scan_fwd_timed(*args, arr, len(timed_events), ctypes.byref(nk),
                                          names)
        where = "ssd_chunk_scan_fwd_timed"
        if st == SSD_OK:
            timed_events_info = [names[i].decode() for i in range(nk.value)]
            return y, final_state, timed_events_info
    if st != SSD_OK:
        raise SsdError(st, where)
    return y, final_state


def ssd_chunk_scan_fwd(x, dt, A, B, C, D=None, initial_state=None, chunk_len=256,
                       ngroups=None, y=None, final_state=None, workspace=None,
                       return_final_state=True, stream=None, dt_bias=None,
                       dt_softplus=False, dt_limit=None, seq_idx=None, z=None):
    """Chunked SSD forward on the current (or given) torch stream.

    x [b,L,H,P] (fp32|bf16), dt [b,L,H] fp32, A [H] fp32, B/C [b,L,G,N] (x's
    dtype), D [H] fp32 or None, initial_state [b,H,P,N] fp32 or None.
    Returns (y [b,L,H,P] in x's dtype, final_state [b,H,P,N] fp32 or None).
    Outputs and workspace are allocated with torch when not supplied;
    final_state may be the initial_state tensor itself.

    With dt_bias ([H] fp32), dt_softplus or dt_limit ((min, max)) given, dt
    is the raw time step and the kernels use min(max(f(dt + dt_bias), min),
    max), f = softplus when dt_softplus (the layer's `dt_bias`,
    `dt_softplus`, `dt_limit` arguments; ssd_chunk_scan_fwd_ex).

    seq_idx ([b, L] int32) packs several sequences per row: the state is
    reset where it changes (ssd_chunk_scan_fwd_varlen).

    z (x's shape and dtype) gates the output, y = (C h + D x) silu(z), and D
    may be [H, P] (per headdim column) as well as [H]
    (ssd_chunk_scan_fwd_full)."""
    dtp = _dt_proc(dt_bias, dt_softplus, dt_limit, A.shape[0], x.device)
    return _forward(None, x, dt, A, B, C, D, initial_state, chunk_len, ngroups, y,
                    final_state, workspace, return_final_state, stream, dtp, seq_idx, z)


def ssd_chunk_scan_fwd_timed(events, x, dt, A, B, C, D=None, initial_state=None,
                             chunk_len=256, ngroups=None, y=None, final_state=None,
                             workspace=None, return_final_state=True, stream=None):
    """``ssd_chunk_scan_fwd`` that also records the given hipEvent_t handles
    (ints, at least max_kernels()+1 of them) around each kernel: events[i]
    before kernel i, events[k] after the last of the k kernels.  Returns
    (y, final_state, kernel_names)."""
    return _forward(list(events), x, dt, A, B, C, D, initial_state, chunk_len, ngroups,
                    y, final_state, workspace, return_final_state, stream)


def ssd_chunk_scan_bwd_workspace_size(batch, seqlen, nheads, headdim, dstate, ngroups,
                                      chunk_len, io_dtype) -> int:
    out = _sz(0)
    st = load().ssd_chunk_scan_bwd_workspace_size(batch, seqlen, nheads, headdim, dstate,
                                                  ngroups, chunk_len, io_dtype,
                                                  ctypes.byref(out))
    if st != SSD_OK:
        raise SsdError(st, "ssd_chunk_scan_bwd_workspace_size")
    return out.value


def bwd_max_kernels() -> int:
    return load().ssd_chunk_scan_bwd_max_kernels()


def ssd_chunk_scan_bwd(x, dt, A, B, C, D, initial_state, dy, dfinal_state=None,
                       chunk_len=256, ngroups=None, want_dD=True, want_dinit=True,
                       out=None, workspace=None, stream=None, events=None):
    """Gradients of the chunked forward (ssd_chunk_scan_bwd).

    The forward's inputs as for ssd_chunk_scan_fwd (processed dt, no gate or
    packed sequences), dy (x's shape and dtype) and dfinal_state ([b,H,P,N]
    fp32 or None = 0).  Returns a dict dx, ddt, dA, dB, dC, dD, dinit (the
    last two None unless wanted), allocated with torch unless ``out`` (a
    dict of the same keys) supplies them.  With ``events`` (at least
    bwd_max_kernels()+1 hipEvent_t handles) the timed twin runs and the dict
    also holds ``kernel_names``."""
    import torch
    lib = load()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    io = _dtype_code(x)
    _check_dev("x", x, None, dev)
    for n, t in (("B", B), ("C", C), ("dy", dy)):
        _check_dev(n, t, x.dtype, dev)
    for n, t in (("dt", dt), ("A", A), ("D", D), ("initial_state", initial_state),
                 ("dfinal_state", dfinal_state)):
        _check_dev(n, t, torch.float32, dev)
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [b,L,H,P] and B/C [b,L,G,N]")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if ngroups is not None and ngroups != G:
        raise ValueError("ngroups=%d but B has %d groups" % (ngroups, G))
    if tuple(dt.shape) != (b, L, H) or tuple(A.shape) != (H,) or \
            tuple(B.shape) != (b, L, G, N) or tuple(C.shape) != (b, L, G, N) or \
            tuple(dy.shape) != tuple(x.shape):
        raise ValueError("inconsistent shapes")
    if D is not None and tuple(D.shape) != (H,):
        raise ValueError("D must be [H]")
    for n, t in (("initial_state", initial_state), ("dfinal_state", dfinal_state)):
        if t is not None and tuple(t.shape) != (b, H, P, N):
            raise ValueError("%s must be [b,H,P,N]" % n)
    o = dict(out or {})
    f32 = torch.float32
    shapes = {"dx": (tuple(x.shape), x.dtype), "ddt": ((b, L, H), f32), "dA": ((H,), f32),
              "dB": ((b, L, G, N), x.dtype), "dC": ((b, L, G, N), x.dtype),
              "dD": ((H,), f32), "dinit": ((b, H, P, N), f32)}
    for k, (shape, dtype) in shapes.items():
        if k == "dD" and not want_dD or k == "dinit" and not want_dinit:
            o.setdefault(k, None)
            continue
        if o.get(k) is None:
            o[k] = torch.empty(shape, dtype=dtype, device=dev)
        _check_dev(k, o[k], dtype, dev)
        if tuple(o[k].shape) != shape:
            raise ValueError("%s must be %s" % (k, shape))
    need = ssd_chunk_scan_bwd_workspace_size(b, L, H, P, N, G, chunk_len, io)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check_dev("workspace", workspace, torch.uint8, dev)
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(initial_state),
            _ptr(dy), _ptr(dfinal_state), int(chunk_len), G, b, L, H, P, N, io,
            _ptr(o["dx"]), _ptr(o["ddt"]), _ptr(o["dA"]), _ptr(o["dB"]), _ptr(o["dC"]),
            _ptr(o["dD"]), _ptr(o["dinit"]), _ptr(workspace), _sz(workspace.numel()),
            _stream_handle(stream))
    if events is None:
        st = lib.ssd_chunk_scan_bwd(*args)
        where = "ssd_chunk_scan_bwd"
    else:
        ev = list(events)
        arr = (ctypes.c_void_p * len(ev))(*[ctypes.c_void_p(e) for e in ev])
        nk = _i(0)
        names = (ctypes.c_char_p * bwd_max_kernels())()
        st = lib.ssd_chunk_scan_bwd_timed(*args, arr, len(ev), ctypes.byref(nk), names)
        where = "ssd_chunk_scan_bwd_timed"
        if st == SSD_OK:
            o["kernel_names"] = [names[i].decode() for i in range(nk.value)]
    if st != SSD_OK:
        raise SsdError(st, where)
    return o


NOALLOC_SCRATCH_BYTES = 64 << 20   # SSD_NOALLOC_SCRATCH_BYTES of include/ssd.h


def ssd_chunk_scan_fwd_noalloc(x, dt, A, B, C, D, initial_state, chunk_len, y, final_state,
                               stream=None):
    """``ssd_chunk_scan_fwd_noalloc``: the forward with no workspace argument
    and no allocation anywhere, neither in the library nor here, so y (and
    final_state, unless None) must be given.  The split path uses the
    library's per-GPU scratch array; calls that overlap on one GPU race."""
    import torch
    lib = load()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    io = _dtype_code(x)
    for n, t in (("x", x), ("B", B), ("C", C), ("y", y)):
        _check_dev(n, t, x.dtype, dev)
    for n, t in (("dt", dt), ("A", A), ("D", D), ("initial_state", initial_state),
                 ("final_state", final_state)):
        _check_dev(n, t, torch.float32, dev)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(y.shape) != tuple(x.shape) or tuple(dt.shape) != (b, L, H) or \
            tuple(B.shape) != (b, L, G, N) or tuple(C.shape) != (b, L, G, N):
        raise ValueError("inconsistent shapes")
    for n, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and tuple(t.shape) != (b, H, P, N):
            raise ValueError("%s must be [b,H,P,N]" % n)
    st = lib.ssd_chunk_scan_fwd_noalloc(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                        _ptr(initial_state), int(chunk_len), G, b, L, H, P, N,
                                        io, _ptr(y), _ptr(final_state), _stream_handle(stream))
    if st != SSD_OK:
        raise SsdError(st, "ssd_chunk_scan_fwd_noalloc")
    return y, final_state


def ssd_state_update(state, x, dt, A, B, C, D=None, ngroups=None, y=None, stream=None,
                     dt_bias=None, dt_softplus=False, dt_limit=None, z=None):
    """One decode token, in place on ``state``.

    state [b,H,P,N] fp32, x [b,H,P] (fp32|bf16), dt [b,H] fp32, A [H],
    B/C [b,G,N] (x's dtype), D [H], [H, P] or None.  Returns y [b,H,P] in
    x's dtype.  dt_bias / dt_softplus / dt_limit: as in ssd_chunk_scan_fwd
    (ssd_state_update_ex); z (x's shape) gates the output
    (ssd_state_update_full)."""
    import torch
    lib = load()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    io = _dtype_code(x)
    _check_dev("state", state, torch.float32, dev)
    _check_dev("x", x, None, dev)
    for n, t in (("B", B), ("C", C)):
        _check_dev(n, t, x.dtype, dev)
    for n, t in (("dt", dt), ("A", A), ("D", D)):
        _check_dev(n, t, torch.float32, dev)
    b, H, P, N = state.shape
    G = B.shape[1]
    if ngroups is not None and ngroups != G:
        raise ValueError("ngroups=%d but B has %d groups" % (ngroups, G))
    if tuple(x.shape) != (b, H, P) or tuple(dt.shape) != (b, H) or tuple(A.shape) != (H,) \
            or tuple(B.shape) != (b, G, N) or tuple(C.shape) != (b, G, N):
        raise ValueError("inconsistent decode shapes")
    gate = _gate(z, D, x, H, P, dev)
    if y is None:
        y = torch.empty_like(x)
    _check_dev("y", y, x.dtype, dev)
    args = (_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), G, b, H, P,
            N, io, _ptr(y), _stream_handle(stream))
    dtp = _dt_proc(dt_bias, dt_softplus, dt_limit, H, dev)
    if gate is not None:
        st = lib.ssd_state_update_full(*args, None if dtp is None else ctypes.byref(dtp),
                                       ctypes.byref(gate))
        where = "ssd_state_update_full"
    elif dtp is None:
        st, where = lib.ssd_state_update(*args), "ssd_state_update"
    else:
        st, where = lib.ssd_state_update_ex(*args, ctypes.byref(dtp)), "ssd_state_update_ex"
    if st != SSD_OK:
        raise SsdError(st, where)
    return y


_ACT = {None: 0, "none": 0, "silu": 1, "swish": 1}


def _conv_params(x, weight, bias, activation, dev):
    import torch
    if activation not in _ACT:
        raise ValueError("activation must be None or 'silu'")
    _check_dev("weight", weight, torch.float32, dev)
    _check_dev("bias", bias, torch.float32, dev)
    D = x.shape[-1]
    if weight.dim() != 2 or weight.shape[0] != D:
        raise ValueError("weight must be [dim, width]")
    if bias is not None and tuple(bias.shape) != (D,):
        raise ValueError("bias must be [dim]")
    return D, weight.shape[1], _ACT[activation]


def ssd_causal_conv1d_fwd(x, weight, bias=None, activation="silu", out=None, conv_state=None,
                          return_conv_state=True, stream=None):
    """Causal depthwise convolution (+ SiLU) over a sequence, from an empty
    cache: x [b, L, dim] (fp32|bf16), weight [dim, width] fp32, bias [dim]
    fp32 or None.  Returns (out [b, L, dim] in x's dtype, conv_state
    [b, dim, width] in x's dtype, the cache for the decode path, or None)."""
    import torch
    lib = load()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    io = _dtype_code(x)
    _check_dev("x", x, None, dev)
    if x.dim() != 3:
        raise ValueError("x must be [b, L, dim]")
    D, W, act = _conv_params(x, weight, bias, activation, dev)
    b, L = x.shape[0], x.shape[1]
    if out is None:
        out = torch.empty_like(x)
    _check_dev("out", out, x.dtype, dev)
    if tuple(out.shape) != tuple(x.shape):
        raise ValueError("out must have x's shape")
    if conv_state is None and return_conv_state:
        conv_state = torch.empty((b, D, W), dtype=x.dtype, device=dev)
    _check_dev("conv_state", conv_state, x.dtype, dev)
    if conv_state is not None and tuple(conv_state.shape) != (b, D, W):
        raise ValueError("conv_state must be [b, dim, width]")
    st = lib.ssd_causal_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), b, L, D, W, act, io,
                                   _ptr(out), _ptr(conv_state), _stream_handle(stream))
    if st != SSD_OK:
        raise SsdError(st, "ssd_causal_conv1d_fwd")
    return out, conv_state


def ssd_causal_conv1d_update(conv_state, x, weight, bias=None, activation="silu", out=None,
                             stream=None):
    """One decode token: conv_state [b, dim, width] (x's dtype) is rolled
    left and x [b, dim] appended, in place; returns out [b, dim]."""
    import torch
    lib = load()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("x must be a GPU tensor")
    io = _dtype_code(x)
    _check_dev("x", x, None, dev)
    _check_dev("conv_state", conv_state, x.dtype, dev)
    if x.dim() != 2:
        raise ValueError("x must be [b, dim]")
    D, W, act = _conv_params(x, weight, bias, activation, dev)
    b = x.shape[0]
    if tuple(conv_state.shape) != (b, D, W):
        raise ValueError("conv_state must be [b, dim, width]")
    if out is None:
        out = torch.empty_like(x)
    _check_dev("out", out, x.dtype, dev)
    st = lib.ssd_causal_conv1d_update(_ptr(conv_state), _ptr(x), _ptr(weight), _ptr(bias), b,
                                      D, W, act, io, _ptr(out), _stream_handle(stream))
    if st != SSD_OK:
        raise SsdError(st, "ssd_causal_conv1d_update")
    return out


def ssd_gated_rmsnorm_fwd(y, z, weight, eps=1e-5, norm_before_gate=False, out=None, stream=None):
    """Gated RMS normalisation over the last axis: y, z [..., dim] (fp32|bf16;
    z may be None), weight [dim] fp32.  Returns out (y's shape and dtype);
    out may be y itself."""
    import torch
    lib = load()
    dev = y.device
    if dev.type != "cuda":
        raise ValueError("y must be a GPU tensor")
    io = _dtype_code(y)
    _check_dev("y", y, None, dev)
    _check_dev("z", z, y.dtype, dev)
    _check_dev("weight", weight, torch.float32, dev)
    dim = y.shape[-1]
    if z is not None and tuple(z.shape) != tuple(y.shape):
        raise ValueError("z must have y's shape")
    if tuple(weight.shape) != (dim,):
        raise ValueError("weight must be [dim]")
    rows = y.numel() // dim
    if out is None:
        out = torch.empty_like(y)
    _check_dev("out", out, y.dtype, dev)
    if tuple(out.shape) != tuple(y.shape):
        raise ValueError("out must have y's shape")
    st = lib.ssd_gated_rmsnorm_fwd(_ptr(y), _ptr(z), _ptr(weight), rows, dim, float(eps),
                                   1 if norm_before_gate else 0, io, _ptr(out),
                                   _stream_handle(stream))
    if st != SSD_OK:
        raise SsdError(st, "ssd_gated_rmsnorm_fwd")
    return out
