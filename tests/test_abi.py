"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments with the documented status codes before
touching the GPU (every call below returns from host-side validation; no
kernel is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


@pytest.fixture(scope="module")
def lib():
    from state_space_sequence_amd import libssd
    if not os.path.exists(libssd.LIB_PATH):
        from state_space_sequence_amd import build_lib
        build_lib.build()
    return libssd.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("ssd_chunk_scan_fwd", "ssd_state_update",
                 "ssd_chunk_scan_fwd_workspace_size", "ssd_status_string"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strings(lib):
    assert lib.ssd_abi_version() == 1
    for code in range(6):
        assert lib.ssd_status_string(code)
    assert b"non-finite" in lib.ssd_status_string(5)
    assert lib.ssd_status_string(99) == b"unknown status"
    assert lib.ssd_chunk_scan_fwd_max_kernels() >= 3


FAKE = 0x10000  # 256-byte aligned, never dereferenced: validation fails first


def ws_size(lib, *args):
    out = ctypes.c_size_t(0)
    st = lib.ssd_chunk_scan_fwd_workspace_size(*args, ctypes.byref(out))
    return st, out.value


def test_workspace_size(lib, monkeypatch):
    nc = 32
    vec = 3 * 4 * 80 * nc * 256 * 4
    monkeypatch.setenv("SSD_FORWARD_PATH", "split")
    st, n = ws_size(lib, 4, 8192, 80, 64, 128, 1, 256, 1)
    assert st == 0
    # prefix sums (two), dt, C B^T, chunk states, packed-sequence starts
    expect = vec + 4 * nc * 1 * 256 * 256 * 4 + 4 * nc * 80 * 64 * 128 * 4 + 4 * nc * 256 * 4
    assert n >= expect and n - expect < 7 * 256
    monkeypatch.setenv("SSD_FORWARD_PATH", "fused")
    st, n = ws_size(lib, 4, 8192, 80, 64, 128, 1, 256, 1)
    assert st == 0 and n == 0                               # the fused pass keeps all on chip
    st, _ = ws_size(lib, 4, 8192, 80, 48, 128, 1, 256, 1)   # headdim 48: no fused path
    assert st == 2
    monkeypatch.delenv("SSD_FORWARD_PATH")
    st, n_auto = ws_size(lib, 4, 8192, 80, 64, 128, 1, 256, 1)
    assert st == 0 and n_auto == n                          # fused is the default here
    st, _ = ws_size(lib, 4, 8192, 80, 64, 128, 3, 256, 1)
    assert st == 1  # nheads % ngroups
    st, _ = ws_size(lib, 4, 8192, 80, 64, 128, 1, 100, 1)
    assert st == 2
    assert lib.ssd_chunk_scan_fwd_workspace_size(1, 1, 1, 16, 16, 1, 16, 0, None) == 1


def fwd(lib, **kw):
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, init=None, Q=64, G=1,
             b=1, L=100, H=2, P=16, N=16, io=0, y=FAKE, fin=None, ws=FAKE,
             wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.ssd_chunk_scan_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"],
                                  a["Q"], a["G"], a["b"], a["L"], a["H"], a["P"], a["N"],
                                  a["io"], a["y"], a["fin"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(G=3, H=4), 1),
    (dict(L=0), 1),
    (dict(b=-1), 1),
    (dict(io=7), 1),
    (dict(x=None), 1),
    (dict(C=None), 1),
    (dict(y=None), 1),
    (dict(x=FAKE + 2), 1),
    (dict(init=FAKE + 4), 1),
    (dict(Q=48), 2),
    (dict(Q=512), 2),
    (dict(P=24), 2),
    (dict(P=256), 2),
    (dict(N=8), 2),
    (dict(N=512), 2),
    (dict(wsb=16), 3),
    (dict(ws=None), 3),
    (dict(ws=FAKE + 16), 3),
])
def test_forward_validation(lib, kw, code):
    assert fwd(lib, **kw) == code


def test_timed_needs_enough_events(lib):
    n = lib.ssd_chunk_scan_fwd_max_kernels()
    arr = (ctypes.c_void_p * n)(*([FAKE] * n))
    st = lib.ssd_chunk_scan_fwd_timed(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 64, 1, 1,
                                      100, 2, 16, 16, 0, FAKE, None, FAKE, 1 << 40, None,
                                      arr, n, None, None)
    assert st == 1


def upd(lib, **kw):
    a = dict(state=FAKE, x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, G=1, b=2, H=4,
             P=16, N=16, io=1, y=FAKE, stream=None)
    a.update(kw)
    return lib.ssd_state_update(a["state"], a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"],
                                a["G"], a["b"], a["H"], a["P"], a["N"], a["io"], a["y"],
                                a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(G=3), 1),
    (dict(b=0), 1),
    (dict(state=None), 1),
    (dict(y=None), 1),
    (dict(io=5), 1),
    (dict(state=FAKE + 8), 1),
    (dict(P=20), 2),
    (dict(N=300), 2),
])
def test_state_update_validation(lib, kw, code):
    assert upd(lib, **kw) == code


def test_binding_refuses_cpu_tensors():
    import torch
    from state_space_sequence_amd import libssd
    x = torch.zeros(1, 4, 2, 16)
    with pytest.raises(ValueError):
        libssd.ssd_chunk_scan_fwd(x, torch.zeros(1, 4, 2), torch.zeros(2),
                                  torch.zeros(1, 4, 1, 16), torch.zeros(1, 4, 1, 16))


@pytest.mark.parametrize("bias,lo,hi", [
    (None, -0.1, 1.0),                   # dt_min < 0
    (None, 0.5, 0.1),                    # dt_min > dt_max
    (None, float("nan"), 1.0),           # NaN bound
    (None, 0.0, float("nan")),
    (FAKE + 2, 0.0, float("inf")),       # misaligned dt_bias
])
def test_dt_proc_validation(lib, bias, lo, hi):
    """Invalid preprocessing options are rejected before anything launches
    (every other argument here is valid)."""
    from state_space_sequence_amd.libssd import DtProc  # the ssd_dt_proc layout
    p = DtProc(bias, 1, lo, hi)
    st = lib.ssd_chunk_scan_fwd_ex(
        ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
        ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None, None, 64, 1, 1, 100, 2, 64, 128,
        1, ctypes.c_void_p(FAKE), None, None, ctypes.c_size_t(0), None, ctypes.byref(p))
    assert st == 1
    st = lib.ssd_state_update_ex(
        ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
        ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None, 1, 2, 4,
        16, 16, 1, ctypes.c_void_p(FAKE), None, ctypes.byref(p))
    assert st == 1


def conv(lib, **kw):
    a = dict(x=FAKE, w=FAKE, bias=None, b=2, L=100, D=64, W=4, act=1, io=1, out=FAKE,
             state=None)
    a.update(kw)
    return lib.ssd_causal_conv1d_fwd(a["x"], a["w"], a["bias"], a["b"], a["L"], a["D"],
                                     a["W"], a["act"], a["io"], a["out"], a["state"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=0), 1),
    (dict(L=0), 1),
    (dict(act=2), 1),
    (dict(io=4), 1),
    (dict(x=None), 1),
    (dict(w=None), 1),
    (dict(out=None), 1),
    (dict(x=FAKE + 2), 1),
    (dict(w=FAKE + 2), 1),
    (dict(D=12), 2),
    (dict(W=5), 2),
    (dict(W=1), 2),
])
def test_conv_validation(lib, kw, code):
    assert conv(lib, **kw) == code


def test_conv_update_validation(lib):
    args = [FAKE, FAKE, FAKE, None, 2, 64, 4, 1, 1, FAKE, None]
    bad_state = list(args)
    bad_state[0] = None
    assert lib.ssd_causal_conv1d_update(*bad_state) == 1
    bad_w = list(args)
    bad_w[6] = 7
    assert lib.ssd_causal_conv1d_update(*bad_w) == 2


def norm(lib, **kw):
    a = dict(y=FAKE, z=None, w=FAKE, rows=4, dim=64, eps=1e-5, nbg=0, io=1, out=FAKE)
    a.update(kw)
    return lib.ssd_gated_rmsnorm_fwd(a["y"], a["z"], a["w"], a["rows"], a["dim"], a["eps"],
                                     a["nbg"], a["io"], a["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=0), 1),
    (dict(dim=0), 1),
    (dict(eps=-1.0), 1),
    (dict(eps=float("nan")), 1),
    (dict(io=3), 1),
    (dict(y=None), 1),
    (dict(w=None), 1),
    (dict(out=None), 1),
    (dict(y=FAKE + 8), 1),
    (dict(z=FAKE + 4), 1),
    (dict(dim=12), 2),
    (dict(dim=8200), 2),
])
def test_norm_validation(lib, kw, code):
    assert norm(lib, **kw) == code


def test_header_status_codes():
    """The status values the header documents, SSD_ERR_NONFINITE among them."""
    text = open(HEADER).read()
    for name, value in (("SSD_OK", 0), ("SSD_ERR_INVALID_ARGUMENT", 1), ("SSD_ERR_UNSUPPORTED", 2),
                        ("SSD_ERR_WORKSPACE", 3), ("SSD_ERR_HIP", 4), ("SSD_ERR_NONFINITE", 5)):
        assert re.search(r"\b%s = %d\b" % (name, value), text), name
    from state_space_sequence_amd import libssd
    assert libssd.SSD_ERR_NONFINITE == 5


def test_finite_check_keeps_validation_first(lib, monkeypatch):
    """With the non-finite check requested, a call with bad arguments still
    returns its validation status before anything is enqueued (no kernel,
    no read-back: this runs without a GPU)."""
    monkeypatch.setenv("SSD_CHECK_FINITE", "1")
    p = ctypes.c_void_p(FAKE)
    # forward: nheads not a multiple of ngroups
    st = lib.ssd_chunk_scan_fwd(p, p, p, p, p, None, None, 64, 3, 1, 64, 4, 16, 16, 0, p, None,
                                None, 0, None)
    assert st == 1
    # forward: unsupported chunk length
    st = lib.ssd_chunk_scan_fwd(p, p, p, p, p, None, None, 100, 1, 1, 64, 4, 16, 16, 0, p, None,
                                None, 0, None)
    assert st == 2
    # decode: missing state
    st = lib.ssd_state_update(None, p, p, p, p, p, None, 1, 2, 4, 16, 16, 0, p, None)
    assert st == 1
    # convolution: width 5
    st = lib.ssd_causal_conv1d_fwd(p, p, None, 1, 10, 16, 5, 1, 1, p, None, None)
    assert st == 2
    # normalisation: dim not a multiple of 8
    st = lib.ssd_gated_rmsnorm_fwd(p, None, p, 4, 12, ctypes.c_float(1e-5), 0, 1, p, None)
    assert st == 2


def test_noalloc_rejects_oversized_problems_before_the_gpu(lib):
    """ssd_chunk_scan_fwd_noalloc: a problem whose workspace exceeds the
    scratch array returns SSD_ERR_WORKSPACE from host validation, and bad
    arguments keep their own status (no GPU needed: nothing is enqueued)."""
    from state_space_sequence_amd import libssd
    p = ctypes.c_void_p(FAKE)
    need = ctypes.c_size_t(0)
    assert lib.ssd_chunk_scan_fwd_workspace_size(1, 8192, 80, 64, 128, 1, 256, 0,
                                                 ctypes.byref(need)) == 0
    assert need.value > libssd.NOALLOC_SCRATCH_BYTES
    st = lib.ssd_chunk_scan_fwd_noalloc(p, p, p, p, p, None, None, 256, 1, 1, 8192, 80, 64, 128,
                                        0, p, None, None)
    assert st == 3
    st = lib.ssd_chunk_scan_fwd_noalloc(p, p, p, p, p, None, None, 256, 3, 1, 64, 80, 64, 128,
                                        0, p, None, None)
    assert st == 1   # nheads % ngroups
    st = lib.ssd_chunk_scan_fwd_noalloc(None, p, p, p, p, None, None, 256, 1, 1, 64, 8, 64, 128,
                                        0, p, None, None)
    assert st == 1   # x missing
    assert "#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in open(HEADER).read()
    assert libssd.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_fused_segments_only_for_few_column_groups(lib, monkeypatch):
    """The fused forward cuts the sequence into segments (and needs a
    workspace for the states they leave) only when the layer has few
    128-column groups: the 8-group layer (b2 L16380 H64 P64 G8: 64 groups,
    1 + 4 segments) but not the 2.7B layer (160 groups) or short sequences."""
    monkeypatch.delenv("SSD_FUSED_SEGMENTS", raising=False)
    monkeypatch.setenv("SSD_FORWARD_PATH", "fused")
    state = 2 * 64 * 64 * 128 * 4
    st, n = ws_size(lib, 2, 16380, 64, 64, 128, 8, 256, 1)
    # segments 0 .. 3 leave a state each, plus their log decays
    assert st == 0 and n // state == 4 and n % state < 4096
    st, n = ws_size(lib, 4, 8192, 80, 64, 128, 1, 256, 1)
    assert st == 0 and n == 0
    st, n = ws_size(lib, 2, 1000, 64, 64, 128, 8, 256, 1)   # 32 blocks: one pass
    assert st == 0 and n == 0
    monkeypatch.setenv("SSD_FUSED_SEGMENTS", "3")
    st, n = ws_size(lib, 2, 1000, 64, 64, 128, 8, 256, 1)
    assert st == 0 and n // state == 2


# ---------------------------------------------------------------- gradients

def bwd(lib, **kw):
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, init=None, dy=FAKE, dfin=None,
             Q=64, G=1, b=1, L=100, H=2, P=16, N=16, io=0, dx=FAKE, ddt=FAKE, dA=FAKE,
             dB=FAKE, dC=FAKE, dD=None, dinit=None, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.ssd_chunk_scan_bwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"],
                                  a["dy"], a["dfin"], a["Q"], a["G"], a["b"], a["L"], a["H"],
                                  a["P"], a["N"], a["io"], a["dx"], a["ddt"], a["dA"], a["dB"],
                                  a["dC"], a["dD"], a["dinit"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(G=3, H=4), 1),
    (dict(L=0), 1),
    (dict(io=7), 1),
    (dict(dy=None), 1),
    (dict(dx=None), 1),
    (dict(ddt=None), 1),
    (dict(dA=None), 1),
    (dict(dB=None), 1),
    (dict(dC=None), 1),
    (dict(dy=FAKE + 2), 1),
    (dict(dfin=FAKE + 4), 1),
    (dict(dinit=FAKE + 8), 1),
    (dict(dD=FAKE + 2), 1),
    (dict(Q=48), 2),
    (dict(P=24), 2),
    (dict(N=512), 2),
    (dict(wsb=16), 3),
    (dict(ws=None), 3),
    (dict(ws=FAKE + 16), 3),
])
def test_backward_validation(lib, kw, code):
    assert bwd(lib, **kw) == code


def test_backward_workspace_size(lib):
    """The recomputed forward's regions plus the gradient pass's: the
    adjoint chunk products (a state per chunk), fp64 chunk-end products per
    state slice, three per-token vectors per head, the summed score tiles
    (a C B^T-sized block in the io type), the per-tile strict row sums and
    column sums, the dD / dA partial sums, and the head
    groups' partial dB and dC."""
    b, L, H, P, N, G, Q = 4, 8192, 80, 64, 128, 1, 256
    nc, nsl, nrb = L // Q, (P * N + 1023) // 1024, Q // 64
    out = ctypes.c_size_t(0)
    assert lib.ssd_chunk_scan_bwd_workspace_size(b, L, H, P, N, G, Q, 1, ctypes.byref(out)) == 0
    fwd_split = 3 * b * H * nc * Q * 4 + b * nc * G * Q * Q * 4 + b * nc * H * P * N * 4 + b * nc * Q * 4
    # the dB / dC kernels split a group's 80 heads so that there are about
    # 2048 workgroups: 512 (batch x chunks x row blocks) -> 4 groups of 20,
    # each with an fp32 partial dB and dC
    nhg = 4
    # the summed-score kernel: 10 tiles x 32 chunks x 4 rows = 1280 workgroups
    # -> 2 head groups of 40 for about 2048, each with fp32 partial tiles
    nhw = 2
    extra = (b * nc * H * P * N * 4 + b * nc * H * nsl * 8 + 3 * b * H * nc * Q * 4 +
             b * nc * G * Q * Q * 2 + b * H * nc * nrb * Q * 8 + b * H * nc * nrb * Q * 8 +
             b * nc * H * nrb * 4 + b * nc * H * 8 + 2 * nhg * b * L * G * N * 4 +
             nhw * b * nc * G * Q * Q * 4)
    assert out.value >= fwd_split + extra and out.value - (fwd_split + extra) < 16 * 256
    assert lib.ssd_chunk_scan_bwd_workspace_size(b, L, H, P, N, 3, Q, 1, ctypes.byref(out)) == 1
    assert lib.ssd_chunk_scan_bwd_max_kernels() == 9


def test_float_quotient_of_staging_indexes_is_exact():
    """The gradient pass's score-tile kernel splits a vector index v of its
    x staging into (row, chunk) as floor((v + 1/2) * fp32(1 / n)) in fp32
    arithmetic, n = headdim / vector width.  The kernel relies on that being
    the integer quotient v // n for every index it forms (v below 64 rows x
    32 chunks) and every n it can see (headdim a multiple of 16, at most 128:
    n from 2 to 32); this checks all of them in the same fp32 arithmetic."""
    import numpy as np
    v = np.arange(0, 64 * 32, dtype=np.int64)
    for n in range(1, 33):
        rcp = np.float32(1.0) / np.float32(n)
        q = ((v.astype(np.float32) + np.float32(0.5)) * rcp).astype(np.float32)
        assert np.array_equal(np.floor(q).astype(np.int64), v // n), n
