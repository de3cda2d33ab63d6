"""The no-allocation forward (ssd_chunk_scan_fwd_noalloc) against the
forward with a caller workspace (ssd_chunk_scan_fwd), through the C ABI.

Two calls in a row, the second on a smaller problem, so the second runs on a
scratch array that still holds the first call's intermediates: each must
equal the workspace entry point bit for bit (the same kernels on the same
inputs).  fp32 problems take the split path, which uses the scratch; a bf16
problem takes the fused pass, which needs none unless its sequence is cut
into segments."""
import numpy as np
import pytest

from state_space_sequence_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

ARGS = ("x", "dt", "A", "B", "C", "D", "initial_state")


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from state_space_sequence_amd import libssd
    libssd.load()
    return torch.device("cuda:0")


def _both(dev, shape, io, Q, seed):
    import torch
    from state_space_sequence_amd import libssd
    from state_space_sequence_amd.inputs import to_torch
    b, L, H, P, N, G = shape
    inp = make_inputs(b, L, H, P, N, G, io_dtype=io, init_std=0.1, seed=seed)
    t = to_torch(inp, io, dev)
    code = libssd.SSD_BF16 if io == "bf16" else libssd.SSD_F32
    need = libssd.ssd_chunk_scan_fwd_workspace_size(b, L, H, P, N, G, Q, code)
    assert need <= libssd.NOALLOC_SCRATCH_BYTES
    y_ws, f_ws = libssd.ssd_chunk_scan_fwd(*(t[k] for k in ARGS), chunk_len=Q)
    y_na = torch.empty_like(t["x"])
    f_na = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    libssd.ssd_chunk_scan_fwd_noalloc(*(t[k] for k in ARGS), Q, y_na, f_na)
    torch.cuda.synchronize()
    print("  %s %s: workspace %d bytes" % (shape, io, need), flush=True)
    return y_ws, f_ws, y_na, f_na, need


def test_noalloc_matches_workspace_entry_point_twice(dev):
    import torch
    # first a larger problem, then a smaller one on the same scratch
    for shape, io, Q, seed, uses_scratch in (
            ((2, 777, 4, 64, 128, 2), "f32", 128, 61, True),
            ((1, 300, 3, 32, 64, 1), "f32", 64, 62, True),
            ((2, 500, 4, 64, 128, 1), "bf16", 256, 63, False)):
        y_ws, f_ws, y_na, f_na, need = _both(dev, shape, io, Q, seed)
        assert (need > 0) == uses_scratch
        assert torch.isfinite(y_na).all() and torch.isfinite(f_na).all()
        assert torch.equal(y_na, y_ws), shape
        assert torch.equal(f_na, f_ws), shape


def test_noalloc_segmented_fused_pass(dev, monkeypatch):
    """The fused pass cut into segments keeps the segments' states in the
    scratch: a larger then a smaller segmented problem, each equal to the
    workspace entry point."""
    import torch
    monkeypatch.setenv("SSD_FORWARD_PATH", "fused")
    for shape, nseg, seed in (((2, 1000, 4, 64, 128, 2), 4, 64), ((1, 600, 2, 64, 128, 1), 2, 65)):
        monkeypatch.setenv("SSD_FUSED_SEGMENTS", str(nseg))
        y_ws, f_ws, y_na, f_na, need = _both(dev, shape, "bf16", 64, seed)
        assert need > 0
        assert torch.equal(y_na, y_ws), shape
        assert torch.equal(f_na, f_ws), shape


def test_noalloc_rejects_a_problem_beyond_the_scratch(dev):
    import torch
    from state_space_sequence_amd import libssd
    b, L, H, P, N, G, Q = 1, 8192, 80, 64, 128, 1, 256
    need = libssd.ssd_chunk_scan_fwd_workspace_size(b, L, H, P, N, G, Q, libssd.SSD_F32)
    assert need > libssd.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((b, L, H, P), device=dev)
    dt = torch.zeros((b, L, H), device=dev)
    A = -torch.ones(H, device=dev)
    Bm = torch.zeros((b, L, G, N), device=dev)
    y = torch.empty_like(x)
    with pytest.raises(libssd.SsdError) as ei:
        libssd.ssd_chunk_scan_fwd_noalloc(x, dt, A, Bm, Bm, None, None, Q, y, None)
    assert ei.value.status == libssd.SSD_ERR_WORKSPACE
    assert np.isfinite(0.0)
