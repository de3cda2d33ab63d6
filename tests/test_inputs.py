"""The seeded input generator: determinism, value ranges, bf16 rounding."""
import numpy as np

from state_space_sequence_amd.inputs import WORKLOADS, make_inputs, round_to_bf16


def test_deterministic():
    a = make_inputs(2, 33, 4, 8, 16, 2, io_dtype="bf16", init_std=0.1, seed=3)
    b = make_inputs(2, 33, 4, 8, 16, 2, io_dtype="bf16", init_std=0.1, seed=3)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_ranges():
    inp = make_inputs(2, 500, 16, 8, 16, 1, io_dtype="f32", seed=1)
    A, dt, D = inp["A"], inp["dt"], inp["D"]
    assert np.all(A <= -1.0) and np.all(A >= -16.0)
    assert np.all(dt > 0) and np.all(np.isfinite(dt))
    assert np.all((D >= 0) & (D <= 1))
    assert inp["initial_state"] is None
    # dt concentrates around softplus(dt_bias) with dt_bias the inverse
    # softplus of a value in [1e-3, 1e-1]
    med = np.median(dt, axis=(0, 1))
    assert np.all(med > 5e-4) and np.all(med < 0.3)


def test_bf16_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-9,
                     1.0 + 2**-8 + 2**-12], dtype=np.float32)
    r = round_to_bf16(vals)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 -> 1+2^-6
    np.testing.assert_array_equal(r, np.array([1.0, 1.0, 1.0 + 2**-6, -2.5, 1.0,
                                               1.0 + 2**-7], dtype=np.float32))
    inp = make_inputs(1, 64, 2, 16, 16, 1, io_dtype="bf16", seed=2)
    for k in ("x", "B", "C"):
        bits = inp[k].view(np.uint32)
        assert np.all(bits & 0xFFFF == 0)


def test_workload_table():
    w = WORKLOADS["mamba2_2p7b"]
    assert (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len) == \
        (4, 8192, 80, 64, 128, 1, 256)
    g = WORKLOADS["grouped_g8"]
    assert g.seqlen % g.chunk_len != 0 and g.nheads // g.ngroups == 8
