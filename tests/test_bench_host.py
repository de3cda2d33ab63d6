"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the algorithmic
byte and flop counts the roofline divides by, and the source hash that keeps
a stored traffic measurement tied to the kernel it was taken on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_headline_algorithmic_bytes_and_flops():
    """The 2.7B-shape layer (b4 L8192 H80 P64 N128 G1 Q256, bf16, zero initial
    state): x and y 335.5 MB each, B and C 16.8 MB, dt 10.5 MB, the final
    state 10.5 MB, A and D 640 B; the chunked flops by term."""
    import bench
    from state_space_sequence_amd.inputs import WORKLOADS
    w = WORKLOADS["mamba2_2p7b"]
    b, L, H, P, N, G, Q = 4, 8192, 80, 64, 128, 1, 256
    assert (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_len) == \
        (b, L, H, P, N, G, Q)
    xy = 2 * (b * L * H * P * 2)
    bc = 2 * b * L * G * N * 2
    dt = b * L * H * 4
    final = b * H * P * N * 4
    assert bench.alg_bytes_forward(w, 2) == xy + bc + dt + final + 2 * H * 4 == 708838016
    nc = L // Q
    tri = Q * (Q + 1) // 2
    flops = (2 * tri * N * b * nc * G            # C B^T, causal triangle
             + 2 * P * Q * N * b * nc * H        # chunk states
             + 2 * Q * N * P * b * nc * H        # output from the entering state
             + 2 * tri * P * b * nc * H          # output within the chunk
             + 2 * P * N * b * nc * H)           # state passing
    assert bench.alg_flops_forward(w) == flops == 130262499328


def test_ragged_length_counts_whole_chunks():
    """A length that is not a multiple of the chunk (16380 = 63 * 256 + 252)
    counts 64 chunks of flops, and bytes for the real tokens only."""
    import bench
    from state_space_sequence_amd.inputs import WORKLOADS
    w = WORKLOADS["grouped_g8"]
    assert w.seqlen % w.chunk_len != 0
    full = bench.alg_flops_forward(w)
    nc = -(-w.seqlen // w.chunk_len)
    per_chunk = full // (nc * w.batch)
    assert full == per_chunk * nc * w.batch
    x = w.batch * w.seqlen * w.nheads * w.headdim * 2
    assert bench.alg_bytes_forward(w, 2) > 2 * x


def test_source_hash_ignores_comments_and_layout():
    import bench
    base = bench.kernel_source_hash()

    def read_commented(path):
        with open(os.path.join(ROOT, path)) as f:
            text = f.read()
        return "// a remark\n" + text.replace("\n", "\n\n") + "\n/* another */\n"

    def read_changed(path):
        with open(os.path.join(ROOT, path)) as f:
            text = f.read()
        return text + "\nstatic const int kChanged = 1;\n"

    assert bench.kernel_source_hash(read_commented) == base
    assert bench.kernel_source_hash(read_changed) != base
