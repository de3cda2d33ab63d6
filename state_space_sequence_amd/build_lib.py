"""Build libssd.so (all HIP sources under csrc/) for gfx950 with hipcc.

Run as ``python -m state_space_sequence_amd.build_lib``; ``__graft_entry__.build``
calls :func:`build`.  The library is written to lib/ next to this file so it
travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "lib", "libssd.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libssd needs the ROCm toolchain to build")


def compile_flags():
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        "-I" + INCLUDE, "-I" + CSRC,
        # packed fp32 instructions stay off: plain float code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in ordinary VGPRs: the kernels update them with
        # vector ALU ops between MFMAs, which the AGPR form turns into copies
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Wno-unused-command-line-argument",
    ]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + compile_flags() + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libssd.so.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(os.path.dirname(LIB_PATH), exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
