"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

- The C oracle, driven through every optional pointer, length 1, ragged and
  grouped shapes and the shapes it refuses (tests/sanitize/oracle_driver.c),
  built with gcc and the sanitizers, leak checking on.
- libssd's host side (validation, path choice, workspace layout), driven
  through workspace queries and rejected calls that never reach a GPU
  (tests/sanitize/api_driver.cpp): ssd_api.hip rebuilt with the sanitizers
  on its host pass only and linked with the library's other objects.

A sanitizer report makes the program exit non-zero."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")


def _run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-6000:])
    return r.stdout


def test_oracle_under_asan_and_ubsan(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "ssd_oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
    assert _run([exe], env=env).strip() == "ok"


def test_host_validation_under_asan_and_ubsan(tmp_path):
    from state_space_sequence_amd import build_lib
    hipcc = build_lib.hipcc()
    objs = [o for o in glob.glob(os.path.join(build_lib.BUILD_DIR, "*.o"))
            if not os.path.basename(o).startswith("ssd_api")]
    if len(objs) < len(build_lib.sources()) - 1:
        build_lib.build()
        objs = [o for o in glob.glob(os.path.join(build_lib.BUILD_DIR, "*.o"))
                if not os.path.basename(o).startswith("ssd_api")]
    # the sanitizers on the host pass only: each -fsanitize= follows -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_o = str(tmp_path / "api_asan.o")
    drv_o = str(tmp_path / "driver.o")
    exe = str(tmp_path / "api_asan")
    flags = [f for f in build_lib.compile_flags() if f not in ("-O3", "-fPIC")]
    _run([hipcc] + flags + ["-O1", "-g"] + san +
         ["-c", os.path.join(build_lib.CSRC, "ssd_api.hip"), "-o", api_o])
    _run([hipcc, "-O1", "-g", "-std=c++17", "-I" + build_lib.INCLUDE] + san +
         ["-c", os.path.join(HERE, "api_driver.cpp"), "-o", drv_o])
    _run([hipcc, "--offload-arch=" + build_lib.ARCH] + san[:4] + [api_o] + objs + [drv_o, "-o", exe])
    # (the HIP runtime's own allocations outlive main: no leak check)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    assert _run([exe], env=env, timeout=120).strip() == "ok"
