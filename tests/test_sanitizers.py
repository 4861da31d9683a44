"""The CPU side under AddressSanitizer and UndefinedBehaviorSanitizer: the host half of the HIP
library (argument validation, plan, overlap and stride checks, the packed-input layout) and the
oracle are rebuilt with both sanitizers, and the CPU test modules that exercise them
(test_oracle.py, test_abi.py, test_c_client.py) run against those builds in a child process. Any
sanitizer report fails the run. No GPU is used: the library's device code is compiled unoptimized
and never launched (every call these modules make is rejected by validation or is host-only)."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

import pytest

import oracle
from masked_depthwise_causal_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm"


def _asan_runtime():
    hits = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


@pytest.mark.slow
def test_cpu_side_clean_under_asan_and_ubsan(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    clang = os.path.join(LLVM, "bin", "clang")
    rt = _asan_runtime()
    if not (os.path.exists(hipcc) and os.path.exists(clang) and rt):
        pytest.skip("hipcc, clang or the clang sanitizer runtime not available")
    lib = str(tmp_path / "libmccb_san.so")
    # host code sanitized (each -fsanitize= applies to the host compilation only); device code
    # built without optimization, since it never runs here
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-shared", "-fPIC",
           "-Xarch_device", "-O0", "-Xarch_device", "-g0",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", build.INCLUDE, build.SRC, "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    orc = str(tmp_path / "libmccb_oracle_san.so")
    cmd = [clang, *oracle.CFLAGS, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", oracle._SRC, "-o", orc, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ,
               LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               MCCB_LIBRARY=lib, MCCB_ORACLE_LIBRARY=orc,
               MCCB_TEST_CC=f"{clang} -fsanitize=address,undefined -shared-libasan "
                            f"-fno-sanitize-recover=all")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider", "tests/test_oracle.py", "tests/test_abi.py",
                          "tests/test_c_client.py"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert run.returncode == 0, out[-6000:]
    assert " passed" in run.stdout
