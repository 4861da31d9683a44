"""Compile the HIP library (libmccb.so) for gfx950 in-tree."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "mccb.hip")
# MCCB_LIBRARY names another build of the library to load instead (the tests' host-sanitized
# build); it is loaded as given and never built.
LIB = os.environ.get("MCCB_LIBRARY") or os.path.join(PKG, "libmccb.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build_library(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, *(extra or []), "-I", INCLUDE, SRC, "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    if verbose:
        print(res.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_library())
