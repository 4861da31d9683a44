"""The C-ABI from C: compile tests/c_abi_client.c against include/mccb.h with gcc in strict C99,
link it to the built library, run it (host-only entry points, no GPU) and compare what it prints
with the Python binding's answers for the same calls."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

import masked_depthwise_causal_amd as mdc
from masked_depthwise_causal_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def client_output(tmp_path_factory):
    # MCCB_TEST_CC: another C compiler command line (the sanitized run uses clang with the
    # address and undefined-behaviour sanitizers)
    cc = os.environ.get("MCCB_TEST_CC", "gcc").split()
    if shutil.which(cc[0]) is None:
        pytest.skip(f"{cc[0]} not available")
    mdc.lib()  # builds the library if it is missing
    lib_dir, lib_name = os.path.split(build.LIB)
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_client")
    cmd = [*cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", build.INCLUDE,
           os.path.join(HERE, "c_abi_client.c"), "-o", exe, "-L", lib_dir, f"-l:{lib_name}",
           f"-Wl,-rpath,{lib_dir}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    out = {}
    for line in run.stdout.splitlines():
        k, v = line.split(" ", 1)
        out[k] = v
    return out


def test_phase1_and_plan_match_binding(client_output):
    o = client_output
    assert int(o["ws_rc"]) == mdc.MCCB_OK and int(o["plan_rc"]) == mdc.MCCB_OK
    want = mdc.mccb_get_workspace_size(16384, 32, 5120, mdc.MCCB_BF16)
    assert int(o["ws_bytes"]) == want == int(o["plan_ws"])
    p = mdc.mccb_get_plan(16384, 32, 5120, mdc.MCCB_BF16)
    assert int(o["rows_per_strip"]) == p["rows_per_strip"]
    assert int(o["n_strips"]) == p["n_strips"]
    # fp64 partials [n_strips][3][B*H]
    assert want == p["n_strips"] * 3 * 32 * 5120 * 8


def test_validation_codes_from_c(client_output):
    o = client_output
    assert int(o["null_out"]) == 161001
    assert int(o["bad_dtype"]) == 161002
    assert int(o["bad_H"]) == 561002
    assert int(o["bad_BS"]) == 561002
    assert int(o["backward_null"]) == 161001
    assert int(o["forward_null"]) == 161001


def test_status_strings_from_c(client_output):
    o = client_output
    assert o["str_ok"] == mdc.mccb_status_string(0)
    assert o["str_shape"] == mdc.mccb_status_string(561002)
    assert o["str_unknown"] == mdc.mccb_status_string(12345)
