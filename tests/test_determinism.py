"""GPU determinism and memory hygiene: repeated runs with a poisoned workspace are bit-identical, a
null mask equals an all-true mask bit for bit, and nothing outside the outputs is written (guard
canaries around gradX, gradWeight and the workspace)."""
from __future__ import annotations

import pytest
import torch

import masked_depthwise_causal_amd as mdc
from synth import WORKLOADS, custom
from synth import workloads as wls

from .gpu_util import announce, gpu_inputs

pytestmark = pytest.mark.gpu


def test_repeat_runs_bit_identical():
    wl = custom(3000, 8, 1024, "bf16", ("bernoulli", 0.9), seed=42)
    gy, x, w, m = gpu_inputs(wl)
    outs = []
    for rep in range(5):
        ws = mdc.workspace_for(wl.S, wl.B, wl.H, gy.dtype, gy.device)
        ws.fill_(0xFF if rep % 2 == 0 else 0x7F)
        announce(f"repeat {rep}")
        gx, gw = mdc.backward(gy, x, w, m, workspace=ws)
        torch.cuda.synchronize()
        outs.append((gx.view(torch.int16).clone(), gw.view(torch.int16).clone()))
    for gx, gw in outs[1:]:
        assert torch.equal(gx, outs[0][0]) and torch.equal(gw, outs[0][1])


def test_null_mask_equals_all_true():
    for dtype in ("bf16", "fp16"):
        wl = custom(777, 3, 448, dtype, ("null",), seed=9)
        gy, x, w, _ = gpu_inputs(wl)
        ones = torch.ones((wl.B, wl.S), dtype=torch.uint8, device="cuda")
        announce(f"null vs all-true {dtype}")
        gx0, gw0 = mdc.backward(gy, x, w, None)
        gx1, gw1 = mdc.backward(gy, x, w, ones)
        gx2, gw2 = mdc.backward(gy, x, w, ones.bool())
        torch.cuda.synchronize()
        for a, b in ((gx0, gx1), (gw0, gw1), (gx0, gx2), (gw0, gw2)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_canaries_untouched():
    wl = custom(600, 3, 448, "bf16", ("bernoulli", 0.8), seed=11)
    gy, x, w, m = gpu_inputs(wl)
    pad = 4096  # elements of guard on each side
    N = wl.S * wl.B * wl.H
    gx_buf = torch.full((N + 2 * pad,), -3.0, dtype=torch.bfloat16, device="cuda")
    gw_buf = torch.full((3 * wl.H + 2 * pad,), -3.0, dtype=torch.bfloat16, device="cuda")
    wsz = mdc.mccb_get_workspace_size(wl.S, wl.B, wl.H, mdc.MCCB_BF16)
    ws_buf = torch.full((wsz + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    gx = gx_buf[pad:pad + N].view(wl.S, wl.B, wl.H)
    gw = gw_buf[pad:pad + 3 * wl.H].view(3, wl.H)
    ws = ws_buf[pad:pad + wsz]
    announce("canaries")
    mdc.backward(gy, x, w, m, gradX=gx, gradWeight=gw, workspace=ws)
    torch.cuda.synchronize()
    for buf, n, fillv in ((gx_buf, N, -3.0), (gw_buf, 3 * wl.H, -3.0)):
        assert torch.all(buf[:pad] == fillv) and torch.all(buf[pad + n:] == fillv)
    assert torch.all(ws_buf[:pad] == 0xA5) and torch.all(ws_buf[pad + wsz:] == 0xA5)
    # and the inputs are unchanged
    assert torch.equal(gy.view(torch.int16), wls.full_tensor(wl, wls.STREAM_GY, "cuda").view(torch.int16))


def test_stream_argument_is_honoured():
    wl = WORKLOADS[0]
    gy, x, w, m = gpu_inputs(wl)
    s = torch.cuda.Stream()
    ref_gx, ref_gw = mdc.backward(gy, x, w, m)
    torch.cuda.synchronize()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gx, gw = mdc.backward(gy, x, w, m, stream=s)
    s.synchronize()
    assert torch.equal(gx.view(torch.int16), ref_gx.view(torch.int16))
    assert torch.equal(gw.view(torch.int16), ref_gw.view(torch.int16))
