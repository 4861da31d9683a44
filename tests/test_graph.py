"""The entry points enqueue kernels only (no allocation, no memset, no host synchronization), so
a caller can capture them in a HIP graph. Capture the backward and the forward once, replay the
graph several times with unrelated eager work and synchronizations in between, and check every
replay against the eager result bit for bit."""
from __future__ import annotations

import pytest
import torch

import masked_depthwise_causal_amd as mdc
from synth import custom

from .gpu_util import announce, gpu_inputs

pytestmark = pytest.mark.gpu


def test_graph_capture_and_replay():
    wl = custom(1000, 3, 448, "bf16", ("bernoulli", 0.8), seed=61)
    gy, x, w, m = gpu_inputs(wl)
    ws = mdc.workspace_for(wl.S, wl.B, wl.H, gy.dtype, gy.device)
    gx_e, gw_e = mdc.backward(gy, x, w, m, workspace=ws)
    y_e = mdc.forward(x, w, m)
    torch.cuda.synchronize()

    gx, gw, y = torch.empty_like(gx_e), torch.empty_like(gw_e), torch.empty_like(y_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    announce("capture mccb_backward + mccb_forward")
    with torch.cuda.graph(g, stream=side):
        mdc.backward(gy, x, w, m, gradX=gx, gradWeight=gw, workspace=ws, stream=side)
        mdc.forward(x, w, m, y=y, stream=side)
    torch.cuda.synchronize()
    for rep in range(4):
        gx.fill_(0)
        gw.fill_(0)
        y.fill_(0)
        ws.fill_(0xFF)  # the workspace needs no initialisation
        scratch = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert torch.equal(gx.view(torch.int16), gx_e.view(torch.int16)), f"replay {rep}: gradX"
        assert torch.equal(gw.view(torch.int16), gw_e.view(torch.int16)), f"replay {rep}: gradWeight"
        assert torch.equal(y.view(torch.int16), y_e.view(torch.int16)), f"replay {rep}: y"
