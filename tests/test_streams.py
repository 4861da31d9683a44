"""The tensor front end on a stream that is not torch's current one: what the call allocates
(outputs, workspace) must belong to the stream the kernels run on, or torch's caching allocator can
hand it to work on the current stream while the kernels still use it."""
from __future__ import annotations

import pytest
import torch

import masked_depthwise_causal_amd as mdc
from synth import custom

from .gpu_util import announce, gpu_inputs

pytestmark = pytest.mark.gpu


def test_side_stream_not_current():
    wl = custom(4096, 4, 4096, "bf16", ("bernoulli", 0.9), seed=81)
    gy, x, w, m = gpu_inputs(wl)
    announce("reference on the current stream")
    gx_ref, gw_ref = mdc.backward(gy, x, w, m)
    torch.cuda.synchronize()
    nws = mdc.mccb_get_workspace_size(wl.S, wl.B, wl.H, mdc.MCCB_BF16)
    side = torch.cuda.Stream()
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        announce(f"side stream, not made current, rep {rep}")
        gx, gw = mdc.backward(gy, x, w, m, stream=side)  # workspace allocated and dropped inside
        # work on the current stream right away, on blocks of the workspace's size, for longer
        # than the backward takes
        for _ in range(50):
            junk = torch.empty(nws, dtype=torch.uint8, device="cuda")
            junk.fill_(0xFF)
            del junk
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(gw.view(torch.int16), gw_ref.view(torch.int16))
        assert torch.equal(gx.view(torch.int16), gx_ref.view(torch.int16))
