"""mccb_backward_noalloc (the entry point for callers that cannot allocate) against mccb_backward on
the same inputs, through the C-ABI: two calls in a row on one device, the second with a smaller
input, so that the second runs on a scratch that still holds the first call's partials. gradX and
gradWeight must be bit-identical to the workspace entry point's (same kernels, same plan).

This module is collected last (test_zz_*): it must pass alone in a fresh process and after every
other GPU test."""
from __future__ import annotations

import pytest
import torch

import masked_depthwise_causal_amd as mdc
from synth import custom

from .gpu_util import announce, gpu_inputs

pytestmark = pytest.mark.gpu


def _both(wl):
    """(gradX, gradWeight) bits of mccb_backward and of mccb_backward_noalloc on one input."""
    gy, x, w, m = gpu_inputs(wl)
    dt = mdc.DTYPE_CODE[gy.dtype]
    st = torch.cuda.current_stream().cuda_stream
    mptr = None if m is None else m.data_ptr()
    ws = mdc.workspace_for(wl.S, wl.B, wl.H, gy.dtype, gy.device)
    ws.fill_(0x5A)
    gx0, gw0 = torch.empty_like(gy), torch.empty_like(w)
    gx1 = torch.full_like(gy, -7.0)
    gw1 = torch.full_like(w, -7.0)
    torch.cuda.synchronize()
    announce(f"mccb_backward {wl.name}")
    rc = mdc.mccb_backward(gy.data_ptr(), x.data_ptr(), w.data_ptr(), mptr, gx0.data_ptr(),
                           gw0.data_ptr(), wl.S, wl.B, wl.H, dt, ws.data_ptr(),
                           ws.numel(), st)
    assert rc == mdc.MCCB_OK, mdc.mccb_status_string(rc)
    announce(f"mccb_backward_noalloc {wl.name}")
    rc = mdc.mccb_backward_noalloc(gy.data_ptr(), x.data_ptr(), w.data_ptr(), mptr,
                                   gx1.data_ptr(), gw1.data_ptr(), wl.S, wl.B, wl.H, dt, st)
    assert rc == mdc.MCCB_OK, mdc.mccb_status_string(rc)
    torch.cuda.synchronize()
    return (gx0.view(torch.int16), gw0.view(torch.int16), gx1.view(torch.int16),
            gw1.view(torch.int16))


def test_noalloc_matches_workspace_entry_point_two_calls():
    big = custom(4096, 4, 4096, "bf16", ("bernoulli", 0.8), seed=71)   # 12.6 MB of partials
    small = custom(333, 3, 448, "fp16", ("prefix",), seed=72)           # fewer, other strips
    for wl in (big, small):
        gx0, gw0, gx1, gw1 = _both(wl)
        assert torch.equal(gx0, gx1), f"{wl.name}: gradX differs between the entry points"
        assert torch.equal(gw0, gw1), f"{wl.name}: gradWeight differs between the entry points"
