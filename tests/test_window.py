"""GPU parity for windows other than the page's W = 3 (W = 1, 2, 4), backward and forward.

The constraints section supports only W = 3 "for now"; the kernels take W = 1..4 through the
extended calls (the binding picks them when the weight is [W,H] with W != 3). Same bars as W = 3:
gradX and y within 1 ulp of the oracle's correctly rounded value (and expected bit-exact),
gradWeight within the relative bar and 1 ulp of the oracle's rounding. Small shapes element by
element, the full-size workloads on sampled channels and rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import masked_depthwise_causal_amd as mdc
from synth import WORKLOADS, custom
from synth import workloads as wls

from .gpu_util import (announce, compare_columns, compare_full, compare_rows, gpu_inputs, gpu_run,
                       sample_channels, sample_rows)
from .test_forward import compare_columns as fwd_compare_columns
from .test_forward import compare_full as fwd_compare_full
from .test_forward import compare_rows as fwd_compare_rows
from .test_forward import gpu_forward
from .test_forward import sample_rows as fwd_sample_rows

pytestmark = pytest.mark.gpu

TAPS = [1, 2, 4]

SHAPES = [
    # (S, B, H, dtype, mask): S below, at and past a wave's turn (8 rows) and a block's round (16)
    (1, 2, 384, "bf16", ("bernoulli", 0.8)),
    (2, 3, 448, "fp16", ("null",)),
    (3, 1, 384, "bf16", ("prefix",)),
    (5, 2, 576, "bf16", ("bernoulli", 0.6)),
    (15, 2, 384, "fp16", ("bernoulli", 0.9)),
    (17, 3, 640, "bf16", ("all_true",)),
    (131, 5, 448, "bf16", ("bernoulli", 0.8)),
    (300, 2, 1024, "fp16", ("prefix",)),
]


def plan_of(wl):
    return mdc.mccb_get_plan(wl.S, wl.B, wl.H, mdc.MCCB_BF16 if wl.dtype == "bf16" else mdc.MCCB_FP16)


@pytest.mark.parametrize("W", TAPS)
@pytest.mark.parametrize("S,B,H,dtype,mask", SHAPES, ids=lambda v: str(v))
def test_backward_window_full(W, S, B, H, dtype, mask):
    wl = custom(S, B, H, dtype, mask, seed=S * 13 + B + 100 * W, W=W)
    gx, gw = gpu_run(wl, poison_workspace=True)
    assert tuple(gw.shape) == (W, H)
    compare_full(wl, gx, gw)


@pytest.mark.parametrize("W", TAPS)
@pytest.mark.parametrize("S,B,H,dtype,mask", SHAPES, ids=lambda v: str(v))
def test_forward_window_full(W, S, B, H, dtype, mask):
    wl = custom(S, B, H, dtype, mask, seed=S * 29 + B + 100 * W, W=W)
    fwd_compare_full(wl, gpu_forward(wl, poison=True))


def test_tile_boundaries_w4():
    """S around the strip and round boundaries the plan picks, with a 3-row look-ahead."""
    base = mdc.mccb_get_plan(4096, 2, 384, mdc.MCCB_BF16)
    Q, T = base["rows_per_round"], base["rows_per_strip"]
    for S in sorted({Q - 3, Q - 1, Q, Q + 1, Q + 3, 2 * Q + 3, T + 1, T + 3}):
        wl = custom(S, 2, 384, "bf16", ("bernoulli", 0.85), seed=S + 5, W=4)
        gx, gw = gpu_run(wl)
        compare_full(wl, gx, gw, tag=f"W=4 S={S}")


def test_strided_inputs_with_w4():
    wl = custom(70, 3, 448, "bf16", ("bernoulli", 0.8), seed=71, W=4)
    gy, x, w, m = gpu_inputs(wl)
    gy_s = gy.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    x_s = torch.zeros((wl.S, wl.B, wl.H, 2), dtype=x.dtype, device="cuda")
    x_s[..., 0] = x
    x_s = x_s[..., 0]  # channels 2 apart: packed
    w_s = w.t().contiguous().t()
    m_s = m.t().contiguous().t()
    gx, gw = mdc.backward(gy_s, x_s, w_s, m_s)
    y = mdc.forward(x_s, w_s, m_s)
    torch.cuda.synchronize()
    compare_full(wl, gx, gw, tag="W=4 strided")
    fwd_compare_full(wl, y, tag="W=4 strided")


@pytest.mark.parametrize("W", [2, 4])
@pytest.mark.parametrize("B,groups", [(24, 3), (32, 4)], ids=["96KiB_rows", "128KiB_rows"])
def test_wide_32KiB_spacing_windows(W, B, groups):
    """Rows of 96 and 128 KiB take the wide layout with column groups 32 KiB apart (3 and 4 groups
    of 256 columns); 2 and 4 taps compared whole, S with a ragged last round."""
    wl = custom(203, B, 2048, "bf16", ("bernoulli", 0.85), seed=203 + W + B, W=W)
    plan = plan_of(wl)
    assert plan["cols_per_block"] == 256 * groups and plan["waves_per_block"] == groups, plan
    assert plan["group_spacing"] == 32768, plan
    gx, gw = gpu_run(wl, poison_workspace=True)
    compare_full(wl, gx, gw, tag=f"W={W} wide {groups} x 32 KiB")


@pytest.mark.parametrize("W,idx", [(2, 3), (4, 3), (4, 4), (1, 2)],
                         ids=lambda v: str(v))
def test_full_size_window_sampled(W, idx):
    wl = wls.with_taps(WORKLOADS[idx], W)
    inputs = gpu_inputs(wl)
    gx, gw = gpu_run(wl, inputs)
    announce(f"compare {wl.name}: sampled channels")
    compare_columns(wl, gx, gw, sample_channels(wl, n_random=8, seed=W))
    announce(f"compare {wl.name}: sampled rows")
    compare_rows(wl, gx, sample_rows(wl, plan_of(wl), n_random=4, seed=W))
    del gx, gw
    y = gpu_forward(wl, (inputs[1], inputs[2], inputs[3]))
    announce(f"compare {wl.name} forward: sampled channels and rows")
    fwd_compare_columns(wl, y, sample_channels(wl, n_random=8, seed=W + 1))
    fwd_compare_rows(wl, y, fwd_sample_rows(wl, plan_of(wl), n_random=4, seed=W + 1))
    del y, inputs
    torch.cuda.empty_cache()


def test_w3_extended_call_equals_plain_call():
    """W = 3 through the extended entry point gives the plain call's bits."""
    wl = custom(200, 3, 448, "bf16", ("bernoulli", 0.8), seed=9)
    gy, x, w, m = gpu_inputs(wl)
    gx0, gw0 = mdc.backward(gy, x, w, m)
    gx1, gw1 = torch.empty_like(gx0), torch.empty_like(gw0)
    n = mdc.mccb_get_workspace_size_ex(gy.data_ptr(), x.data_ptr(), w.data_ptr(), wl.S, wl.B, wl.H,
                                       3, mdc.MCCB_BF16, None)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    rc = mdc.mccb_backward_ex(gy.data_ptr(), x.data_ptr(), w.data_ptr(), m.data_ptr(),
                              gx1.data_ptr(), gw1.data_ptr(), wl.S, wl.B, wl.H, 3, mdc.MCCB_BF16,
                              None, ws.data_ptr(), n, torch.cuda.current_stream().cuda_stream)
    assert rc == mdc.MCCB_OK
    torch.cuda.synchronize()
    assert torch.equal(gx0.view(torch.int16), gx1.view(torch.int16))
    assert torch.equal(gw0.view(torch.int16), gw1.view(torch.int16))
    assert np.array_equal(gw0.shape, (3, wl.H))
