"""GPU parity with strided (non-contiguous) inputs, the parameter table's non-contiguous gradY, x,
weight and mask.

Each case builds device views with the same values as the seeded contiguous inputs but another
memory layout, runs mccb_backward_ex / mccb_forward_ex through the binding, and compares with the
CPU oracle on the contiguous values (layout is not arithmetic: the oracle is unchanged) and, bit
for bit, with the contiguous GPU path. Cases cover both ways the library reads a strided input: in
place (channels contiguous, aligned strides) and packed into the workspace first.
"""
from __future__ import annotations

import pytest
import torch

import masked_depthwise_causal_amd as mdc
from synth import WORKLOADS, custom
from synth import workloads as wls

from .gpu_util import (announce, compare_columns, compare_full, gpu_inputs, sample_channels)
from .test_forward import compare_columns as fwd_compare_columns
from .test_forward import compare_full as fwd_compare_full

pytestmark = pytest.mark.gpu


def as_bsh(t):
    """Same values, stored [B,S,H] (the permuted layout of a batch-major producer)."""
    return t.permute(1, 0, 2).contiguous().permute(1, 0, 2)


def as_h_slice(t, pad=64, off=32):
    """Same values as the middle of a wider-H tensor (row stride B*(H+pad), batch stride H+pad)."""
    S, B, H = t.shape
    big = torch.zeros((S, B, H + pad), dtype=t.dtype, device=t.device)
    big[:, :, off:off + H] = t
    return big[:, :, off:off + H]


def as_channel_strided(t):
    """Same values with channels 2 elements apart (forces the pack path)."""
    S, B, H = t.shape
    big = torch.zeros((S, B, H, 2), dtype=t.dtype, device=t.device)
    big[..., 0] = t
    return big[..., 0]


def as_odd_base(t):
    """Same values starting 2 bytes past a 16-byte boundary (forces the pack path)."""
    flat = torch.zeros(t.numel() + 8, dtype=t.dtype, device=t.device)
    flat[1:1 + t.numel()] = t.reshape(-1)
    return flat[1:1 + t.numel()].view(t.shape)


def transposed_weight(w):
    return w.t().contiguous().t()  # [3,H] view of [H,3] storage


def transposed_mask(m):
    return None if m is None else m.t().contiguous().t()  # [B,S] view of [S,B] storage


LAYOUTS = {
    "bsh": (as_bsh, as_bsh),
    "hslice": (as_h_slice, as_bsh),
    "gy_chstride_x_oddbase": (as_channel_strided, as_odd_base),
    "gy_oddbase_x_hslice": (as_odd_base, as_h_slice),
}


def run_both(wl, layout, tw=True, tm=True):
    gy, x, w, m = gpu_inputs(wl)
    fg, fx = LAYOUTS[layout]
    gy_s, x_s = fg(gy), fx(x)
    w_s = transposed_weight(w) if tw else w
    m_s = transposed_mask(m) if tm else m
    assert torch.equal(gy_s.view(torch.int16), gy.view(torch.int16))
    assert torch.equal(x_s.view(torch.int16), x.view(torch.int16))
    announce(f"mccb_backward_ex {wl.name} layout={layout} w^T={tw} mask^T={tm}")
    gx_s, gw_s = mdc.backward(gy_s, x_s, w_s, m_s)
    announce(f"mccb_backward {wl.name} (contiguous reference)")
    gx, gw = mdc.backward(gy, x, w, m)
    torch.cuda.synchronize()
    return (gx_s, gw_s), (gx, gw)


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("shape", [(37, 3, 448, "bf16", ("bernoulli", 0.8)),
                                   (130, 2, 384, "fp16", ("prefix",)),
                                   (20, 5, 576, "bf16", ("null",))],
                         ids=lambda v: str(v))
def test_backward_strided_small(layout, shape):
    S, B, H, dt, mk = shape
    wl = custom(S, B, H, dt, mk, seed=S + 7 * B)
    (gx_s, gw_s), (gx, gw) = run_both(wl, layout)
    compare_full(wl, gx_s, gw_s, tag=f"{wl.name} strided {layout}")
    assert torch.equal(gx_s.view(torch.int16), gx.view(torch.int16))
    assert torch.equal(gw_s.view(torch.int16), gw.view(torch.int16))


def test_backward_broadcast_batch():
    """x shared by every batch (batch stride 0) is read in place."""
    wl = custom(40, 4, 384, "bf16", ("bernoulli", 0.9), seed=77)
    gy, x, w, m = gpu_inputs(wl)
    xb = x[:, :1, :].expand(wl.S, wl.B, wl.H)
    assert xb.stride()[1] == 0
    gx_s, gw_s = mdc.backward(gy, xb, w, m)
    gx, gw = mdc.backward(gy, xb.contiguous(), w, m)
    torch.cuda.synchronize()
    assert torch.equal(gx_s.view(torch.int16), gx.view(torch.int16))
    assert torch.equal(gw_s.view(torch.int16), gw.view(torch.int16))


@pytest.mark.parametrize("layout", ["bsh", "gy_chstride_x_oddbase"])
def test_backward_strided_full_size(layout):
    """The headline workload with strided inputs, checked on sampled channels against the oracle
    and everywhere against the contiguous path."""
    wl = WORKLOADS[3]
    (gx_s, gw_s), (gx, gw) = run_both(wl, layout)
    assert torch.equal(gx_s.view(torch.int16), gx.view(torch.int16))
    assert torch.equal(gw_s.view(torch.int16), gw.view(torch.int16))
    del gx, gw
    compare_columns(wl, gx_s, gw_s, sample_channels(wl, n_random=8, seed=31),
                    tag=f"{wl.name} strided {layout}")
    torch.cuda.empty_cache()


FWD_LAYOUTS = {
    "bsh": as_bsh,                     # in place: row/batch strides multiples of 8
    "hslice": lambda t: as_h_slice(t, pad=64, off=32),  # in place
    "hslice_off2": lambda t: as_h_slice(t, pad=64, off=2),  # 4-byte base: packed
    "chstride": as_channel_strided,    # packed
}


@pytest.mark.parametrize("layout", list(FWD_LAYOUTS))
@pytest.mark.parametrize("shape", [(37, 3, 448, "bf16", ("bernoulli", 0.8)),
                                   (19, 2, 576, "fp16", ("null",))], ids=lambda v: str(v))
def test_forward_strided_small(layout, shape):
    S, B, H, dt, mk = shape
    wl = custom(S, B, H, dt, mk, seed=S + 3 * B)
    x = wls.full_tensor(wl, wls.STREAM_X, "cuda")
    w = wls.weight_tensor(wl, "cuda")
    m = wls.mask_tensor(wl, "cuda")
    x_s = FWD_LAYOUTS[layout](x)
    announce(f"mccb_forward_ex {wl.name} layout={layout}")
    y_s = mdc.forward(x_s, transposed_weight(w), transposed_mask(m))
    y = mdc.forward(x, w, m)
    torch.cuda.synchronize()
    fwd_compare_full(wl, y_s, tag=f"{wl.name} strided {layout}")
    assert torch.equal(y_s.view(torch.int16), y.view(torch.int16))


def test_forward_strided_full_size():
    wl = WORKLOADS[3]
    x = wls.full_tensor(wl, wls.STREAM_X, "cuda")
    w = wls.weight_tensor(wl, "cuda")
    m = wls.mask_tensor(wl, "cuda")
    xs = as_bsh(x)
    announce(f"mccb_forward_ex {wl.name} layout=bsh")
    y_s = mdc.forward(xs, w, m)
    y = mdc.forward(x, w, m)
    torch.cuda.synchronize()
    assert torch.equal(y_s.view(torch.int16), y.view(torch.int16))
    del y, xs, x
    fwd_compare_columns(wl, y_s, sample_channels(wl, n_random=8, seed=32),
                        tag=f"{wl.name} strided bsh")
    torch.cuda.empty_cache()
