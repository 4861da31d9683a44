"""GPU parity of the forward (mccb_forward) against the CPU fp64 oracle on the same seeded inputs.

The forward y = mask * causal depthwise conv(x, w) rounds the exact three-term sum once, so the bar
is the gradX one: within 1 ulp of the oracle's correctly rounded value, and expected bit-exact.
Small shapes are compared element by element; the full-size workloads, in the launch configuration
the benchmark times, on every element of sampled channels and of sampled rows. Inputs come from
the same generator streams the backward uses for x and the weight.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import masked_depthwise_causal_amd as mdc
import oracle
from synth import WORKLOADS, custom
from synth import workloads as wls

from .gpu_util import announce, bits16, check_gradx

pytestmark = pytest.mark.gpu


def fplan(wl):
    return mdc.mccb_get_plan(wl.S, wl.B, wl.H, mdc.MCCB_BF16 if wl.dtype == "bf16" else mdc.MCCB_FP16)


def gpu_forward(wl, inputs=None, poison=False):
    if inputs is None:
        announce(f"generate {wl.name} (x, w, mask) on cuda")
        inputs = (wls.full_tensor(wl, wls.STREAM_X, "cuda"), wls.weight_tensor(wl, "cuda"),
                  wls.mask_tensor(wl, "cuda"))
    x, w, m = inputs
    y = torch.empty_like(x)
    if poison:
        y.view(torch.int16).fill_(0x7F80 if wl.dtype == "bf16" else 0x7C00)  # +inf everywhere
    announce(f"mccb_forward {wl.name} S={wl.S} B={wl.B} H={wl.H} W={wl.W} {wl.dtype} "
             f"mask={wl.mask[0]}")
    mdc.forward(x, w, m, y=y)
    torch.cuda.synchronize()
    return y


def oracle_forward(wl, x_bits, w_bits, m):
    return oracle.get().forward16(wl.dtype, x_bits, w_bits, None if m is None else m.numpy())


def compare_full(wl, y, tag=None):
    inp = wls.host_inputs(wl)
    ref = oracle_forward(wl, wls.bits(inp["x"]), wls.bits(inp["w"]), inp["mask"])
    check_gradx(bits16(y), ref["y16"], (tag or wl.name) + " forward")


def compare_columns(wl, y, hs, tag=None):
    """Every element of the channels `hs`: the [S,B,len(hs)] slice of x holds all they depend on."""
    hs_t = torch.from_numpy(hs)
    x_c = wls.bits(wls.column_tensor(wl, wls.STREAM_X, hs_t))
    w_c = wls.bits(wls.weight_tensor(wl, "cpu")[:, hs_t])
    ref = oracle_forward(wl, x_c, w_c, wls.mask_tensor(wl, "cpu"))
    got = bits16(y.index_select(2, hs_t.to(y.device)))
    check_gradx(got, ref["y16"], (tag or wl.name) + " forward (columns)")


def compare_rows(wl, y, rows, tag=None):
    """Whole output rows: row i depends on x rows i-W+1..i (fewer at the start) and mask row i."""
    m = wls.mask_tensor(wl, "cpu")
    w = wls.bits(wls.weight_tensor(wl, "cpu"))
    for r in rows:
        r = int(r)
        lo = max(r - (wl.W - 1), 0)
        rr = torch.arange(lo, r + 1, dtype=torch.int64)
        x_r = wls.bits(wls.row_tensor(wl, wls.STREAM_X, rr))
        m_r = None if m is None else m[:, lo:r + 1].contiguous()
        ref = oracle_forward(wl, x_r, w, m_r)
        check_gradx(bits16(y[r]), ref["y16"][-1], f"{tag or wl.name} forward (row {r})")


def sample_channels(wl, n_random=16, seed=0):
    H = wl.H
    rng = np.random.default_rng(seed)
    edges = [0, 1, 3, 4, 5, 7, 8, 255, 256, 511, 512, 2047, 2048, H // 2, H - 5, H - 4, H - 1]
    hs = set(h for h in edges if 0 <= h < H)
    hs.update(int(h) for h in rng.integers(0, H, n_random))
    return np.array(sorted(hs), dtype=np.int64)


def sample_rows(wl, plan, n_random=6, seed=1):
    S, R = wl.S, plan["fwd_rows_per_tile"]
    rng = np.random.default_rng(seed)
    cand = {0, 1, 2, 3, R - 2, R - 1, R, R + 1, R + 2, 2 * R - 1, 2 * R, S - 3, S - 2, S - 1}
    cand.update(int(r) for r in rng.integers(0, S, n_random))
    return np.array(sorted(r for r in cand if 0 <= r < S), dtype=np.int64)


def test_small_workload_full():
    wl = WORKLOADS[0]  # S=64 B=1 H=384 bf16, Bernoulli(0.8) mask
    compare_full(wl, gpu_forward(wl))


EDGE = [
    # (S, B, H, dtype, mask): S around the row tile, B*H below, at and past the column tile
    # (2048 columns by default), every mask kind
    (1, 2, 384, "bf16", ("bernoulli", 0.8)),
    (2, 1, 384, "fp16", ("null",)),
    (3, 3, 448, "bf16", ("prefix",)),
    (7, 2, 384, "fp16", ("bernoulli", 0.5)),
    (8, 1, 512, "bf16", ("all_true",)),
    (9, 4, 512, "bf16", ("bernoulli", 0.9)),
    (10, 5, 576, "fp16", ("null",)),
    (17, 3, 448, "bf16", ("bernoulli", 0.7)),
    (63, 2, 384, "bf16", ("prefix",)),
    (100, 7, 640, "fp16", ("bernoulli", 0.8)),
    (33, 1, 24576, "bf16", ("null",)),
    (5, 32, 24576, "fp16", ("bernoulli", 0.6)),
    (16, 32, 384, "bf16", ("all_false",)),
    (1000, 2, 1024, "bf16", ("bernoulli", 0.9)),
    (12, 8, 512, "bf16", ("bernoulli", 0.8)),
    (21, 5, 832, "fp16", ("prefix",)),
    # narrow rows: the block's waves stack along the rows (1, 2 or 4 across)
    (70, 1, 1024, "bf16", ("bernoulli", 0.8)),
    (100, 1, 2048, "fp16", ("null",)),
    (33, 1, 5120, "bf16", ("bernoulli", 0.9)),
    (65, 1, 384, "bf16", ("prefix",)),
    (3, 1, 5120, "fp16", ("null",)),
    # rows an odd number of 64 KiB (64, 192, 320 KiB): a block's 4 waves take chunks 16 KiB apart
    (40, 8, 4096, "bf16", ("bernoulli", 0.8)),
    (13, 6, 16384, "fp16", ("prefix",)),
    (9, 32, 5120, "bf16", ("bernoulli", 0.9)),
]


@pytest.mark.parametrize("S,B,H,dtype,mask", EDGE, ids=lambda v: str(v))
def test_edge_shapes_full(S, B, H, dtype, mask):
    m = ("bernoulli", 0.0) if mask[0] == "all_false" else mask
    wl = custom(S, B, H, dtype, m, seed=S * 17 + B)
    compare_full(wl, gpu_forward(wl, poison=True))


def test_subnormal_outputs_full():
    cases = [custom(40, 2, 384, "fp16", ("bernoulli", 0.8), seed=11, x=("normal", 1e-3),
                    w=("normal", 1e-2)),
             custom(40, 2, 384, "bf16", ("bernoulli", 0.8), seed=12, x=("normal", 2.0 ** -120),
                    w=("normal", 2.0 ** -12))]
    for wl in cases:
        compare_full(wl, gpu_forward(wl), tag=wl.name + " subnormal")


@pytest.mark.parametrize("idx", [1, 2, 3, 4], ids=lambda i: WORKLOADS[i].name)
def test_full_size_workload_sampled(idx):
    wl = WORKLOADS[idx]
    inputs = (wls.full_tensor(wl, wls.STREAM_X, "cuda"), wls.weight_tensor(wl, "cuda"),
              wls.mask_tensor(wl, "cuda"))
    y = gpu_forward(wl, inputs)
    announce(f"compare {wl.name} forward: sampled channels")
    compare_columns(wl, y, sample_channels(wl, seed=idx))
    announce(f"compare {wl.name} forward: sampled rows")
    compare_rows(wl, y, sample_rows(wl, fplan(wl), seed=idx))
    y2 = gpu_forward(wl, inputs, poison=True)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    del y, y2, inputs
    torch.cuda.empty_cache()


def test_null_mask_equals_all_true():
    wl = custom(50, 3, 448, "bf16", ("null",), seed=5)
    x, w = wls.full_tensor(wl, wls.STREAM_X, "cuda"), wls.weight_tensor(wl, "cuda")
    y0 = mdc.forward(x, w, None)
    y1 = mdc.forward(x, w, torch.ones((3, 50), dtype=torch.bool, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


def test_output_canaries_untouched():
    """The kernel writes y and nothing next to it (lanes past B*H and rows past S store nothing)."""
    wl = custom(19, 3, 448, "fp16", ("bernoulli", 0.8), seed=23)
    x, w, m = (wls.full_tensor(wl, wls.STREAM_X, "cuda"), wls.weight_tensor(wl, "cuda"),
               wls.mask_tensor(wl, "cuda"))
    n = x.numel()
    buf = torch.full((n + 2 * 4096,), 12345, dtype=torch.int16, device="cuda")
    y = buf[4096:4096 + n].view(torch.float16).view(x.shape)
    mdc.forward(x, w, m, y=y)
    torch.cuda.synchronize()
    assert torch.all(buf[:4096] == 12345) and torch.all(buf[4096 + n:] == 12345)
    compare_full(wl, y)
