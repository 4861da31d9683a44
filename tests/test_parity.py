"""GPU parity: the HIP path against the CPU fp64 oracle on the same seeded inputs.

Bars (stated in the tests): gradX within 1 ulp of the oracle's correctly rounded value (and, by
design, bit-exact); gradWeight within relative error 8e-3 (bf16) / 1e-3 (fp16) of the oracle's exact
fp64 value (and, by design, equal to its rounding up to 1 ulp). Small shapes are compared element by
element; the full-size workloads are compared whole in test_full_parity.py, and the longest sequence
(S=524288, B=1) here on every element of sampled channels and of sampled rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import masked_depthwise_causal_amd as mdc
from synth import WORKLOADS, custom
from synth import workloads as wls

from .gpu_util import (announce, bits16, compare_columns, compare_full, compare_rows, gpu_inputs,
                       gpu_run, sample_channels, sample_rows)

pytestmark = pytest.mark.gpu


def plan_of(wl):
    return mdc.mccb_get_plan(wl.S, wl.B, wl.H, mdc.MCCB_BF16 if wl.dtype == "bf16" else mdc.MCCB_FP16)


def test_small_workload_full():
    wl = WORKLOADS[0]  # S=64 B=1 H=384 bf16, Bernoulli(0.8) mask
    gx, gw = gpu_run(wl)
    compare_full(wl, gx, gw)


def test_call_example_all_zero():
    # the page's call example: S=1, B=2, H=384, FLOAT16, every input and the mask zero
    S, B, H = 1, 2, 384
    z = torch.zeros((S, B, H), dtype=torch.float16, device="cuda")
    w = torch.zeros((3, H), dtype=torch.float16, device="cuda")
    m = torch.zeros((B, S), dtype=torch.uint8, device="cuda")
    gx = torch.full_like(z, 7.0)
    gw = torch.full_like(w, 7.0)
    announce("call example S=1 B=2 H=384 fp16 zeros")
    mdc.backward(z, z.clone(), w, m, gradX=gx, gradWeight=gw)
    torch.cuda.synchronize()
    assert torch.all(gx == 0) and torch.all(gw == 0)


EDGE = [
    # (S, B, H, dtype, mask)
    (1, 2, 384, "bf16", ("bernoulli", 0.8)),
    (2, 2, 384, "bf16", ("null",)),
    (3, 3, 384, "fp16", ("bernoulli", 0.5)),
    (4, 1, 384, "bf16", ("all_true",)),
    (5, 2, 448, "fp16", ("prefix",)),
    (63, 1, 384, "bf16", ("bernoulli", 0.9)),
    (64, 1, 384, "bf16", ("bernoulli", 0.9)),
    (65, 1, 384, "bf16", ("bernoulli", 0.9)),
    (66, 3, 640, "bf16", ("bernoulli", 0.7)),
    (255, 2, 384, "fp16", ("null",)),
    (256, 2, 384, "bf16", ("bernoulli", 0.6)),
    (257, 2, 448, "bf16", ("prefix",)),
    (258, 5, 384, "fp16", ("bernoulli", 0.9)),
    (513, 3, 576, "bf16", ("null",)),
    (1000, 7, 448, "bf16", ("bernoulli", 0.8)),
    (16, 32, 384, "bf16", ("bernoulli", 0.5)),
    (16, 32, 384, "fp16", ("all_false",)),
    (8, 1, 24576, "bf16", ("bernoulli", 0.9)),
    (3, 2, 24576, "fp16", ("null",)),
    (4, 32, 24576, "bf16", ("bernoulli", 0.7)),  # the widest row: B*H = 786432
]


@pytest.mark.parametrize("S,B,H,dtype,mask", EDGE, ids=lambda v: str(v))
def test_edge_shapes_full(S, B, H, dtype, mask):
    if mask[0] == "all_false":
        wl = custom(S, B, H, dtype, ("bernoulli", 0.0), seed=S * 31 + B)
    else:
        wl = custom(S, B, H, dtype, mask, seed=S * 31 + B)
    gx, gw = gpu_run(wl, poison_workspace=True)
    compare_full(wl, gx, gw)


def test_tile_boundaries_full():
    """S on and around the strip and wave-run boundaries the plan picks for this shape."""
    B, H = 2, 384
    base = mdc.mccb_get_plan(4096, B, H, mdc.MCCB_BF16)
    R, Q = base["rows_per_turn"], base["rows_per_round"]
    cases = {R - 1, R + 1, R + 2, Q - 1, Q, Q + 1, Q + 2, 2 * Q + 3}
    for S in sorted(cases):
        # the strip length follows S; also check S just around the strip of a longer tensor
        wl = custom(S, B, H, "bf16", ("bernoulli", 0.85), seed=S)
        gx, gw = gpu_run(wl)
        compare_full(wl, gx, gw, tag=f"S={S} (turn {R}, round {Q})")
    T = base["rows_per_strip"]
    for S in (4096, T + 1, T + R + 3):
        wl = custom(S, B, H, "bf16", ("bernoulli", 0.85), seed=S + 1)
        p = mdc.mccb_get_plan(S, B, H, mdc.MCCB_BF16)
        gx, gw = gpu_run(wl)
        compare_full(wl, gx, gw, tag=f"S={S} (strip {p['rows_per_strip']} x {p['n_strips']})")


def test_subnormal_outputs_full():
    # results in the subnormal range of each format must still be correctly rounded
    cases = [custom(70, 2, 384, "fp16", ("bernoulli", 0.8), seed=5, gy=("normal", 2e-3),
                    x=("normal", 1e-3), w=("normal", 1e-2)),
             custom(70, 2, 384, "bf16", ("bernoulli", 0.8), seed=6, gy=("normal", 2.0 ** -118),
                    x=("normal", 2.0 ** -10), w=("normal", 2.0 ** -12))]
    for wl in cases:
        gx, gw = gpu_run(wl)
        compare_full(wl, gx, gw, tag=wl.name + " subnormal")


def test_generator_same_bits_on_gpu_and_cpu():
    """The oracle regenerates its inputs on the CPU: check the GPU-generated tensors agree."""
    wl = WORKLOADS[3]
    small = custom(64, 4, 512, "bf16", ("bernoulli", 0.9), seed=wl.seed)
    g_gpu = wls.full_tensor(small, wls.STREAM_GY, "cuda").cpu()
    g_cpu = wls.full_tensor(small, wls.STREAM_GY, "cpu")
    assert torch.equal(g_gpu.view(torch.int16), g_cpu.view(torch.int16))
    hs = torch.tensor([0, 5, 511])
    assert torch.equal(wls.column_tensor(small, wls.STREAM_GY, hs).view(torch.int16),
                       g_cpu[:, :, hs].contiguous().view(torch.int16))


def test_max_sequence_length_sampled():
    """The longest sequence the constraints allow (B*S = 524288 with B = 1), narrowest H."""
    wl = custom(524288, 1, 384, "bf16", ("bernoulli", 0.9), seed=524)
    inputs = gpu_inputs(wl)
    gx, gw = gpu_run(wl, inputs)
    hs = sample_channels(wl, n_random=6, seed=5)
    announce(f"compare {wl.name}: sampled channels")
    compare_columns(wl, gx, gw, hs)
    compare_rows(wl, gx, sample_rows(wl, plan_of(wl), seed=5))
    del gx, gw
    from .test_forward import compare_columns as fwd_columns
    from .test_forward import gpu_forward
    y = gpu_forward(wl, (inputs[1], inputs[2], inputs[3]))
    fwd_columns(wl, y, hs)


@pytest.mark.parametrize("S,dtype,mask", [(64, "bf16", ("bernoulli", 0.8)), (37, "fp16", ("null",)),
                                          (128, "bf16", ("prefix",)), (1, "bf16", ("null",))])
def test_direct_gradweight_equals_two_kernel_path(S, dtype, mask):
    """One strip of one batch: the fused kernel writes gradWeight itself (no reduction kernel, no
    workspace). The same values as batch 0 of a two-batch problem whose batch 1 has gradY = 0 (so
    adds nothing) run the two-kernel path with the same per-column sums: gradX of batch 0 and
    gradWeight must be the same bits."""
    H = 448
    one = custom(S, 1, H, dtype, mask, seed=S + 1)
    assert mdc.mccb_get_workspace_size(S, 1, H, mdc.DTYPE_CODE[torch.bfloat16]) == 0
    assert mdc.mccb_get_workspace_size(S, 2, H, mdc.DTYPE_CODE[torch.bfloat16]) > 0
    gy, x, w, m = gpu_inputs(one)
    gy2 = torch.cat([gy, torch.zeros_like(gy)], dim=1).contiguous()
    x2 = torch.cat([x, x.flip(0)], dim=1).contiguous()
    m2 = None if m is None else torch.cat([m, torch.ones_like(m)], dim=0).contiguous()
    announce(f"direct path S={S} B=1 {dtype}")
    gx1, gw1 = mdc.backward(gy, x, w, m)
    announce(f"two-kernel path S={S} B=2 {dtype}")
    gx2, gw2 = mdc.backward(gy2, x2, w, m2)
    torch.cuda.synchronize()
    assert torch.equal(gw1.view(torch.int16), gw2.view(torch.int16))
    assert torch.equal(gx1[:, 0].view(torch.int16), gx2[:, 0].view(torch.int16))
    compare_full(one, gx1, gw1, tag=f"direct S={S}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_gradx_double_rounding_cases(dtype):
    """gradX sums built to sit just beside a midpoint between two neighbouring values of the
    format, closer than fp32 resolves: rounding to fp32 first lands exactly on the midpoint, and a
    second round-to-nearest-even would then go the wrong way for sums just above it. Compared with
    the oracle's correctly rounded values, and checked against the expected bits directly."""
    import oracle

    orc = oracle.get()
    S, B, H = 4, 1, 384
    # the sum at row 0 is gy0*w2 + gy1*w1 + gy2*w0 = 1 + half an ulp of the format at 1 + d
    half = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    tiny, wscale = (2.0 ** -40, 1.0) if dtype == "bf16" else (2.0 ** -20, 2.0 ** -20)
    gy = np.zeros((S, B, H))
    w = np.ones((3, H))
    sign = np.where(np.arange(H) % 2 == 0, 1.0, -1.0)      # the sum's sign
    d_sign = np.where(np.arange(H) % 4 < 2, 1.0, -1.0)     # d above or below the midpoint
    d_zero = np.arange(H) % 8 == 7                         # d = 0: an exact midpoint
    gy[0, 0] = sign
    gy[1, 0] = sign * half
    gy[2, 0] = np.where(d_zero, 0.0, sign * d_sign * tiny)
    w[0] = wscale  # gy2 meets w[0]
    x = np.ones((S, B, H))
    gy16, x16, w16 = (orc.encode(dtype, a) for a in (gy, x, w))
    assert np.array_equal(orc.decode(dtype, gy16), gy) and np.array_equal(orc.decode(dtype, w16), w)
    acc = np.zeros((3, H))
    ref = orc.backward_rows(dtype, S, 0, S, gy16, x16, w16, None, acc)
    one = 0x3F80 if dtype == "bf16" else 0x3C00
    up = np.where(d_zero, one, np.where(d_sign > 0, one + 1, one))  # magnitude bits of row 0
    assert np.array_equal(ref[0, 0] & 0x7FFF, up.astype(np.uint16))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    to_dev = lambda a: torch.from_numpy(a.astype(np.int16)).view(tdt).to("cuda")  # noqa: E731
    announce(f"mccb_backward double-rounding cases {dtype}")
    gx, _ = mdc.backward(to_dev(gy16), to_dev(x16), to_dev(w16), None)
    torch.cuda.synchronize()
    got = gx.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} gradX elements differ"
