"""Seeded random cases across every path: shape, dtype, mask kind, window W, input layout
(contiguous, [B,S,H]-stored, an H-slice of a wider tensor, or channels 2 apart, which the library
packs first), and the packed variable-length layout. Each case runs the backward and the forward
through the binding and compares with the CPU oracle on the same seeded values: gradX and y bit for
bit (within the 1-ulp bar, expected exact), gradWeight within the relative bar and 1 ulp of the
oracle's rounding. The cases are drawn once from a fixed seed, so a failure names a reproducible
case.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import masked_depthwise_causal_amd as mdc
from synth import custom

from .gpu_util import announce, bits16, check_gradw, check_gradx, compare_full, gpu_inputs
from .test_forward import compare_full as fwd_compare_full
from .test_strided import as_bsh, as_channel_strided, as_h_slice
from .test_varlen import oracle_backward, oracle_forward, packed_inputs

pytestmark = pytest.mark.gpu

LAYOUTS = {
    "contiguous": lambda t: t,
    "bsh": as_bsh,
    "hslice": lambda t: as_h_slice(t, pad=128, off=64),
    "chstride": as_channel_strided,
}


def _draw_cases(n: int, seed: int) -> list:
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        S = int(rng.integers(1, 41)) if rng.random() < 0.4 else int(rng.integers(41, 700))
        B = int(rng.integers(1, 7))
        H = 64 * int(rng.integers(6, 21))
        dtype = "bf16" if rng.random() < 0.6 else "fp16"
        kind = rng.choice(["null", "all_true", "bernoulli", "prefix"])
        mask = ("bernoulli", float(rng.uniform(0.3, 0.95))) if kind == "bernoulli" else (str(kind),)
        W = int(rng.integers(1, 5))
        layout = str(rng.choice(list(LAYOUTS)))
        cases.append((i, S, B, H, dtype, mask, W, layout))
    return cases


CASES = _draw_cases(80, seed=20261202)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"case{c[0]}-S{c[1]}-B{c[2]}-H{c[3]}-"
                                                       f"{c[4]}-{c[5][0]}-W{c[6]}-{c[7]}")
def test_random_case(case):
    i, S, B, H, dtype, mask, W, layout = case
    wl = custom(S, B, H, dtype, mask, seed=5000 + i, W=W)
    gy, x, w, m = gpu_inputs(wl)
    f = LAYOUTS[layout]
    gy_l, x_l = f(gy), f(x)
    announce(f"random case {i}: backward/forward S={S} B={B} H={H} {dtype} mask={mask[0]} "
             f"W={W} layout={layout}")
    gx, gw = mdc.backward(gy_l, x_l, w, m)
    y = mdc.forward(x_l, w, m)
    torch.cuda.synchronize()
    compare_full(wl, gx, gw, tag=f"random case {i}")
    fwd_compare_full(wl, y, tag=f"random case {i}")


def _draw_varlen(n: int, seed: int) -> list:
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        nseq = int(rng.integers(1, 12))
        lengths = [int(v) for v in rng.integers(0, 90, nseq)]
        if rng.random() < 0.3:
            lengths[int(rng.integers(0, nseq))] = int(rng.integers(200, 600))
        if sum(lengths) == 0:
            lengths[0] = 1
        H = 64 * int(rng.integers(6, 17))
        dtype = "bf16" if rng.random() < 0.6 else "fp16"
        W = int(rng.integers(1, 5))
        p = None if rng.random() < 0.5 else float(rng.uniform(0.5, 0.95))
        cases.append((i, lengths, H, dtype, W, p))
    return cases


VARLEN_CASES = _draw_varlen(24, seed=777)


@pytest.mark.parametrize("case", VARLEN_CASES,
                         ids=lambda c: f"varlen{c[0]}-n{len(c[1])}-T{sum(c[1])}-H{c[2]}-W{c[4]}")
def test_random_varlen_case(case):
    i, lengths, H, dtype, W, p = case
    S, B = max(max(lengths), 1), len(lengths)
    wl = custom(S, B, H, dtype, ("null",), seed=9000 + i, W=W)
    gy, x, w, cu, m = packed_inputs(wl, lengths, "cuda", p)
    announce(f"random varlen case {i}: T={sum(lengths)} nseq={B} H={H} {dtype} W={W}")
    gx, gw = mdc.varlen_backward(gy, x, w, cu, m)
    y = mdc.varlen_forward(x, w, cu, m)
    torch.cuda.synchronize()
    ref = oracle_backward(wl, lengths, gy, x, w, m)
    check_gradx(bits16(gx), ref["gx16"], f"random varlen case {i} gradX")
    check_gradw(bits16(gw), ref, dtype, f"random varlen case {i} gradWeight")
    refy = oracle_forward(wl, lengths, x, w, m)
    check_gradx(bits16(y), refy["y16"], f"random varlen case {i} forward")
