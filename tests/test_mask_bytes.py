"""The mask's bytes: any nonzero byte keeps its row (the bool tensor is stored one byte per element,
and a uint8 mask may hold any nonzero value for true). Both ops must give bit for bit the same
outputs for a 0/1 mask and for the same mask with its kept bytes replaced by other nonzero values
(drawn from all 255), on each way the kernels read the mask: the forward's 8-byte words (unit row
stride, rows a multiple of 8 apart) and its byte path (S not a multiple of 8, or a strided mask),
and the backward's staging into LDS. The 0/1 results themselves are checked against the oracle by
the other tests.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import masked_depthwise_causal_amd as mdc
from synth import custom

from .gpu_util import announce, bits16, gpu_inputs

pytestmark = pytest.mark.gpu

KEEP_VALUES = torch.arange(1, 256, dtype=torch.int32).to(torch.uint8)  # every nonzero byte


def nonzero_variant(m: torch.Tensor, seed: int) -> torch.Tensor:
    """The same keep/drop pattern as `m`, each kept byte drawn from KEEP_VALUES."""
    g = torch.Generator().manual_seed(seed)
    pick = torch.randint(0, len(KEEP_VALUES), tuple(m.shape), generator=g)
    raw = torch.where(m.cpu().bool(), KEEP_VALUES[pick], torch.zeros((), dtype=torch.uint8))
    return raw.to(m.device)


def strided_copy(m: torch.Tensor) -> torch.Tensor:
    """A [B,S] view of an [S,B] tensor holding the same bytes (row stride B, not 1)."""
    return m.t().contiguous().t()


CASES = [
    # (S, B, H, dtype, strided mask)
    (64, 3, 448, "bf16", False),     # forward: every tile reads 8-byte mask words
    (61, 3, 448, "fp16", False),     # S % 8 != 0: byte path
    (1000, 2, 1024, "bf16", False),  # words, last tile partial
    (96, 4, 512, "bf16", True),      # strided mask: byte path
]


@pytest.mark.parametrize("S,B,H,dtype,strided", CASES, ids=lambda v: str(v))
def test_nonzero_bytes_equal_ones(S, B, H, dtype, strided):
    wl = custom(S, B, H, dtype, ("bernoulli", 0.6), seed=S * 7 + B)
    gy, x, w, m = gpu_inputs(wl)
    m01 = m.to(torch.uint8)
    raw = nonzero_variant(m01, seed=S + H)
    assert torch.equal(raw != 0, m01 != 0)
    if S * B >= 1000:  # enough kept bytes to see (almost) every value
        assert len(torch.unique(raw)) > 200
    if strided:
        m01, raw = strided_copy(m01), strided_copy(raw)
        assert m01.stride() == (1, B)
    announce(f"nonzero mask bytes S={S} B={B} H={H} {dtype} strided={strided}")

    y_ref = mdc.forward(x, w, m01)
    y_raw = mdc.forward(x, w, raw)
    gx_ref, gw_ref = mdc.backward(gy, x, w, m01)
    gx_raw, gw_raw = mdc.backward(gy, x, w, raw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits16(y_raw), bits16(y_ref))
    np.testing.assert_array_equal(bits16(gx_raw), bits16(gx_ref))
    np.testing.assert_array_equal(bits16(gw_raw), bits16(gw_ref))
    # and the mask took effect: some rows are dropped, so y has zero rows where m is 0
    dropped = (m01 == 0).t().cpu()  # [S, B]
    assert bool(dropped.any())
    assert torch.all(y_ref.cpu()[dropped] == 0)
