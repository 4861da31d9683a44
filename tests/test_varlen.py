"""GPU parity of the packed variable-length layout (mccb_varlen_backward / mccb_varlen_forward)
against the oracle's packed-layout functions on the same seeded values.

Packed inputs are the valid tokens of a padded seeded workload, gathered in sequence order; the
oracle receives the same tokens from the CPU generator. Bars as for the padded layout: gradX and y
within 1 ulp of the oracle's correctly rounded value (expected bit-exact), gradWeight within the
relative bar and 1 ulp of the oracle's rounding. The padded path with the prefix mask computes the
same gradX on the valid tokens, which is checked bit for bit as well.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import masked_depthwise_causal_amd as mdc
import oracle
from synth import WORKLOADS, custom
from synth import workloads as wls

from .gpu_util import announce, bits16, check_gradw, check_gradx

pytestmark = pytest.mark.gpu


def packed_inputs(wl, lengths, device, token_mask_p=None):
    """gY, x packed [T,H], weight [W,H], cu_seqlens, optional per-token mask [T]."""
    gy = wls.pack_tokens(wls.full_tensor(wl, wls.STREAM_GY, device), lengths)
    x = wls.pack_tokens(wls.full_tensor(wl, wls.STREAM_X, device), lengths)
    w = wls.weight_tensor(wl, device)
    cu = wls.cu_seqlens(lengths, device)
    m = None
    if token_mask_p is not None:
        T = int(sum(int(v) for v in lengths))
        g = torch.Generator().manual_seed(wl.seed)
        m = (torch.rand(T, generator=g) < token_mask_p).to(torch.uint8).to(device)
    return gy, x, w, cu, m


def oracle_backward(wl, lengths, gy, x, w, m, cols=None):
    cu = wls.cu_seqlens(lengths).numpy()
    g, xx, ww = wls.bits(gy.cpu()), wls.bits(x.cpu()), wls.bits(w.cpu())
    if cols is not None:
        g, xx, ww = g[:, cols], xx[:, cols], ww[:, cols]
    return oracle.get().backward_varlen(wl.dtype, g, xx, ww, cu,
                                        None if m is None else m.cpu().numpy(), want_gx64=False)


def oracle_forward(wl, lengths, x, w, m, cols=None):
    cu = wls.cu_seqlens(lengths).numpy()
    xx, ww = wls.bits(x.cpu()), wls.bits(w.cpu())
    if cols is not None:
        xx, ww = xx[:, cols], ww[:, cols]
    return oracle.get().forward16_varlen(wl.dtype, xx, ww, cu,
                                         None if m is None else m.cpu().numpy())


CASES = [
    # (lengths, H, dtype, W, token mask probability)
    ([5, 1, 3], 384, "bf16", 3, None),
    ([7], 448, "fp16", 3, 0.8),
    ([2, 0, 6, 4, 1], 384, "bf16", 3, None),
    ([1] * 40, 384, "bf16", 3, None),
    ([3, 0, 0, 2, 9, 17, 33, 1], 576, "fp16", 4, 0.7),
    ([100, 37, 250, 64], 640, "bf16", 2, 0.9),
    ([1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17], 384, "bf16", 4, None),
    ([1000, 1500, 700], 1024, "bf16", 3, 0.85),
    ([129, 4], 384, "fp16", 1, None),
]


@pytest.mark.parametrize("lengths,H,dtype,W,p", CASES, ids=lambda v: str(v)[:40])
def test_varlen_small_full(lengths, H, dtype, W, p):
    S, B = max(max(lengths), 1), len(lengths)
    wl = custom(S, B, H, dtype, ("null",), seed=sum(lengths) + 7 * W, W=W)
    gy, x, w, cu, m = packed_inputs(wl, lengths, "cuda", p)
    T = int(sum(lengths))
    announce(f"mccb_varlen_backward T={T} nseq={B} H={H} W={W} {dtype}")
    gx, gw = mdc.varlen_backward(gy, x, w, cu, m)
    announce(f"mccb_varlen_forward T={T} nseq={B} H={H} W={W} {dtype}")
    y = mdc.varlen_forward(x, w, cu, m)
    torch.cuda.synchronize()
    ref = oracle_backward(wl, lengths, gy, x, w, m)
    check_gradx(bits16(gx), ref["gx16"], f"varlen {lengths} gradX")
    check_gradw(bits16(gw), ref, dtype, f"varlen {lengths} gradWeight")
    refy = oracle_forward(wl, lengths, x, w, m)
    check_gradx(bits16(y), refy["y16"], f"varlen {lengths} forward")


@pytest.mark.parametrize("W", [2, 3, 4])
def test_varlen_sequence_starts_at_every_tile_offset(W):
    """Sequence starts at every offset inside a wave's 8-row tile (and on tile edges), with
    lengths around the look-back: the forward takes the unlimited form only for tiles whose last
    row has at least 7 + W - 1 earlier rows in its sequence, and clears the window at each start."""
    lengths = []
    for off in range(8):
        lengths += [8 + off, 1, W - 1, W, 16 - off]
    lengths = [v for v in lengths if v > 0]
    H = 640
    wl = custom(max(lengths), len(lengths), H, "bf16", ("null",), seed=900 + W, W=W)
    gy, x, w, cu, m = packed_inputs(wl, lengths, "cuda", 0.9)
    T = int(sum(lengths))
    announce(f"mccb_varlen_forward/backward tile offsets T={T} nseq={len(lengths)} W={W}")
    gx, gw = mdc.varlen_backward(gy, x, w, cu, m)
    y = mdc.varlen_forward(x, w, cu, m)
    torch.cuda.synchronize()
    ref = oracle_backward(wl, lengths, gy, x, w, m)
    check_gradx(bits16(gx), ref["gx16"], f"tile offsets W={W} gradX")
    check_gradw(bits16(gw), ref, "bf16", f"tile offsets W={W} gradWeight")
    refy = oracle_forward(wl, lengths, x, w, m)
    check_gradx(bits16(y), refy["y16"], f"tile offsets W={W} forward")


def test_varlen_matches_padded_prefix_mask():
    """Packed layout vs the padded layout with each batch's mask cut at its length: the same
    gradX on the valid tokens, bit for bit (both are correctly rounded)."""
    wl = custom(600, 6, 448, "bf16", ("prefix",), seed=44)
    lengths = wls.varlen_lengths(wl)
    gy_p = wls.full_tensor(wl, wls.STREAM_GY, "cuda")
    x_p = wls.full_tensor(wl, wls.STREAM_X, "cuda")
    w = wls.weight_tensor(wl, "cuda")
    m_p = wls.mask_tensor(wl, "cuda")
    gx_p, gw_p = mdc.backward(gy_p, x_p, w, m_p)
    y_p = mdc.forward(x_p, w, m_p)
    gy, x = wls.pack_tokens(gy_p, lengths), wls.pack_tokens(x_p, lengths)
    cu = wls.cu_seqlens(lengths, "cuda")
    gx, gw = mdc.varlen_backward(gy, x, w, cu)
    y = mdc.varlen_forward(x, w, cu)
    torch.cuda.synchronize()
    assert torch.equal(gx.view(torch.int16), wls.pack_tokens(gx_p, lengths).view(torch.int16))
    assert torch.equal(y.view(torch.int16), wls.pack_tokens(y_p, lengths).view(torch.int16))
    ref = oracle_backward(wl, lengths, gy, x, w, None)
    check_gradw(bits16(gw), ref, "bf16", "varlen vs padded: varlen gradWeight")
    check_gradw(bits16(gw_p), ref, "bf16", "varlen vs padded: padded gradWeight")


def test_varlen_repeat_bit_identical():
    wl = custom(900, 5, 512, "fp16", ("null",), seed=3)
    lengths = [900, 3, 450, 0, 77]
    gy, x, w, cu, m = packed_inputs(wl, lengths, "cuda", 0.9)
    ws = torch.full((mdc.mccb_varlen_get_workspace_size(sum(lengths), 5, 512, 3, 1),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    a = mdc.varlen_backward(gy, x, w, cu, m, workspace=ws)
    a = (a[0].clone(), a[1].clone())
    ws.fill_(0x5A)
    b = mdc.varlen_backward(gy, x, w, cu, m, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))


def _sample_rows(lengths, n_random=8, seed=0):
    """Tokens at and around sequence starts and ends, plus random ones."""
    cu = np.cumsum(lengths)
    T = int(cu[-1])
    rows = set()
    for e in [0] + list(cu):
        for d in (-3, -2, -1, 0, 1, 2):
            if 0 <= e + d < T:
                rows.add(int(e + d))
    rows.update(int(r) for r in np.random.default_rng(seed).integers(0, T, n_random))
    return sorted(rows)


@pytest.mark.parametrize("W", [3, 4])
def test_varlen_full_size_sampled(W):
    """The headline shape's tokens packed: 32 sequences with lengths uniform in [S/2, S] for
    S = 16384, H = 5120, bf16 (about 393K tokens)."""
    wl = wls.with_taps(WORKLOADS[3], W)
    lengths = wls.varlen_lengths(wl)
    T = int(lengths.sum())
    gy_p = wls.full_tensor(wl, wls.STREAM_GY, "cuda")
    gy = wls.pack_tokens(gy_p, lengths)
    del gy_p
    x_p = wls.full_tensor(wl, wls.STREAM_X, "cuda")
    x = wls.pack_tokens(x_p, lengths)
    del x_p
    w = wls.weight_tensor(wl, "cuda")
    cu = wls.cu_seqlens(lengths, "cuda")
    announce(f"mccb_varlen_backward T={T} nseq=32 H=5120 W={W}")
    gx, gw = mdc.varlen_backward(gy, x, w, cu)
    y = mdc.varlen_forward(x, w, cu)
    torch.cuda.synchronize()
    # every element of sampled channels
    rng = np.random.default_rng(W)
    cols = np.array(sorted({0, 1, 7, 8, 511, 512, 2047, 2048, 5119} |
                           set(int(c) for c in rng.integers(0, 5120, 6))))
    cols_t = torch.from_numpy(cols).cuda()
    announce("compare sampled channels")
    ref = oracle_backward(wl, lengths, gy.index_select(1, cols_t), x.index_select(1, cols_t),
                          w.index_select(1, cols_t), None)
    check_gradx(bits16(gx.index_select(1, cols_t)), ref["gx16"], "varlen full gradX columns")
    check_gradw(bits16(gw.index_select(1, cols_t)), ref, wl.dtype, "varlen full gradWeight")
    refy = oracle_forward(wl, lengths, x.index_select(1, cols_t), w.index_select(1, cols_t), None)
    check_gradx(bits16(y.index_select(1, cols_t)), refy["y16"], "varlen full forward columns")
    # whole rows at and around sequence boundaries: the oracle runs on each row's slab
    announce("compare sampled rows")
    cu_np = np.cumsum(lengths.numpy())
    for t in _sample_rows(lengths.numpy(), seed=W):
        b = int(np.searchsorted(cu_np, t, side="right"))
        start, end = (0 if b == 0 else int(cu_np[b - 1])), int(cu_np[b])
        hi = min(t + W, end)
        r = oracle.get().backward_varlen(wl.dtype, wls.bits(gy[t:hi].cpu()),
                                         wls.bits(x[t:hi].cpu()), wls.bits(w.cpu()),
                                         np.array([hi - t]), None, want_gx64=False)
        check_gradx(bits16(gx[t:t + 1]), r["gx16"][:1], f"varlen gradX row {t}")
        lo = max(t - W + 1, start)
        ry = oracle.get().forward16_varlen(wl.dtype, wls.bits(x[lo:t + 1].cpu()),
                                           wls.bits(w.cpu()), np.array([t + 1 - lo]), None)
        check_gradx(bits16(y[t:t + 1]), ry["y16"][-1:], f"varlen forward row {t}")
    del gy, x, gx, gw, y
    torch.cuda.empty_cache()
