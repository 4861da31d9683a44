"""Helpers shared by the GPU tests: run the HIP path, run the oracle on the same seeded inputs, and
compare. The oracle side regenerates its inputs on the CPU from the counter-based generator; it never
reads a value produced by the HIP library."""
from __future__ import annotations

import sys

import numpy as np
import torch

import masked_depthwise_causal_amd as mdc
import oracle
from synth import workloads as wls

RTOL = {"bf16": 8e-3, "fp16": 1e-3}  # gradWeight relative-error bar per dtype
# Spacing of the subnormal range of each dtype. A relative bar cannot hold for results below the
# smallest normal number (even the correctly rounded value misses it), so there the bound is one
# subnormal step.
SUBNORMAL_STEP = {"bf16": 2.0 ** -133, "fp16": 2.0 ** -24}


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def ordered(bits: np.ndarray) -> np.ndarray:
    """Map 16-bit float patterns to integers whose difference counts ulps (+0 and -0 both 0)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_dist(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ordered(a) - ordered(b))


def gpu_inputs(wl, device="cuda"):
    announce(f"generate {wl.name} on {device}")
    gy = wls.full_tensor(wl, wls.STREAM_GY, device)
    x = wls.full_tensor(wl, wls.STREAM_X, device)
    w = wls.weight_tensor(wl, device)
    m = wls.mask_tensor(wl, device)
    return gy, x, w, m


def workspace_for(wl, gy, x, w):
    """Workspace of the call the binding makes for these tensors (plain or extended)."""
    if wl.W == 3:
        return mdc.workspace_for(wl.S, wl.B, wl.H, gy.dtype, gy.device)
    n = mdc.mccb_get_workspace_size_ex(gy.data_ptr(), x.data_ptr(), w.data_ptr(), wl.S, wl.B,
                                       wl.H, wl.W, mdc.DTYPE_CODE[gy.dtype], None)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=gy.device)


def gpu_run(wl, inputs=None, device="cuda", poison_workspace=False):
    gy, x, w, m = inputs if inputs is not None else gpu_inputs(wl, device)
    ws = workspace_for(wl, gy, x, w)
    if poison_workspace:
        ws.fill_(0xFF)
    announce(f"mccb_backward {wl.name} S={wl.S} B={wl.B} H={wl.H} W={wl.W} {wl.dtype} "
             f"mask={wl.mask[0]}")
    gx, gw = mdc.backward(gy, x, w, m, workspace=ws)
    torch.cuda.synchronize()
    return gx, gw


def bits16(t: torch.Tensor) -> np.ndarray:
    return wls.bits(t)


def check_gradx(gpu_bits: np.ndarray, ref_bits: np.ndarray, tag: str) -> None:
    d = ulp_dist(gpu_bits, ref_bits)
    worst = int(d.max()) if d.size else 0
    n_off = int(np.count_nonzero(d))
    # the bar is 1 ulp; the kernel rounds the exact sum once, so it is expected to match exactly
    assert worst <= 1, f"{tag}: gradX max ulp distance {worst}"
    assert n_off == 0, f"{tag}: {n_off} gradX elements differ by 1 ulp (expected bit-exact)"


def check_gradw(gpu_bits: np.ndarray, ref: dict, dtype: str, tag: str, cols=None) -> None:
    gw64 = ref["gw64"] if cols is None else ref["gw64"][:, cols]
    got = oracle.get().decode(dtype, gpu_bits)  # decoding is exact, see the oracle's pins
    err = np.abs(got - gw64)
    bound = np.maximum(RTOL[dtype] * np.abs(gw64), SUBNORMAL_STEP[dtype])
    bad = err > bound
    assert not bad.any(), (f"{tag}: gradWeight rel err > {RTOL[dtype]} at {np.argwhere(bad)[:5]}, "
                           f"max rel {float((err / np.maximum(np.abs(gw64), 1e-300)).max())}")
    # fp64 accumulation end to end: expected to equal the correctly rounded value
    ref16 = ref["gw16"] if cols is None else ref["gw16"][:, cols]
    assert int(ulp_dist(gpu_bits, ref16).max(initial=0)) <= 1, f"{tag}: gradWeight ulp > 1"


def oracle_full(wl):
    inp = wls.host_inputs(wl)
    m = inp["mask"]
    return oracle.get().backward(wl.dtype, wls.bits(inp["gy"]), wls.bits(inp["x"]),
                                 wls.bits(inp["w"]), None if m is None else m.numpy(),
                                 want_gx64=False)


def compare_full(wl, gx, gw, tag=None):
    """Whole-tensor comparison (small workloads)."""
    tag = tag or wl.name
    ref = oracle_full(wl)
    check_gradx(bits16(gx), ref["gx16"], tag)
    check_gradw(bits16(gw), ref, wl.dtype, tag)


def sample_channels(wl, n_random: int = 16, seed: int = 0) -> np.ndarray:
    """Channels to check at full size: both ends, lane-vector and block edges, and random ones."""
    H = wl.H
    rng = np.random.default_rng(seed)
    edges = [0, 1, 3, 4, 7, 8, 255, 256, 511, 512, H // 2, H - 9, H - 8, H - 2, H - 1]
    hs = set(h for h in edges if 0 <= h < H)
    hs.update(int(h) for h in rng.integers(0, H, n_random))
    return np.array(sorted(hs), dtype=np.int64)


def compare_columns(wl, gx, gw, hs: np.ndarray, tag=None):
    """Exact check of every gradX element and every gradWeight entry of the channels `hs`: the
    oracle runs on the [S,B,len(hs)] column slices, which hold everything those outputs depend on."""
    tag = tag or wl.name
    hs_t = torch.from_numpy(hs)
    gy_c = wls.column_tensor(wl, wls.STREAM_GY, hs_t)
    x_c = wls.column_tensor(wl, wls.STREAM_X, hs_t)
    w_c = wls.weight_tensor(wl, "cpu")[:, hs_t]
    m = wls.mask_tensor(wl, "cpu")
    ref = oracle.get().backward(wl.dtype, wls.bits(gy_c), wls.bits(x_c), wls.bits(w_c),
                                None if m is None else m.numpy(), want_gx64=False)
    idx = hs_t.to(gx.device)
    gx_c = bits16(gx.index_select(2, idx))
    gw_c = bits16(gw.index_select(1, idx))
    check_gradx(gx_c, ref["gx16"], tag + " (columns)")
    check_gradw(gw_c, ref, wl.dtype, tag + " (columns)")


def compare_rows(wl, gx, rows: np.ndarray, tag=None):
    """Exact check of whole gradX rows: row i depends only on gradY rows i..i+W-1 and the mask
    there, so the oracle runs on that W-row (or shorter, at the end) slab."""
    tag = tag or wl.name
    m = wls.mask_tensor(wl, "cpu")
    w = wls.bits(wls.weight_tensor(wl, "cpu"))
    for r in rows:
        r = int(r)
        rr = torch.arange(r, min(r + wl.W, wl.S), dtype=torch.int64)
        gy_r = wls.bits(wls.row_tensor(wl, wls.STREAM_GY, rr))
        x_r = wls.bits(wls.row_tensor(wl, wls.STREAM_X, rr))
        m_r = None if m is None else m[:, r:r + len(rr)].numpy()
        ref = oracle.get().backward(wl.dtype, gy_r, x_r, w, m_r, want_gx64=False)
        check_gradx(bits16(gx[r]), ref["gx16"][0], f"{tag} (row {r})")


def sample_rows(wl, plan: dict, n_random: int = 6, seed: int = 1) -> np.ndarray:
    S = wl.S
    rng = np.random.default_rng(seed)
    R, T = plan["rows_per_turn"], plan["rows_per_strip"]
    cand = {0, 1, 2, S - 3, S - 2, S - 1, R - 1, R, R + 1, T - 2, T - 1, T, T + 1, 2 * T - 1}
    cand.update(int(r) for r in rng.integers(0, S, n_random))
    return np.array(sorted(r for r in cand if 0 <= r < S), dtype=np.int64)
