"""Precision report (needs a GPU): for every benchmark workload, the ulp histogram of gradX and of
the forward's y against the oracle's correctly rounded values, and gradWeight's errors against the
oracle's unrounded fp64 sums. Workload 0 is compared whole; the larger ones on the channels and rows
the full-size parity tests sample (every element of a sampled channel, over all rows and batches,
and every element of a sampled row). Prints one markdown table.

    python -m tests.precision_report
"""
from __future__ import annotations

import numpy as np
import torch

import masked_depthwise_causal_amd as mdc
import oracle
from synth import WORKLOADS
from synth import workloads as wls

from .gpu_util import bits16, gpu_inputs, sample_channels, sample_rows, ulp_dist


def hist(d: np.ndarray) -> tuple:
    return int(np.count_nonzero(d == 0)), int(np.count_nonzero(d == 1)), int(np.count_nonzero(d > 1))


def plan_of(wl) -> dict:
    return mdc.mccb_get_plan(wl.S, wl.B, wl.H, mdc.MCCB_BF16 if wl.dtype == "bf16" else mdc.MCCB_FP16)


def report(idx: int) -> str:
    wl = WORKLOADS[idx]
    gy, x, w, m = gpu_inputs(wl)
    gx, gw = mdc.backward(gy, x, w, m)
    y = mdc.forward(x, w, m)
    torch.cuda.synchronize()
    orc = oracle.get()
    m_cpu = wls.mask_tensor(wl, "cpu")
    m_np = None if m_cpu is None else m_cpu.numpy()
    gx_d, y_d = [], []
    if idx == 0:
        hs = np.arange(wl.H, dtype=np.int64)
    else:
        hs = sample_channels(wl, seed=idx)
    hs_t = torch.from_numpy(hs)
    gy_c = wls.bits(wls.column_tensor(wl, wls.STREAM_GY, hs_t))
    x_c = wls.bits(wls.column_tensor(wl, wls.STREAM_X, hs_t))
    w_c = wls.bits(wls.weight_tensor(wl, "cpu")[:, hs_t])
    ref = orc.backward(wl.dtype, gy_c, x_c, w_c, m_np, want_gx64=False)
    idx_t = hs_t.to(gx.device)
    gx_d.append(ulp_dist(bits16(gx.index_select(2, idx_t)), ref["gx16"]).ravel())
    gw_bits = bits16(gw.index_select(1, idx_t))
    gw_got = orc.decode(wl.dtype, gw_bits)
    gw64 = ref["gw64"]
    err = np.abs(gw_got - gw64)
    rel_max = float((err / np.abs(gw64)).max())
    norm_rel = float(np.linalg.norm(err) / np.linalg.norm(gw64))
    gw_h = hist(ulp_dist(gw_bits, ref["gw16"]).ravel())
    ref_y = orc.forward16(wl.dtype, x_c, w_c, m_np)["y16"]
    y_d.append(ulp_dist(bits16(y.index_select(2, idx_t)), ref_y).ravel())
    n_rows = 0
    if idx != 0:
        wb = wls.bits(wls.weight_tensor(wl, "cpu"))
        for r in sample_rows(wl, plan_of(wl), seed=idx):
            r = int(r)
            rr = torch.arange(r, min(r + wl.W, wl.S), dtype=torch.int64)
            gy_r = wls.bits(wls.row_tensor(wl, wls.STREAM_GY, rr))
            x_r = wls.bits(wls.row_tensor(wl, wls.STREAM_X, rr))
            m_r = None if m_np is None else m_np[:, r:r + len(rr)]
            ref_r = orc.backward(wl.dtype, gy_r, x_r, wb, m_r, want_gx64=False)
            gx_d.append(ulp_dist(bits16(gx[r]), ref_r["gx16"][0]).ravel())
            # y row r depends on x rows r-W+1 .. r
            ry = torch.arange(max(r - wl.W + 1, 0), r + 1, dtype=torch.int64)
            x_y = wls.bits(wls.row_tensor(wl, wls.STREAM_X, ry))
            m_y = None if m_np is None else m_np[:, int(ry[0]):r + 1]
            ref_yr = orc.forward16(wl.dtype, x_y, wb, m_y)["y16"][-1]
            y_d.append(ulp_dist(bits16(y[r]), ref_yr).ravel())
            n_rows += 1
    gxh, yh = hist(np.concatenate(gx_d)), hist(np.concatenate(y_d))
    where = "whole" if idx == 0 else f"{len(hs)} channels + {n_rows} rows"
    return (f"| {idx}: S={wl.S} B={wl.B} H={wl.H} {wl.dtype} | {where} | {gxh[0]:,} / {gxh[1]} / "
            f"{gxh[2]} | {yh[0]:,} / {yh[1]} / {yh[2]} | {len(hs) * wl.W} | {gw_h[0]} / {gw_h[1]} / "
            f"{gw_h[2]} | {rel_max:.2e} | {norm_rel:.2e} |")


def main() -> None:
    print("| workload | compared | gradX ulp 0 / 1 / >1 | y ulp 0 / 1 / >1 | gradWeight entries | "
          "gradWeight ulp 0 / 1 / >1 (vs oracle rounding) | gradWeight max rel err | normwise rel err |")
    print("|---|---|---|---|---|---|---|---|")
    for idx in range(len(WORKLOADS)):
        print(report(idx), flush=True)
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
