#!/usr/bin/env python3
"""Benchmark: effective HBM bandwidth of the masked causal conv1d backward (fused gradX + gradWeight)
on one MI355X, for the workload S=16384, B=32 (B*S = 512K), H=5120, bf16, Bernoulli(0.9) mask.

A step is one mccb_backward call (the fused mask + gradX + gradWeight-partials kernel and the
fixed-order gradWeight reduction) over inputs already resident in HBM. Effective GB/s counts the
bytes the method must move: read gradY and x, write gradX (2 bytes each per element), read the mask
(1 byte per (j,i)), read the weight and write gradWeight; workspace traffic is not counted.

The same run also times the forward (mccb_forward, y = mask * causal conv(x, w)) on the same x,
weight and mask, reported in the "forward" object of the same line: effective GB/s over its
algorithmic bytes (read x, write y, read the mask and the weight); and both ops again on the same
values stored [B,S,H] and passed as strided [S,B,H] views ("strided" object), with 2- and 4-tap
windows instead of the page's 3 ("taps" object), and on the workload's valid tokens packed into
the variable-length layout ("varlen" object).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
METRIC = "effective HBM GB/s (and % of peak) for fused gradX+gradWeight, B*S=512K H=5120"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def traffic_file(kernel: str, workload_name: str) -> str:
    """The committed rocprofv3 counter summary of one kernel on one workload."""
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload_name}_traffic.txt")


TRAFFIC_FILE = traffic_file("mccb_fused_bwd", "S16384_B32_H5120_bf16")
FWD_TRAFFIC_FILE = traffic_file("mccb_fwd", "S16384_B32_H5120_bf16")
KERNEL_SRC = os.path.join(ROOT, "masked_depthwise_causal_amd", "csrc", "mccb.hip")


def measured_traffic(workload_name: str, path: str = TRAFFIC_FILE):
    """HBM bytes per kernel launch from a committed rocprofv3 counter summary, or None if that
    summary is for another workload or for a different kernel source than the one built."""
    import hashlib

    try:
        kv = {}
        for line in open(path):
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k.strip()] = v.strip()
        src_hash = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
        if kv.get("source_sha256") != src_hash or kv.get("workload") != workload_name:
            return None
        return int(float(kv["hbm_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def copy_ceiling(torch, device, nbytes: int = 4 << 30, reps: int = 10) -> float:
    """GB/s (read + write) of torch's device-to-device copy, a plain streaming reference."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / dt / 1e9


def cpu_baseline(wl, gy, x, w, m, seconds: float, rows_per_chunk: int = 64) -> dict:
    """Time the CPU fp64 oracle on consecutive row chunks of the same inputs until `seconds` of
    compute have run. Chunk copies to the host and input decoding set-up are not timed; the
    oracle's own decode + compute + encode is."""
    import oracle
    from synth import workloads as wls

    orc = oracle.get()
    w16 = wls.bits(w)
    elapsed, elems, chunks = 0.0, 0, 0
    r = 0
    while elapsed < seconds and r < wl.S:
        r1 = min(r + rows_per_chunk, wl.S)
        gyc, xc = wls.bits(gy[r:r1]), wls.bits(x[r:r1])
        mc = None if m is None else m[:, r:r1].cpu().numpy()
        t0 = time.perf_counter()
        orc.backward(wl.dtype, gyc, xc, w16, mc, want_gx64=False)
        elapsed += time.perf_counter() - t0
        elems += (r1 - r) * wl.B * wl.H
        chunks += 1
        r = r1
    rows = r
    alg = 3 * elems * 2 + (rows * wl.B if m is not None else 0) + chunks * 2 * 3 * wl.H * 2
    return {
        "value": round(alg / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": orc.num_threads(),
        "kind": "oracle",
        "sample": (f"rows 0..{rows - 1} of the workload in {chunks} independent chunks of "
                   f"{rows_per_chunk} rows (x B={wl.B} x H={wl.H}), {elapsed:.1f} s of oracle time"),
    }


def cpu_single_thread(workloads, seconds: float, rows_per_chunk: int = 64) -> list:
    """The oracle on one thread, on bounded samples of the small workloads (0-2): consecutive
    64-row chunks, regenerated on the CPU, until `seconds` of oracle time per workload."""
    import torch

    import oracle
    from synth import workloads as wls

    orc = oracle.get()
    n0 = orc.num_threads()
    out = []
    try:
        orc.set_num_threads(1)
        for wl in workloads:
            w16 = wls.bits(wls.weight_tensor(wl, "cpu"))
            mfull = wls.mask_tensor(wl, "cpu")
            elapsed, rows, chunks = 0.0, 0, 0
            while elapsed < seconds and rows < wl.S:
                r1 = min(rows + rows_per_chunk, wl.S)
                rr = torch.arange(rows, r1, dtype=torch.int64)
                gyc = wls.bits(wls.row_tensor(wl, wls.STREAM_GY, rr))
                xc = wls.bits(wls.row_tensor(wl, wls.STREAM_X, rr))
                mc = None if mfull is None else mfull[:, rows:r1].contiguous().numpy()
                t0 = time.perf_counter()
                orc.backward(wl.dtype, gyc, xc, w16, mc, want_gx64=False)
                elapsed += time.perf_counter() - t0
                chunks += 1
                rows = r1
            elems = rows * wl.B * wl.H
            alg = 3 * elems * 2 + (rows * wl.B if mfull is not None else 0) + chunks * 12 * wl.H
            out.append({"workload": wl.describe(), "value": round(alg / elapsed / 1e9, 4),
                        "unit": "GB/s", "cores": 1,
                        "sample": (f"rows 0..{rows - 1} of {wl.S} in {chunks} chunk(s) of up to "
                                   f"{rows_per_chunk} rows, {elapsed:.2f} s of oracle time")})
    finally:
        orc.set_num_threads(n0)
    return out


def stream_ceiling(torch, a, b, stream, reps: int = 20) -> float:
    """GB/s of torch's elementwise a + b into a third tensor (2 reads, 1 write of the same shape
    as the backward's streams), timed between events on `stream`."""
    c = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        torch.add(a, b, out=c)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        torch.add(a, b, out=c)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del c
    torch.cuda.empty_cache()
    return 3 * a.numel() * a.element_size() / (ms * 1e-3) / 1e9


def time_all_configs(torch, mdc, workloads, wls, dev, stream, reps: int) -> list:
    """Backward and forward of every workload, each call timed on its own between HIP events,
    after reading a 1 GiB scratch buffer so that no input is left in the 256 MB Infinity Cache or
    the L2s (the small workloads would otherwise run from cache). The flush reads rather than
    writes, so no dirty lines are left to be written back during the timed call. Each series
    starts with 10 untimed calls. Median and minimum.

    For the backward a second pass of the same calls records the library's HIP events around its
    two kernels (mccb_profile_begin/_end): `fused_kernel` is the fused kernel's average duration
    between those events (which include its dispatch) and its roofline fraction (its algorithmic
    bytes: everything the call moves except the gradWeight write, which the reduction kernel does,
    unless the fused kernel writes gradWeight itself). `flat_stream` is torch's elementwise
    gradY + x into a third tensor of the same shape (the backward's 2 reads and 1 write with no
    stencil, mask or reduction), timed the same way, and the backward against it. `traffic` is the
    fused kernel's HBM bytes per launch from the committed counter summary for this workload
    (null when there is none for the built kernel source)."""
    import statistics

    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def per_call(fn, warm=10):
        # untimed calls first: a kernel's first calls after the inputs are generated or another
        # kernel has run take up to 20 % longer, and settle after about ten
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        times = []
        for r in range(reps):
            flush.sum()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return statistics.median(times), min(times)

    def pct(nbytes, ms):
        return round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)

    rows = []
    for wlc in workloads:
        gy_c = wls.full_tensor(wlc, wls.STREAM_GY, dev)
        x_c = wls.full_tensor(wlc, wls.STREAM_X, dev)
        w_c, m_c = wls.weight_tensor(wlc, dev), wls.mask_tensor(wlc, dev)
        gx_c, gw_c, y_c = torch.empty_like(gy_c), torch.empty_like(w_c), torch.empty_like(x_c)
        ws_c = mdc.workspace_for(wlc.S, wlc.B, wlc.H, gy_c.dtype, dev)
        torch.cuda.synchronize()
        bwd = lambda: mdc.backward(gy_c, x_c, w_c, m_c, gradX=gx_c, gradWeight=gw_c,  # noqa: E731
                                   workspace=ws_c, stream=stream)
        b_med, b_min = per_call(bwd)
        # a second pass of the same per-call timing with the library's kernel events on (they add
        # their own time to the call, so the call's own figure comes from the pass above)
        mdc.mccb_profile_begin(reps)
        per_call(bwd, warm=0)
        k1_ms, k2_ms, n_prof = mdc.mccb_profile_end()
        f_med, f_min = per_call(lambda: mdc.forward(x_c, w_c, m_c, y=y_c, stream=stream))
        s_med, _ = per_call(lambda: torch.add(gy_c, x_c, out=gx_c))
        b_alg = wlc.algorithmic_bytes()
        # with one strip of one batch (no workspace) the fused kernel writes gradWeight itself
        direct = mdc.mccb_get_workspace_size(wlc.S, wlc.B, wlc.H, mdc.DTYPE_CODE[gy_c.dtype]) == 0
        k1_alg = b_alg - (0 if direct else 3 * wlc.H * 2)
        f_alg = 4 * wlc.N + (wlc.B * wlc.S if m_c is not None else 0) + 3 * wlc.H * 2
        s_alg = 3 * wlc.N * 2
        k1_avg = k1_ms / max(n_prof, 1)
        rows.append({
            "workload": wlc.describe(),
            "backward": {"median_ms": round(b_med, 5), "min_ms": round(b_min, 5),
                         "gbs": round(b_alg / (b_med * 1e-3) / 1e9, 1),
                         "pct_of_hbm_peak": pct(b_alg, b_med),
                         "fused_kernel": {"avg_ms": round(k1_avg, 5),
                                          "algorithmic_bytes": k1_alg,
                                          "frac": round(pct(k1_alg, k1_avg) / 100, 4),
                                          "traffic": measured_traffic(
                                              wlc.name, traffic_file("mccb_fused_bwd", wlc.name))},
                         # no reduction kernel runs when the fused kernel writes gradWeight
                         "reduce_kernel_avg_ms": (None if direct
                                                  else round(k2_ms / max(n_prof, 1), 5)),
                         "flat_stream": {"median_ms": round(s_med, 5),
                                         "pct_of_hbm_peak": pct(s_alg, s_med),
                                         "backward_pct_of_flat_stream": round(
                                             100 * pct(b_alg, b_med) / pct(s_alg, s_med), 2)}},
            "forward": {"median_ms": round(f_med, 5), "min_ms": round(f_min, 5),
                        "gbs": round(f_alg / (f_med * 1e-3) / 1e9, 1),
                        "pct_of_hbm_peak": pct(f_alg, f_med)},
        })
        log(f"config {wlc.name}: backward {b_med:.4f} ms (fused kernel {k1_avg:.4f}), forward "
            f"{f_med:.4f} ms, flat stream {s_med:.4f} ms")
        del gy_c, x_c, w_c, m_c, gx_c, gw_c, y_c, ws_c
        torch.cuda.empty_cache()
    del flush
    return rows


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed calls before each timed leg (the backward reaches its steady "
                         "duration after about ten calls)")
    ap.add_argument("--workload", type=int, default=None,
                    help="index into synth.WORKLOADS (default: the B*S=512K H=5120 workload)")
    ap.add_argument("--rows", type=int, default=None,
                    help="run the workload with this many rows S instead (same B, H, dtype and "
                         "mask kind): a shorter stand-in for counter passes on inputs too large "
                         "to generate under the profiler")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-single-seconds", type=float, default=1.5,
                    help="oracle time per workload for the single-thread samples (workloads 0-2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-forward", action="store_true", help="skip timing the forward")
    ap.add_argument("--no-strided", action="store_true",
                    help="skip timing both ops on [B,S,H]-stored (strided) inputs")
    ap.add_argument("--no-taps", action="store_true",
                    help="skip timing both ops with 2- and 4-tap windows")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip timing both ops on the packed variable-length layout")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-call timing of every workload")
    ap.add_argument("--config-reps", type=int, default=15)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU only (--gpus 1). The backward shards across GPUs "
              "by channel with no communication, or by sequence with a 2-row halo and a [3,H] "
              "sum; no multi-GPU runner is provided.", file=sys.stderr)
        return 2

    import torch

    import masked_depthwise_causal_amd as mdc
    from synth import HEADLINE, WORKLOADS
    from synth import workloads as wls

    wl = WORKLOADS[HEADLINE if args.workload is None else args.workload]
    if args.rows is not None:
        wl = dataclasses.replace(wl, S=args.rows, name=f"{wl.name}_rows{args.rows}")
    dev = torch.device("cuda:0")
    log(f"workload {wl.name}: {wl.describe()}")
    gy = wls.full_tensor(wl, wls.STREAM_GY, dev)
    x = wls.full_tensor(wl, wls.STREAM_X, dev)
    w = wls.weight_tensor(wl, dev)
    m = wls.mask_tensor(wl, dev)
    gx = torch.empty_like(gy)
    gw = torch.empty_like(w)
    ws = mdc.workspace_for(wl.S, wl.B, wl.H, gy.dtype, dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    log("inputs resident")

    def step():
        mdc.backward(gy, x, w, m, gradX=gx, gradWeight=gw, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    mdc.mccb_profile_begin(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fused_ms, reduce_ms, n_prof = mdc.mccb_profile_end()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f})")

    alg = wl.algorithmic_bytes()
    value = alg / (ms_per_step * 1e-3) / 1e9
    # dominant kernel: the fused pass moves everything except the gradWeight write
    fused_alg = alg - 3 * wl.H * 2
    fused_avg_ms = fused_ms / max(n_prof, 1)
    achieved = fused_alg / (fused_avg_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(wl.name), "algorithmic_bytes": fused_alg,
                "kernel": "mccb_fused_bwd", "avg_ms": round(fused_avg_ms, 5),
                "timing_source": ("HIP events the library records on the launch stream around "
                                  "the fused kernel (mccb_profile_begin/_end), averaged over the "
                                  f"{n_prof} timed steps"),
                "reduce_avg_ms": round(reduce_ms / max(n_prof, 1), 5)}

    fwd = None
    if not args.no_forward:
        y = torch.empty_like(x)
        for _ in range(args.warmup):
            mdc.forward(x, w, m, y=y, stream=stream)
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(args.steps):
            mdc.forward(x, w, m, y=y, stream=stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        fwd_ms = ev0.elapsed_time(ev1) / args.steps
        fwd_alg = 4 * wl.N + (wl.B * wl.S if m is not None else 0) + 3 * wl.H * 2
        fwd_gbs = fwd_alg / (fwd_ms * 1e-3) / 1e9
        log(f"forward: {fwd_ms:.4f} ms/step, {fwd_gbs:.1f} GB/s")
        fwd = {"metric": "effective HBM GB/s, masked causal conv1d forward, same workload",
               "value": round(fwd_gbs, 1), "unit": "GB/s", "ms_per_step": round(fwd_ms, 5),
               "algorithmic_bytes": fwd_alg,
               "roofline": {"bound": "hbm", "achieved": round(fwd_gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(fwd_gbs / HBM_PEAK_GBS, 4),
                            "traffic": measured_traffic(wl.name, FWD_TRAFFIC_FILE),
                            "kernel": "mccb_fwd", "avg_ms": round(fwd_ms, 5)}}
        del y

    strided = None
    if not args.no_strided:
        # the same values stored [B,S,H] (a batch-major producer), passed as [S,B,H] views: the
        # kernels read them in place through their strides
        gy_p = gy.permute(1, 0, 2).contiguous().permute(1, 0, 2)
        x_p = x.permute(1, 0, 2).contiguous().permute(1, 0, 2)
        ws_p = torch.empty(max(1, mdc.mccb_get_workspace_size_ex(
            gy_p.data_ptr(), x_p.data_ptr(), w.data_ptr(), wl.S, wl.B, wl.H, 3,
            mdc.DTYPE_CODE[gy.dtype], mdc._strides(gy_p, x_p, w, m))), dtype=torch.uint8,
            device=dev)
        y = torch.empty_like(x)

        def timed(fn):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            ev0.record(stream)
            for _ in range(args.steps):
                fn()
            ev1.record(stream)
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / args.steps

        b_ms = timed(lambda: mdc.backward(gy_p, x_p, w, m, gradX=gx, gradWeight=gw, workspace=ws_p,
                                          stream=stream))
        f_ms = timed(lambda: mdc.forward(x_p, w, m, y=y, stream=stream))
        f_alg = 4 * wl.N + (wl.B * wl.S if m is not None else 0) + 3 * wl.H * 2
        strided = {"layout": "gradY and x stored [B,S,H], passed as [S,B,H] views, read in place",
                   "backward": {"value": round(alg / (b_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                                "ms_per_step": round(b_ms, 5)},
                   "forward": {"value": round(f_alg / (f_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                               "ms_per_step": round(f_ms, 5)}}
        log(f"strided [B,S,H] inputs: backward {b_ms:.4f} ms, forward {f_ms:.4f} ms")
        del gy_p, x_p, ws_p, y
        torch.cuda.empty_cache()

    taps = None
    if not args.no_taps:
        taps = {}
        for W in (2, 4):
            wlw = wls.with_taps(wl, W)
            ww = wls.weight_tensor(wlw, dev)
            gww = torch.empty_like(ww)
            ws_w = torch.empty(max(1, mdc.mccb_get_workspace_size_ex(
                gy.data_ptr(), x.data_ptr(), ww.data_ptr(), wl.S, wl.B, wl.H, W,
                mdc.DTYPE_CODE[gy.dtype], None)), dtype=torch.uint8, device=dev)
            y = torch.empty_like(x)

            def timed_w(fn):
                for _ in range(args.warmup):
                    fn()
                torch.cuda.synchronize()
                ev0.record(stream)
                for _ in range(args.steps):
                    fn()
                ev1.record(stream)
                torch.cuda.synchronize()
                return ev0.elapsed_time(ev1) / args.steps

            b_ms = timed_w(lambda: mdc.backward(gy, x, ww, m, gradX=gx, gradWeight=gww,
                                                workspace=ws_w, stream=stream))
            f_ms = timed_w(lambda: mdc.forward(x, ww, m, y=y, stream=stream))
            b_alg = wlw.algorithmic_bytes()
            f_alg = 4 * wl.N + (wl.B * wl.S if m is not None else 0) + W * wl.H * 2
            taps[f"W{W}"] = {"backward": {"value": round(b_alg / (b_ms * 1e-3) / 1e9, 1),
                                          "unit": "GB/s", "ms_per_step": round(b_ms, 5)},
                             "forward": {"value": round(f_alg / (f_ms * 1e-3) / 1e9, 1),
                                         "unit": "GB/s", "ms_per_step": round(f_ms, 5)}}
            log(f"W={W}: backward {b_ms:.4f} ms, forward {f_ms:.4f} ms")
            del ww, gww, ws_w, y
        torch.cuda.empty_cache()

    varlen = None
    if not args.no_varlen:
        # the workload's tokens packed: one sequence per batch, lengths uniform in [S/2, S]
        lengths = wls.varlen_lengths(wl)
        T = int(lengths.sum())
        gy_v, x_v = wls.pack_tokens(gy, lengths), wls.pack_tokens(x, lengths)
        cu = wls.cu_seqlens(lengths, dev)
        gx_v, gw_v, y_v = torch.empty_like(gy_v), torch.empty_like(w), torch.empty_like(x_v)
        ws_b = torch.empty(mdc.mccb_varlen_get_workspace_size(T, wl.B, wl.H, 3,
                                                              mdc.DTYPE_CODE[gy.dtype]),
                           dtype=torch.uint8, device=dev)
        ws_f = torch.empty(mdc.mccb_varlen_forward_get_workspace_size(T, wl.B, wl.H, 3,
                                                                      mdc.DTYPE_CODE[gy.dtype]),
                           dtype=torch.uint8, device=dev)

        def timed_v(fn):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            ev0.record(stream)
            for _ in range(args.steps):
                fn()
            ev1.record(stream)
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / args.steps

        b_ms = timed_v(lambda: mdc.varlen_backward(gy_v, x_v, w, cu, None, gradX=gx_v,
                                                   gradWeight=gw_v, workspace=ws_b, stream=stream))
        f_ms = timed_v(lambda: mdc.varlen_forward(x_v, w, cu, None, y=y_v, workspace=ws_f,
                                                  stream=stream))
        b_alg = 6 * T * wl.H + 2 * 3 * wl.H * 2 + 8 * wl.B
        f_alg = 4 * T * wl.H + 3 * wl.H * 2 + 8 * wl.B
        varlen = {"layout": f"packed [T,H], T={T} tokens in {wl.B} sequences (lengths uniform in "
                            f"[S/2, S]), H={wl.H}, no mask",
                  "backward": {"value": round(b_alg / (b_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                               "ms_per_step": round(b_ms, 5), "algorithmic_bytes": b_alg},
                  "forward": {"value": round(f_alg / (f_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                              "ms_per_step": round(f_ms, 5), "algorithmic_bytes": f_alg}}
        log(f"varlen T={T}: backward {b_ms:.4f} ms, forward {f_ms:.4f} ms")
        del gy_v, x_v, gx_v, gw_v, y_v, ws_b, ws_f
        torch.cuda.empty_cache()

    ceiling = stream_gbs = None
    if not args.no_ceiling:
        ceiling = round(copy_ceiling(torch, dev), 1)
        log(f"copy ceiling {ceiling} GB/s")
        stream_gbs = round(stream_ceiling(torch, gy, x, stream), 1)
        log(f"read-2/write-1 streaming ceiling (torch add) {stream_gbs} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl, gy, x, w, m, args.cpu_seconds)
        log(f"cpu baseline {cpu['value']} GB/s on {cpu['cores']} threads")
        cpu["single_thread"] = cpu_single_thread(WORKLOADS[:3], args.cpu_single_seconds)
        log("cpu single thread: " + ", ".join(str(r["value"]) for r in cpu["single_thread"]))

    configs = None
    if not args.no_configs:
        del gy, x, gx, ws, m
        torch.cuda.empty_cache()
        configs = time_all_configs(torch, mdc, WORKLOADS, wls, dev, stream, args.config_reps)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",  # arithmetic: every sum is an fp64 FMA chain; storage is config.storage_dtype
        "data": "synthetic",
        "config": {"workload": wl.describe(), "S": wl.S, "B": wl.B, "H": wl.H,
                   "storage_dtype": wl.dtype,
                   "algorithmic_bytes": alg, "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "copy_ceiling_gbs": ceiling, "stream_ceiling_gbs": stream_gbs,
                   "pct_of_stream_ceiling": (round(100 * value / stream_gbs, 2)
                                             if stream_gbs else None)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "forward": fwd,
        "strided": strided,
        "taps": taps,
        "varlen": varlen,
        "configs": configs,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
