"""Host-side checks of bench.py (no GPU): the single-GPU guard, the counter-summary lookup that fills
`roofline.traffic` (only for the kernel source it was measured on), and the CPU-oracle baseline
legs on the smallest workload."""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

import bench
import oracle
from synth import WORKLOADS
from synth import workloads as wls

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
    assert r.stdout == ""


def _summary(tmp_path, src_hash, workload, nbytes=123456789):
    p = tmp_path / "traffic.txt"
    p.write_text(f"# comment line\nworkload={workload}\nsource_sha256={src_hash}\n"
                 f"hbm_bytes_per_launch={nbytes}\n")
    return str(p)


def test_traffic_is_read_only_for_the_built_source(tmp_path):
    src = hashlib.sha256(open(bench.KERNEL_SRC, "rb").read()).hexdigest()
    name = WORKLOADS[3].name
    assert bench.measured_traffic(name, _summary(tmp_path, src, name)) == 123456789
    # another kernel source, another workload, a missing file: no traffic figure
    assert bench.measured_traffic(name, _summary(tmp_path, "0" * 64, name)) is None
    assert bench.measured_traffic("other", _summary(tmp_path, src, name)) is None
    assert bench.measured_traffic(name, str(tmp_path / "missing.txt")) is None


def test_committed_summaries_name_their_source():
    for path in (bench.TRAFFIC_FILE, bench.FWD_TRAFFIC_FILE):
        kv = dict(line.strip().split("=", 1) for line in open(path)
                  if "=" in line and not line.startswith("#"))
        assert len(kv["source_sha256"]) == 64
        assert kv["workload"] == WORKLOADS[3].name
        assert int(float(kv["hbm_bytes_per_launch"])) > 0


def test_cpu_baseline_legs_on_the_smallest_workload():
    wl = WORKLOADS[0]
    inp = wls.host_inputs(wl)
    r = bench.cpu_baseline(wl, inp["gy"], inp["x"], inp["w"], inp["mask"], seconds=0.05)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert r["cores"] == oracle.get().num_threads()
    single = bench.cpu_single_thread(WORKLOADS[:1], seconds=0.05)
    assert len(single) == 1 and single[0]["cores"] == 1 and single[0]["value"] > 0
    assert oracle.get().num_threads() == r["cores"]  # the thread count is restored
