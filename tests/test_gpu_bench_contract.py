"""bench.py end to end on the tiny workload: one JSON line with the metric, the roofline of the
dominant kernel, the CPU oracle baseline on its stated sample, the step's byte accounting and the
probe statistics, all consistent with each other."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_consistent_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--steps", "20", "--warmup", "4"], cwd=ROOT, stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["metric"].startswith("embedding rows looked up+updated/sec")
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 4 and d["unit"] == "rows/s"
    assert d["config"]["workload"] == "tiny_f1_k10k_d16_fp32" and d["dtype"] == "f32"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value is (lookups + row updates) per second over the timed steps
    per_step = d["config"]["mean_lookups_per_step"] + d["config"]["mean_rows_updated_per_step"]
    assert abs(d["value"] * d["ms_per_step"] / 1e3 / per_step - 1) < 0.05
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert rf["kernel"] in d["kernels"] and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    assert abs(rf["achieved"] - rf["alg_bytes_per_launch"] / rf["avg_launch_ms"] / 1e6) < 1e-6 * rf["achieved"]
    longest = max(d["kernels"].values(), key=lambda k: k["avg_launch_ms"])
    assert d["kernels"][rf["kernel"]] is longest
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0 and cb["sample"]
    s = d["step_hbm"]
    assert s["b_min_per_step"] < s["alg_bytes_per_step"]
    assert s["amplification_sort"] == pytest.approx(
        (s["alg_bytes_per_step"] + s["sort_bytes_per_step"]) / s["alg_bytes_per_step"])
    # medians of the per-step event times over one pass of the ring
    m = {k: s[k] for k in ("t_step_median_ms", "t_fwd_median_ms", "t_bwd_median_ms")}
    assert all(v > 0 for v in m.values())
    assert m["t_fwd_median_ms"] < m["t_step_median_ms"] and m["t_bwd_median_ms"] < m["t_step_median_ms"]
    p = d["probe_stats"]
    assert p["scans"] > 0 and 1.0 <= p["buckets_per_scan"] <= p["max_buckets_one_scan"]
    assert d["pass_flash"]["bytes"] > 0
