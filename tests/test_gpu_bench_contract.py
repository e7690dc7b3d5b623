"""bench.py's output line on a GPU: one JSON object with every field the
measurement contract names, at a small workload (GPT-2-small, rank 0 of 8)
so that it runs in seconds.  The bench runs as a child process, as the
throughput run does."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def test_bench_prints_one_complete_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload",
                        "gpt2_small", "--steps", "3", "--warmup", "1", "--cpu-seconds", "1"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    import bench
    assert d["metric"] == bench.METRIC and d["unit"] == "params/s"
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["data"] == "synthetic" and d["dtype"] == "f32"
    assert isinstance(d["config"]["workload"], str) and d["config"]["shard_elems"] == 15_555_008
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value = real shard elements / wall time per step
    assert abs(d["value"] * d["ms_per_step"] * 1e-3 / d["config"]["real_elems"] - 1) < 1e-9
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["achieved"] < rf["peak"] * 1.2       # the MALL can lift a small shard
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    assert rf["traffic"] is None                       # counters are for the default workload
    k = d["kernels"]["adam_fused"]
    assert abs(rf["achieved"] - 28 * 15_555_008 / (k["avg_ms"] * 1e-3) / 1e9) < 1e-6 * rf["achieved"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "params/s" and cb["cores"] == 1
    assert cb["value"] > 0 and isinstance(cb["sample"], str)
    assert cb["all_cores"]["cores"] >= 1 and cb["all_cores"]["value"] > 0
    assert d["graph_replay"]["ms_per_step"] > 0
    fb = d["kernels"]["flatten_by_bucket"]
    assert fb["calls"] >= 1 and fb["ms"] > 0 and fb["bytes_per_elem"] == 4


def _bench(*args, timeout=300):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, r.stderr[-3000:]
    return r.stdout


def test_placement_probe_reports_every_trial():
    out = _bench("--workload", "gpt2_small", "--placement-probe", "0,1")
    trials = [ln for ln in out.splitlines() if ln.startswith("[placement]")]
    assert len(trials) == 4, out[-2000:]           # 2 ballasts x 2 layouts
    d = json.loads(out.strip().splitlines()[-1])
    assert d["placement_probe_elems"] == 15_555_008 and d["ballasts_gb"] == [0.0, 1.0]
    for layout in ("separate", "one"):
        s = d["layouts"][layout]
        assert 0 < s["min_ms"] <= s["median_ms"] <= s["max_ms"] and s["spread_pct"] >= 0


def test_offload_timeline_is_summarised_and_written(tmp_path):
    path = tmp_path / "timeline.json"
    out = _bench("--mode", "offload", "--workload", "gpt2_small", "--steps", "4", "--warmup", "1",
                 "--no-cpu-baseline", "--timeline", str(path))
    d = json.loads(out.strip().splitlines()[-1])
    tl = json.load(open(path))
    for lag in ("lag1", "lag0"):
        s = d["offload"][lag]["timeline"]
        assert s["pieces"] >= 1 and s["steps"] >= 1
        assert s["gradient_copy_ms"] > 0 and s["host_update_ms"] > 0 and s["parameter_copy_ms"] > 0
        assert 0 <= s["copies_during_update_ms"] <= s["gradient_copy_ms"] + s["parameter_copy_ms"]
        kinds = {r["kind"] for r in tl[lag]}
        assert kinds == {"gradient copy", "host update", "parameter copy"}
        hu = d["offload"][lag]
        assert hu["host_update_gbps"] > 0
        assert abs(hu["host_update_frac"] - hu["host_update_gbps"] / d["offload"]["host_ceiling"]["gbps"]) < 1e-12
    hc = d["offload"]["host_ceiling"]
    assert hc["bytes"] >= 1 << 29 and hc["threads"] == d["offload"]["host_threads"]
    assert hc["gbps"] == max(hc["gbps_before"], hc["gbps_after"]) > 0
