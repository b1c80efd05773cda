"""The benchmark's JSON line on a short run of the tiny workload: every field
of the contract is present and consistent (one GPU, the metric's unit, the
roofline of the dominant kernel, the oracle's CPU baseline)."""
import json
import os
import subprocess
import sys

import pytest

from gpu_helpers import need_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    need_gpu()
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "tiny",
           "--steps", "5", "--warmup", "2", "--profile-steps", "3", "--warm-steps", "3",
           "--cpu-steps", "1", "--layers", "2"]
    print("bench:", " ".join(cmd[2:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 5 and j["warmup"] == 2
    assert j["unit"] == "keys/s" and j["value"] > 0 and j["higher_is_better"] is True
    assert j["ms_per_step"] > 0 and j["vs_baseline"] is None
    assert j["config"]["workload"]
    assert j["dtype"] == "f32"  # the tiny workload stores and computes in fp32
    roof = j["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    # the whole step against the same peak
    sr = j["step_roofline"]
    assert sr["algorithmic_bytes_per_step"] >= roof["algorithmic_bytes_per_launch"]
    assert abs(sr["frac"] - sr["achieved"] / sr["peak"]) < 1e-9
    assert 0 < sr["frac"] < 1 and sr["floor_us_at_peak"] < j["ms_per_step"] * 1e3
    cb = j["cpu_baseline"]
    for key in ("value", "unit", "cores", "threads", "host_cores", "kind", "sample"):
        assert key in cb, key
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["threads"] == cb["cores"] and cb["host_cores"] == os.cpu_count()
    # the timed region: 5 graph-replayed parts of one step, median and p90
    ts = j["timed_step_us"]
    assert ts["parts"] == 5 and sum(ts["steps_per_part"]) == 5
    assert 0 < ts["median"] <= ts["p90"]
    # recall split by stage: the vote stage's candidates, then the rerank
    st = j["recall"]["stages"]
    assert 0.0 <= st["candidate_recall_min"] <= st["candidate_recall_mean"] <= 1.0
    assert j["recall"]["mean"] <= st["candidate_recall_mean"] + 1e-12
