"""The benchmark's output contract: a short run of bench.py prints exactly one
JSON line on stdout with the fields its readers parse, and the line is
consistent with itself -- value is the algorithmic bytes of a step over its
wall time, the fractions are achieved over peak, the roofline kernel's rate
is its bytes per launch over its average launch time -- and carries the
HBM-only (delay-line) figure, whose output equals the pipeline's."""
import json
import os
import subprocess
import sys
import time

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def close(a, b, rel):
    return abs(a - b) <= rel * abs(b)


def test_bench_line_contract():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
           "--no-configs", "--no-ep", "--no-overlap", "--no-cpu-baseline", "--no-variant"]
    print("running", " ".join(cmd[1:]), flush=True)
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    print(f"bench.py returned {r.returncode} after {time.time() - t0:.1f} s; its log ends:\n"
          + r.stderr[-1200:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "hbm_cold", "copy_peak", "kernels"):
        assert key in d, key
    assert d["metric"].startswith("dispatch+combine HBM GB/s")
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 3, 1)
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["dtype"] == "bf16" and d["data"] == "synthetic"
    c = d["config"]
    assert (c["T"], c["H"], c["E"], c["k"], c["R"], c["chunks"]) == (16384, 7168, 256, 8, 32, 8)
    assert d["algorithmic_bytes_per_step"] == 4248829952
    assert close(d["value"], d["algorithmic_bytes_per_step"] / (d["ms_per_step"] * 1e-3) / 1e9,
                 2e-3)
    assert close(d["pct_of_peak"], 100 * d["value"] / 8000.0, 2e-3)
    roof = d["roofline"]
    assert (roof["bound"], roof["unit"], roof["peak"], roof["kernel"]) == \
        ("hbm", "GB/s", 8000.0, "combine_pack")
    assert close(roof["frac"], roof["achieved"] / roof["peak"], 2e-3)
    assert close(roof["achieved"],
                 roof["algorithmic_bytes_per_launch"] / (roof["avg_launch_us"] * 1e-6) / 1e9, 2e-3)
    assert roof["min_launch_us"] <= roof["median_launch_us"] <= 1.5 * roof["avg_launch_us"]
    assert roof["traffic"] is None or roof["traffic"] > roof["algorithmic_bytes_per_launch"] * 0.9
    assert 0 < roof["frac"] < 1.2 and 0 < roof["hbm_cold"]["frac"] <= roof["frac"] * 1.05
    cold = d["hbm_cold"]
    assert cold["output_equals_pipeline"] is True
    assert cold["algorithmic_bytes_per_step"] == d["algorithmic_bytes_per_step"]
    assert d["copy_peak"]["copy_gbs"] > 0 and d["copy_peak"]["read_gbs"] > 0
    assert set(d["kernels"]) >= {"route_layout", "pack", "combine_pack", "combine"}
