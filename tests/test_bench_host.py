"""Host-side checks of the benchmark's contract (no GPU needed): more than
one GPU is refused with a message and a non-zero status before anything
touches a device, and the algorithmic byte counts follow the stated formula
(the 2*T*k*H*b exchange volume of the communication-wall explainer, plus the
token reads/writes and index traffic)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_formula():
    T, H, E, k = 16384, 7168, 256, 8
    b = bench.algorithmic_bytes(T, H, E, k, T * k, 0)
    assert b["pack"] + b["combine"] - 2 * T * H * 2 - T * k * 12 == 2 * T * k * H * 2  # 2TkHb
    assert b["route"] == T * E * 4 + T * k * 8
    assert b["total"] == 4248829952                      # 4.249 GB per step at this shape
    # quantised rows: codes plus the 4-byte scale kept beside them
    assert bench.payload_bytes(H, 1) == H + 4 and bench.payload_bytes(H, 2) == H // 2 + 4
    assert bench.payload_bytes(H, 3) == H + 4 and bench.payload_bytes(H, 0) == 2 * H
    i8 = bench.algorithmic_bytes(T, H, E, k, T * k, 1)
    assert abs((i8["pack"] - T * H * 2 - T * k * 4) / (T * k * 2 * H) - 0.5003) < 1e-4
