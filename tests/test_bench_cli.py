"""The benchmark's command line and pure helpers (no GPU)."""

from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_percentiles_nearest_rank():
    xs = [float(i) for i in range(1, 11)]          # 1 .. 10
    assert bench.percentiles(xs) == [2.0, 6.0, 9.0]  # indexes floor(p (n - 1) + 1/2): 1, 5, 8
    assert bench.percentiles([]) is None
    assert bench.percentiles([3.5]) == [3.5, 3.5, 3.5]


class _Shape:
    def __init__(self, Hq, Hkv, D, dtype):
        self.Hq, self.Hkv, self.D, self.dtype = Hq, Hkv, D, dtype


def test_side_bytes_of_a_decode():
    # beam shape: 32 layers, 8 branches, Hq 32, Hkv 8, D 128, bf16; 64 partial rows per plane
    sh = _Shape(32, 8, 128, "bf16")
    info = {"partial_rows": 64, "workspace_bytes": 64 * 32 * 8 * (128 + 2) * 4 + 1792,
            "plan_bytes": 1632}
    b = bench.side_bytes(sh, 32, 8, info)
    assert b["q"] == 32 * 8 * 32 * 128 * 2
    assert b["out"] == 32 * 8 * 32 * 128 * 4
    assert b["partials"] == 2 * 64 * 32 * 8 * 130 * 4
    assert b["plan"] == 1632 and b["plan_in_launch_args"]
    info["plan_bytes"] = 9000
    assert not bench.side_bytes(sh, 32, 8, info)["plan_in_launch_args"]
