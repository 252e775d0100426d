"""The benchmark's command-line contract, checked without a GPU: more than
one GPU is refused with a message and exit status 2 (the path runs on one
GPU), and the JSON line's fields and its roofline object have the shape the
contract names."""

import json
import os
import subprocess
import sys
from types import SimpleNamespace

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8", "--steps", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_json_line_fields():
    args = SimpleNamespace(steps=20, warmup=5)
    line = bench.base_line(args, "splice_32k_27layer", 6100.123, 0.1881234, {"layers": 27})
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 20 and line["warmup"] == 5
    assert line["higher_is_better"] is True and line["vs_baseline"] is None
    assert line["config"]["workload"] == "splice_32k_27layer" and "model" not in line["config"]
    json.dumps(line)


def test_roofline_object():
    # 10 launches of 1.148 GB in 1.8 ms in all: 180 us each
    r = bench.roofline("splice_kernel", "splice_32k_27layer", 10, 1.8, 10 * 1148110848)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - 1148110848 / 180e-6 / 1e9) < 0.01
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-4
    assert "traffic" in r and r["kernel_avg_us"] == 180.0 and r["bytes_per_launch"] == 1148110848
    # a workload with no counter summary reports no traffic
    assert bench.roofline("splice_kernel", "no_such_workload", 1, 1.0, 1)["traffic"] is None
