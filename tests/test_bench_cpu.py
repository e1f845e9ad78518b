"""bench.py's host-side contract, on the CPU: more than one GPU is refused
with a message, the algorithmic byte count is the documented sum, and the
CPU baseline reports what it timed."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _run_bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300, env=env)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = _run_bench("--gpus", str(n))
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _run_bench(env=env)
    assert r.returncode == 2 and "WORLD_SIZE=2" in r.stderr


def test_algorithmic_bytes_is_sources_plus_rows():
    import bench
    import vision_image_preprocessing_amd as V
    import workloads as W

    b = W.uniform_images([(300, 200, 3), (45, 77, 4), (1024, 1024, 3)], seed=5)
    plan = V.plan_batch(b.shapes)
    src = sum(h * w * c for h, w, c in b.shapes)
    rows = int(plan.desc["rows"].sum())
    assert bench.algorithmic_bytes(plan, 4, 1) == {"read": src, "write": rows * 1536 * 4,
                                                   "total": src + rows * 1536 * 4}
    assert bench.algorithmic_bytes(plan, 2, 2)["total"] == src + 2 * rows * 1536 * 2


def test_cpu_baseline_reports_its_sample():
    import bench
    import vision_image_preprocessing_amd as V
    import workloads as W

    b = W.uniform_images([(64, 64, 3), (40, 90, 4), (100, 30, 3)], seed=6)
    plan = V.plan_batch(b.shapes)
    res = bench.cpu_baseline(b, plan, sample=2, threads=2)
    assert res["kind"] == "oracle" and res["cores"] == 2 and res["unit"] == "images/s"
    assert res["value"] > 0 and np.isfinite(res["value"])
    assert res["sample"].startswith("first 2 of 3 images")
    src = 64 * 64 * 3 + 40 * 90 * 4
    rows = int(plan.desc["rows"][0] + plan.desc["rows"][1])
    assert res["GB/s"] == pytest.approx((src + rows * 1536 * 4) / res["seconds"] / 1e9)
