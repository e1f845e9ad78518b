"""The library opened before torch is imported: torch and the library must
still share one HIP runtime (torch ships its own under the system's
sonames), so that the library can use torch's device memory.  Runs in a
child process, since the order only matters before the first import."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import vision_image_preprocessing_amd as V
V.load()                      # before any import of torch
import numpy as np
import torch
import oracle
import workloads as W
b = W.uniform_images([(45, 77, 3), (64, 64, 4)], seed=3)
plan = V.plan_batch(b.shapes)
src = V.processor.upload_sources(b.packed, plan)
out = V.preprocess(src, plan, mean=b.mean, std=b.std, out_dtype="f32")
torch.cuda.synchronize()
got = out["pixel_values"].cpu().numpy()
for i in range(len(b)):
    d = plan.desc[i]
    m, s = oracle.stats255(b.mean, b.std)
    ref = oracle.preprocess_image(b.image(i), int(d["dst_h"]), int(d["dst_w"]), m, s)
    r0 = int(d["row_offset"])
    assert np.abs(got[r0:r0 + int(d["rows"])] - ref).max() <= 1e-4, i
print("import-order ok", flush=True)
"""


def test_library_opened_before_torch():
    if os.environ.get("HIP_VISIBLE_DEVICES") == "":
        pytest.skip("no GPU visible")
    print("[gpu-import-order] child process", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "import-order ok" in r.stdout
