#!/usr/bin/env python3
"""Throughput of the MiMo-V2 image pixel path on one MI355X.

A step is one pass of the whole pixel path over one batch: one call of
mimo_preprocess_batch, which uploads the batch's descriptor table and runs
the fused kernel (flatten, cast, bilinear resize, standardise, two frames,
patch rows in merge-block order and, for the throughput batch, the same rows
in column order).  Inputs are resident in HBM before timing starts.

Default workload: 512 RGB uint8 1024x1024 images (seeded uniform pixels),
ImageNet statistics, float32 rows in merge-block and column order.

Prints one JSON line: images/s, step time, achieved algorithmic HBM
bandwidth of the fused kernel against the 8 TB/s peak, and the CPU oracle
timed on a bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "images/s and achieved HBM GB/s (% of peak), 1×MI355X, preprocess_batch"
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "vision_image_preprocessing_amd", "csrc", "preprocess.hip")
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def algorithmic_bytes(plan, out_bytes_per_value: int, outputs: int) -> dict:
    """uint8 sources read once + every output row written once per output
    (1536 values per row, both frames counted)."""
    read = int(plan.total_src_bytes)
    write = int(plan.total_rows) * 1536 * out_bytes_per_value * outputs
    return {"read": read, "write": write, "total": read + write}


def measured_traffic(workload: str):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counters,
    scaled by the copy-kernel calibration, if they were taken on the
    current kernel source; else None."""
    path = os.path.join(PROFILES, f"preprocess_kernel_{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (as lscpu reports it)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_threads() -> int:
    """Threads for the CPU baseline: the CPUs this process may run on, at
    most 16 -- one GPU's share of the host on the GPU machines, whatever larger
    count os.cpu_count() shows there."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(16, avail))


def cpu_baseline(batch, plan, sample: int, threads: int, out_bytes_per_value: int = 4) -> dict:
    """The oracle, as it is, on the first `sample` items (images, or clips
    for a video batch), one item per thread at a time.  "GB/s" counts the
    sampled items' source bytes plus their rows once at out_bytes_per_value
    (the oracle computes merge-block order; the column order is an index
    permutation of it)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    m, s = oracle.stats255(batch.mean, batch.std)
    idx = list(range(min(sample, len(batch))))

    def one(i):
        d = plan.desc[i]
        if batch.is_media:
            oracle.preprocess_video(batch.clip(i), int(d["dst_h"]), int(d["dst_w"]), m, s)
        else:
            oracle.preprocess_image(batch.image(i), int(d["dst_h"]), int(d["dst_w"]), m, s)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, idx))
    dt = time.perf_counter() - t0
    counts = batch.frame_counts
    units = sum(counts[i] for i in idx)
    nbytes = sum(int(plan.desc["src_h"][i]) * int(plan.desc["src_w"][i]) * int(plan.desc["channels"][i]) *
                 counts[i] + int(plan.desc["rows"][i]) * 1536 * out_bytes_per_value for i in idx)
    unit = "frames/s" if batch.is_media else "images/s"
    what = "clips" if batch.is_media else "images"
    return {"value": units / dt, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"first {len(idx)} of {len(batch)} {what} of the same batch"
                      + (f" ({units} frames)" if batch.is_media else "")
                      + f", one item per thread, {threads} threads, {dt:.2f} s wall",
            "seconds": dt, "GB/s": nbytes / dt / 1e9, "cpu_model": cpu_model(),
            "host_cpus_visible": os.cpu_count()}


def time_launches(V, fn, reps: int, stream):
    """Mean kernel time (ms) of `reps` calls of fn, each launch bracketed by
    the library's launch events."""
    import numpy as np
    import torch

    fn()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for ev in starts + ends:
        ev.record(stream)
    torch.cuda.synchronize()
    for i in range(reps):
        V.set_launch_events(starts[i], ends[i])
        fn()
    V.set_launch_events(None, None)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in zip(starts, ends)]))


def vit_tables_rates(V, plan, ws, reps: int, rope_dim: int = 32) -> dict:
    """The ViT index-table kernels on the same batch, rows in column order:
    algorithmic bytes are what they write (int32 (h, w) + float32 cos and sin
    per row; int64 index and inverse per merge unit)."""
    import torch

    stream = torch.cuda.current_stream()
    rows, units = plan.total_rows, plan.total_rows // 4
    pos = torch.empty((rows, 2), dtype=torch.int32, device="cuda")
    cos = torch.empty((rows, rope_dim), dtype=torch.float32, device="cuda")
    sin = torch.empty_like(cos)
    idx = torch.empty(units, dtype=torch.int64, device="cuda")
    inv = torch.empty_like(idx)
    out = {}
    ms = time_launches(V, lambda: V.rotary_tables(plan.desc, ws, pos=pos, cos=cos, sin=sin,
                                                   column=True, rope_dim=rope_dim), reps, stream)
    b = rows * (8 + 2 * 4 * rope_dim)
    out["rotary_tables_kernel"] = {"rows": rows, "rope_dim": rope_dim, "bytes": b, "ms": ms,
                                   "GB/s": b / (ms * 1e-3) / 1e9,
                                   "frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    ms = time_launches(V, lambda: V.window_index(plan.desc, ws, index=idx, inverse=inv,
                                                  column_major=True), reps, stream)
    b = units * 16
    out["window_index_kernel"] = {"units": units, "bytes": b, "ms": ms,
                                  "GB/s": b / (ms * 1e-3) / 1e9,
                                  "frac": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def hf_contrast_rates(V, batch, plan, src, rows, reps: int) -> dict:
    """The stock-HF contrast path on the same batch (stills only): kernel
    time against the same algorithmic bytes as the MiMo kernel (sources read
    once, rows written once per output), and the pixel shift between the two
    paths' merge-order rows, in units of the channel standard deviation."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream()
    plan_h = V.plan_batch_hf(batch.shapes, check=False)
    if (plan_h.desc["status"] != 0).any() or not np.array_equal(plan_h.image_grid_thw,
                                                               plan.image_grid_thw):
        return {"skipped": "the stock geometry refuses or differs from the MiMo one on this batch"}
    tdtype = rows.dtype
    out = torch.empty_like(rows)
    out_col = torch.empty_like(rows) if batch.column_order else None
    ws = torch.empty(V.hf_workspace_bytes(plan_h.desc), dtype=torch.uint8, device="cuda")
    call = lambda: V.preprocess_hf(src, plan_h, mean=batch.mean, std=batch.std,
                                   out_dtype="f32" if tdtype == torch.float32 else "bf16",
                                   column_order=batch.column_order, rows=out, rows_col=out_col,
                                   workspace=ws)
    ms = time_launches(V, call, reps, stream)
    bpv = 4 if tdtype == torch.float32 else 2
    alg = plan_h.total_src_bytes + plan_h.total_rows * 1536 * bpv * (2 if batch.column_order else 1)
    diff = (rows.float() - out.float()).abs()
    res = {"kernel": "hf_preprocess_kernel", "ms": ms, "algorithmic_bytes": alg,
           "GB/s": alg / (ms * 1e-3) / 1e9, "frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "shift_vs_mimo_std_units": {"mean": float(diff.mean()), "max": float(diff.max())}}
    del out, out_col, ws, diff
    torch.cuda.empty_cache()
    return res


def patch_embed_rates(V, batch, plan, src, ws, reps: int, embed_dim: int = 1280) -> dict:
    """The patch embedding (the rows' Conv3d consumer) on the same batch's
    rows emitted in bf16: the full weight (K = 1536) and, for a batch of
    stills, the folded weight (K = 768).  Synthetic N(0, 0.02) weights."""
    import torch

    stream = torch.cuda.current_stream()
    rows = torch.empty((plan.total_rows, 1536), dtype=torch.bfloat16, device="cuda")
    V.preprocess(src, plan, mean=batch.mean, std=batch.std, out_dtype="bf16", rows=rows,
                 workspace=ws)
    g = torch.Generator(device="cuda").manual_seed(0)
    w = (torch.randn((embed_dim, 1536), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    bias = torch.zeros(embed_dim, dtype=torch.float32, device="cuda")
    out = torch.empty((plan.total_rows, embed_dim), dtype=torch.bfloat16, device="cuda")
    res = {"rows": plan.total_rows, "embed_dim": embed_dim, "out": "bf16",
           "weights": "synthetic N(0, 0.02^2) bf16"}
    forms = [("full", w, 1536)]
    if not batch.is_media:
        forms.append(("folded", V.fold_patch_weights(w), 768))
    for name, wt, k in forms:
        ms = time_launches(V, lambda: V.patch_embed(rows, wt, bias, out=out), reps, stream)
        tflops = 2.0 * plan.total_rows * embed_dim * k / (ms * 1e-3) / 1e12
        res[name] = {"k": k, "ms": ms, "TFLOP/s": tflops, "frac": tflops / MFMA_BF16_PEAK_TFLOPS}
    if not batch.is_media:
        # pixels -> embeddings, stills: the pair (bf16 rows, then the folded
        # GEMM over them) against the fused kernel, which never writes the rows
        ms_rows = time_launches(V, lambda: V.preprocess(src, plan, mean=batch.mean, std=batch.std,
                                                         out_dtype="bf16", rows=rows, workspace=ws),
                                reps, stream)
        wp, bp = V.prepare_pixel_embed_weights(w, bias, batch.mean, batch.std)
        ms_fused = time_launches(V, lambda: V.embed_pixels(src, plan, wp, bp, out=out, workspace=ws),
                                 reps, stream)
        tflops = 2.0 * plan.total_rows * embed_dim * 768 / (ms_fused * 1e-3) / 1e12
        pair = ms_rows + res["folded"]["ms"]
        res["pixels_to_embed"] = {"kernel": "pixel_embed_kernel", "rows_then_folded_gemm_ms": pair,
                                  "rows_kernel_ms": ms_rows, "fused_ms": ms_fused,
                                  "fused_TFLOP/s": tflops, "fused_frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                                  "speedup_vs_pair": pair / ms_fused}
    # the same product through torch's bf16 matmul (vendor GEMM), for context
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.matmul(rows, w.t(), out=out)
    e0.record(stream)
    for _ in range(reps):
        torch.matmul(rows, w.t(), out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    res["torch_matmul_full"] = {"ms": ms, "TFLOP/s": 2.0 * plan.total_rows * embed_dim * 1536 / (ms * 1e-3) / 1e12}
    del rows, out
    torch.cuda.empty_cache()
    return res


def pixel_rates(V, batch, plan, src, out_dtype: str, merge: bool, column: bool, reps: int,
                rows=None, ws=None) -> dict:
    """Kernel time of mimo_preprocess_batch on a resident batch (launch
    events around each launch), against the algorithmic bytes: sources read
    once, every row written once per requested order."""
    import torch

    tdtype = torch.float32 if out_dtype == "f32" else torch.bfloat16
    bpv = 4 if out_dtype == "f32" else 2
    if merge and rows is None:
        rows = torch.empty((plan.total_rows, 1536), dtype=tdtype, device="cuda")
    rows_col = torch.empty((plan.total_rows, 1536), dtype=tdtype, device="cuda") if column else None
    if ws is None:
        ws = torch.empty(V.workspace_bytes(len(plan)), dtype=torch.uint8, device="cuda")
    call = lambda: V.preprocess(src, plan, mean=batch.mean, std=batch.std, out_dtype=out_dtype,
                                merge_order=merge, column_order=column, rows=rows,
                                rows_col=rows_col, workspace=ws)
    ms = time_launches(V, call, reps, torch.cuda.current_stream())
    alg = algorithmic_bytes(plan, bpv, int(merge) + int(column))
    gbs = alg["total"] / (ms * 1e-3) / 1e9
    res = {"kernel": "preprocess_kernel", "dtype": out_dtype,
           "orders": "+".join(o for o, on in (("merge", merge), ("column", column)) if on),
           "rows": int(plan.total_rows), "ms": ms, "algorithmic_bytes": alg["total"],
           "GB/s": gbs, "frac": gbs / HBM_PEAK_GBPS,
           "images/s": sum(batch.frame_counts) / (ms * 1e-3)}
    return res, (rows if merge else rows_col)


def merge_only_leg(V, batch, plan, src, rows, ws, reps: int) -> dict:
    """The throughput batch in float32, merge-block order only: the
    configuration the 60%-of-HBM target is stated on (3.02 ms)."""
    res, _ = pixel_rates(V, batch, plan, src, "f32", True, False, reps, rows=rows, ws=ws)
    res["target_ms_at_60pct_of_peak"] = res["algorithmic_bytes"] / (0.6 * HBM_PEAK_GBPS * 1e9) * 1e3
    return res


def large_batch_leg(V, workloads, reps: int) -> dict:
    """16 RGB 6000x4000 images downscaled to 3520x2336, bf16, merge order:
    the bilinear path at size.  Beside it, the stock-HF contrast path on the
    same resized batch: its kernel rate and the pixel shift between the two
    paths' rows, in standard deviations."""
    import torch

    log("large batch: generating 16 x 6000x4000")
    batch = workloads.large_16_6000x4000()
    plan = V.plan_batch(batch.shapes)
    src = V.processor.upload_sources(batch.packed, plan)
    batch.packed = None
    res, rows = pixel_rates(V, batch, plan, src, "bf16", True, False, reps)
    res = {"workload": "large_16_6000x4000", **res}
    log("large batch: stock-HF contrast path")
    res["hf_contrast"] = hf_contrast_rates(V, batch, plan, src, rows, reps)
    del rows, src
    torch.cuda.empty_cache()
    return res


def single_image_leg(V, workloads, calls: int) -> dict:
    """One 300x200 RGB image (resized to 288x192, float32): latency bound.
    us_per_call is the host clock over `calls` back-to-back preprocess calls
    with the outputs and workspace kept (synchronised once at the end);
    us_per_call_allocating lets preprocess allocate them each call; kernel_us
    is the launch-event time of the kernel alone.  The stock path's shift on
    this uniform-noise image is beside it."""
    import numpy as np
    import torch

    batch = workloads.single_rgb_300x200()
    plan = V.plan_batch(batch.shapes)
    src = V.processor.upload_sources(batch.packed, plan)
    rows = torch.empty((plan.total_rows, 1536), dtype=torch.float32, device="cuda")
    ws = torch.empty(V.workspace_bytes(1), dtype=torch.uint8, device="cuda")
    call = lambda: V.preprocess(src, plan, mean=batch.mean, std=batch.std, rows=rows, workspace=ws)
    for _ in range(50):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        call()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / calls * 1e6
    t0 = time.perf_counter()
    for _ in range(calls):
        V.preprocess(src, plan, mean=batch.mean, std=batch.std)
    torch.cuda.synchronize()
    us_alloc = (time.perf_counter() - t0) / calls * 1e6
    kernel_ms = time_launches(V, call, 200, torch.cuda.current_stream())
    res = {"workload": "single_rgb_300x200", "rows": int(plan.total_rows), "us_per_call": us,
           "us_per_call_allocating": us_alloc, "kernel_us": kernel_ms * 1e3, "calls": calls,
           "images/s": 1e6 / us}
    res["hf_contrast"] = hf_contrast_rates(V, batch, plan, src, rows, 20)
    return res


def calibrate_copy(gib: float, reps: int):
    """A plain elementwise copy kernel of known size (read N bytes, write N
    bytes) for scaling the HBM byte counters."""
    import torch

    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mul(a, 1.0, out=b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"calibration": "elementwise copy (torch.mul by 1.0)", "bytes_read": 4 * n,
                      "bytes_written": 4 * n, "launches": reps + 1, "ms_per_launch": ms,
                      "GB/s": 8 * n / (ms * 1e-3) / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="throughput_512_1024")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=512)
    ap.add_argument("--gather", action="store_true",
                    help="also time the standalone column_permute gather kernel")
    ap.add_argument("--no-vit-tables", action="store_true",
                    help="skip timing the ViT index-table kernels on the same batch")
    ap.add_argument("--no-embed", action="store_true",
                    help="skip timing the patch embedding on the same batch's rows")
    ap.add_argument("--no-hf", action="store_true",
                    help="skip timing the stock-HF contrast path on the same batch")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the other configurations (float32 merge order only, the "
                         "6000x4000 batch, the single image)")
    ap.add_argument("--calibrate-copy", type=float, default=0.0, metavar="GIB",
                    help="only run a plain copy kernel of this size (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this pixel path runs on one GPU only (asked for {args.gpus} GPUs, "
              f"WORLD_SIZE={world}); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy > 0:
        calibrate_copy(args.calibrate_copy, max(args.steps, 1))
        return

    import vision_image_preprocessing_amd as V
    import workloads

    V.load()  # fails loudly if the HIP library is not built
    log("generating", args.workload)
    batch = workloads.WORKLOADS[args.workload]()
    t_plan = time.perf_counter()
    if batch.is_media:
        plan = V.plan_media(batch.items, video_budget=batch.video_budget)
    else:
        plan = V.plan_batch(batch.shapes)
    plan_ms = (time.perf_counter() - t_plan) * 1e3
    torch.cuda.synchronize()
    t_up = time.perf_counter()
    src = V.processor.upload_sources(batch.packed, plan)
    torch.cuda.synchronize()
    upload_ms = (time.perf_counter() - t_up) * 1e3
    # again, with the pinned staging chunks already allocated
    t_up = time.perf_counter()
    src = V.processor.upload_sources(batch.packed, plan)
    torch.cuda.synchronize()
    upload_warm_ms = (time.perf_counter() - t_up) * 1e3
    out_dtype = batch.out_dtype
    tdtype = torch.float32 if out_dtype == "f32" else torch.bfloat16
    bpv = 4 if out_dtype == "f32" else 2
    rows = torch.empty((plan.total_rows, 1536), dtype=tdtype, device="cuda")
    rows_col = torch.empty_like(rows) if batch.column_order else None
    ws = torch.empty(V.workspace_bytes(len(plan)), dtype=torch.uint8, device="cuda")
    alg = algorithmic_bytes(plan, bpv, 2 if batch.column_order else 1)

    def step():
        V.preprocess(src, plan, mean=batch.mean, std=batch.std, out_dtype=out_dtype,
                     merge_order=True, column_order=batch.column_order, rows=rows,
                     rows_col=rows_col, workspace=ws)

    log("warmup", args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Kernel time: the library records these events on the launch stream
    # right before and after each fused-kernel launch (the per-call
    # descriptor upload falls outside).  Step time: events around all steps.
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for ev in starts + ends:
        ev.record(stream)  # creates the underlying hipEvent_t
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    dispatch0 = V.dispatch_count()
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(args.steps):
        V.set_launch_events(starts[i], ends[i])
        step()
    t_end.record(stream)
    V.set_launch_events(None, None)
    torch.cuda.synchronize()
    assert V.dispatch_count() == dispatch0 + args.steps
    total_ms = t_begin.elapsed_time(t_end)
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    mean_launch_ms = float(np.mean(per_launch_ms))
    log(f"timed {args.steps} steps: {total_ms:.3f} ms")

    n_img = sum(batch.frame_counts)  # images, or frames of a video batch
    unit = "frames/s" if batch.is_media else "images/s"
    achieved = alg["total"] / (mean_launch_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.workload)
    result = {
        "metric": METRIC,
        "value": n_img * args.steps / (total_ms * 1e-3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": out_dtype,
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            ("frames" if batch.is_media else "images"): n_img,
            "source": "uint8 " + ("mixed sizes" if len(set(batch.shapes)) > 1 else
                                  "{}x{}x{}".format(*batch.shapes[0])) +
                      (f", {len(batch)} clips" if batch.is_media else ""),
            "output": f"{out_dtype} rows [{plan.total_rows}, 1536]" +
                      (" in merge-block and column order" if batch.column_order else
                       " in merge-block order"),
            "statistics": "ImageNet" if tuple(batch.mean) == workloads.IMAGENET_MEAN else "CLIP",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
        },
        "algorithmic_bytes_per_step": alg,
        "kernel": "preprocess_kernel<{}, {}>".format("float" if out_dtype == "f32" else "bf16",
                                                     "clips" if batch.is_media else "stills"),
        "launch_ms_mean": mean_launch_ms,
        "launch_ms_min": float(np.min(per_launch_ms)),
        "launch_ms_median": float(np.median(per_launch_ms)),
        "published_throughput": "none (the pages publish no throughput for this path)",
        # host work outside the timed region: the geometry plan, and the one
        # copy of the packed sources from pageable host memory into HBM
        "host": {"plan_ms": plan_ms, "source_upload_ms": upload_ms,
                 "source_upload_GB/s": alg["read"] / (upload_ms * 1e-3) / 1e9,
                 "source_upload_warm_ms": upload_warm_ms,
                 "source_upload_warm_GB/s": alg["read"] / (upload_warm_ms * 1e-3) / 1e9},
    }

    if args.gather and rows_col is not None:
        gathered = torch.empty_like(rows)
        for _ in range(2):
            V.column_permute(plan.desc, rows, gathered, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            V.column_permute(plan.desc, rows, gathered, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gb = 2 * plan.total_rows * 1536 * bpv / (ms * 1e-3) / 1e9
        result["column_permute_gather"] = {"ms": ms, "GB/s": gb, "frac": gb / HBM_PEAK_GBPS}
        del gathered

    if not args.no_legs and args.workload == "throughput_512_1024":
        log("float32, merge-block order only")
        result["merge_order_f32"] = merge_only_leg(V, batch, plan, src, rows, ws, reps=10)

    if not args.no_vit_tables:
        log("vit tables")
        result["vit_tables"] = vit_tables_rates(V, plan, ws, reps=10)

    if not args.no_hf and not batch.is_media:
        log("stock-HF contrast path")
        result["hf_contrast"] = hf_contrast_rates(V, batch, plan, src, rows, reps=5)

    if not args.no_embed:
        log("patch embed")
        result["patch_embed"] = patch_embed_rates(V, batch, plan, src, ws, reps=5)

    if not args.no_legs and args.workload == "throughput_512_1024":
        del rows, rows_col, src
        torch.cuda.empty_cache()
        result["large_16_6000x4000"] = large_batch_leg(V, workloads, reps=10)
        log("single image")
        result["single_rgb_300x200"] = single_image_leg(V, workloads, calls=2000)

    if not args.no_cpu_baseline:
        threads = host_threads()
        log("cpu baseline (oracle)", args.cpu_sample, "images,", threads, "threads")
        result["cpu_baseline"] = cpu_baseline(batch, plan, args.cpu_sample, threads, bpv)
        log("cpu baseline (oracle), one thread")
        result["cpu_baseline"]["single_thread"] = cpu_baseline(batch, plan, min(args.cpu_sample, 32), 1, bpv)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
