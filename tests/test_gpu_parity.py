"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: geometry, row counts and permutation indices bit-exact; float32 pixels
within 1e-4 in normalised units, and within 4 float32 ulps of the oracle's
value (of max(|value|, 1)), since only the standardisation's rounding
differs; bf16 within 1 bf16 ulp of the oracle's
float32 value rounded to nearest even; both frames bitwise identical; every
output element written (outputs are prefilled with NaN).

Small batches are compared in full; the five workloads at full size are
compared in full where the oracle takes seconds, and on sampled rows (the
oracle computes them one element at a time) plus whole-output properties
where it does not.
"""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32_TOL = 1e-4


def _say(*a):
    print("[gpu-parity]", *a, flush=True)


@pytest.fixture(scope="module")
def V():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vision_image_preprocessing_amd as V
    V.load()
    return V


def _run(V, batch, out_dtype="f32", merge=True, column=False, min_pixels=None,
         max_pixels=None, check=True):
    plan = V.plan_batch(batch.shapes, min_pixels=min_pixels, max_pixels=max_pixels, check=check)
    src = V.processor.upload_sources(batch.packed, plan)
    tdtype = torch.float32 if out_dtype == "f32" else torch.bfloat16
    n = max(plan.total_rows, 1)
    rows = torch.full((n, 1536), float("nan"), dtype=tdtype, device="cuda") if merge else None
    rows_col = torch.full((n, 1536), float("nan"), dtype=tdtype, device="cuda") if column else None
    before = V.dispatch_count()
    out = V.preprocess(src, plan, mean=batch.mean, std=batch.std, out_dtype=out_dtype,
                       merge_order=merge, column_order=column, rows=rows, rows_col=rows_col)
    torch.cuda.synchronize()
    if plan.total_rows > 0:
        assert V.dispatch_count() == before + 1  # the HIP kernel ran
    return plan, out


def _stats(batch):
    return oracle.stats255(batch.mean, batch.std)


def _assert_close(got, ref, out_dtype, what=""):
    """got: float32 view of the GPU rows (bf16 widened); ref: oracle float32."""
    assert got.shape == ref.shape, what
    if out_dtype == "f32":
        err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        assert np.isfinite(got).all(), what
        assert err.max() <= F32_TOL, (what, float(err.max()), np.unravel_index(err.argmax(), err.shape))
        # tighter: the resize is the oracle's float32 arithmetic in the same
        # order; only the standardisation differs (a product with the rounded
        # 1/S against a quotient by S), by at most 3 float32 ulps of the value
        bound = 4.0 * 2.0 ** -24 * np.maximum(np.abs(ref.astype(np.float64)), 1.0)
        assert (err <= bound).all(), (what, "beyond 4 ulps", float((err / bound).max()))
    else:
        want = oracle.to_bf16_bits(ref).astype(np.int32)
        have = got.astype(np.float32).view(np.uint32) >> 16
        # ordered integer image of bf16 bit patterns (sign-magnitude -> two's complement)
        def ordered(b):
            b = b.astype(np.int64)
            return np.where(b & 0x8000, -(b & 0x7FFF), b)
        ulps = np.abs(ordered(have) - ordered(want))
        assert ulps.max() <= 1, (what, int(ulps.max()))


def _to_np(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _check_full(V, batch, plan, out, out_dtype, images=None, column=False, min_pixels=None,
                max_pixels=None):
    m, s = _stats(batch)
    rows = out["pixel_values"]
    rows_col = out["pixel_values_col"]
    idx = range(len(batch)) if images is None else images
    for i in idx:
        d = plan.desc[i]
        if d["status"] != 0:
            continue
        h, w, c = batch.shapes[i]
        bounds = dict(min_pixels=oracle.MIN_PIXELS if min_pixels is None else min_pixels,
                      max_pixels=oracle.MAX_PIXELS if max_pixels is None else max_pixels)
        g, nrows, _ = oracle.image_grid(h, w, **bounds)
        assert (d["grid_t"], d["grid_h"], d["grid_w"]) == g and d["rows"] == nrows
        ref = oracle.preprocess_image(batch.image(i), int(d["dst_h"]), int(d["dst_w"]), m, s)
        r0, r1 = int(d["row_offset"]), int(d["row_offset"] + d["rows"])
        if rows is not None:
            _assert_close(_to_np(rows[r0:r1]), ref, out_dtype, f"image {i} {batch.shapes[i]}")
        if column:
            perm = oracle.column_permutation(1, int(d["grid_h"]), int(d["grid_w"]))
            _assert_close(_to_np(rows_col[r0:r1]), ref[perm], out_dtype, f"col image {i}")


def _check_properties(out):
    for key in ("pixel_values", "pixel_values_col"):
        t = out[key]
        if t is None:
            continue
        assert bool(torch.isfinite(t).all()), f"{key}: unwritten (NaN) or non-finite elements"
        v = t.view(-1, 3, 2, 256)
        assert torch.equal(v[:, :, 0], v[:, :, 1]), f"{key}: frames differ"


# ----------------------------------------------------------- small batches
RAGGED_SHAPES = [
    (200, 300, 3), (45, 77, 4), (16, 192, 3), (8, 500, 3), (31, 31, 3), (1, 64, 3),
    (1, 1, 3), (97, 61, 4), (480, 640, 4), (33, 1000, 3), (1000, 33, 4), (513, 257, 3),
    (64, 64, 3), (96, 352, 3), (37, 29, 4), (700, 1000, 3), (2, 3, 4), (129, 4095, 3),
]


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_ragged_small_batch_full(V, out_dtype):
    _say("ragged small batch", out_dtype)
    b = W.uniform_images(RAGGED_SHAPES, seed=21)
    plan, out = _run(V, b, out_dtype, merge=True, column=True)
    _check_full(V, b, plan, out, out_dtype, column=True)
    _check_properties(out)


@pytest.mark.parametrize("seed", [91, 92])
def test_random_shapes_full(V, seed):
    """120 random images: sides log-uniform in [1, 700] on each axis (so
    every branch of smart_resize, upscales, downscales and identity on a
    multiple of 32 all occur), RGB and RGBA, both row orders, every row
    compared with the oracle."""
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(120):
        h, w = (int(np.exp(rng.uniform(0.0, np.log(700.0)))) for _ in range(2))
        if rng.random() < 0.1:  # land some on multiples of 32 (identity resize)
            h, w = 32 * max(3, h // 32), 32 * max(3, w // 32)
        shapes.append((max(h, 1), max(w, 1), int(rng.choice([3, 4]))))
    _say("random shapes", seed)
    b = W.uniform_images(shapes, seed=seed)
    plan, out = _run(V, b, "f32", merge=True, column=True, check=False)
    _check_full(V, b, plan, out, "f32", column=True)
    _check_properties(out)


def test_rgba_content_and_alpha_extremes(V):
    _say("rgba extremes")
    rng = np.random.default_rng(5)
    imgs = []
    for (h, w) in ((100, 140), (33, 47), (64, 96)):
        im = rng.integers(0, 256, (h, w, 4), dtype=np.uint8)
        im[: h // 3, :, 3] = 0
        im[h // 3: 2 * h // 3, :, 3] = 255
        imgs.append(im)
    b = W._from_images("rgba", imgs, mean=W.CLIP_MEAN, std=W.CLIP_STD, out_dtype="f32")
    plan, out = _run(V, b)
    _check_full(V, b, plan, out, "f32")


def test_large_downscale_uses_global_taps(V):
    """A downscale whose source band exceeds the LDS budget takes the
    direct-read route; results must be the same arithmetic."""
    _say("large downscale")
    b = W.uniform_images([(3000, 2600, 3), (2048, 4000, 4)], seed=8)
    plan, out = _run(V, b, max_pixels=40000)
    assert plan.desc["dst_h"][0] < 3000 / 8
    _check_full(V, b, plan, out, "f32", max_pixels=40000)
    _check_properties(out)


def test_max_size_image(V):
    """1x8192 -> 32x262144 = max_pixels exactly: 32768 rows in one block row."""
    _say("max size image")
    b = W.uniform_images([(1, 8192, 3), (8192, 1, 4)], seed=9)
    plan, out = _run(V, b, column=True)
    assert plan.total_rows == 2 * 32768
    _check_full(V, b, plan, out, "f32", column=True)


def test_failed_images_are_skipped(V):
    _say("failed images")
    shapes = [(64, 64, 3), (32, 6401, 3), (40, 50, 3), (1, 8193, 3), (20, 30, 4)]
    b = W.uniform_images(shapes, seed=10)
    plan, out = _run(V, b, check=False)
    st = plan.desc["status"]
    assert st[1] == V.MIMO_E_ASPECT and st[3] == V.MIMO_E_DEGENERATE
    assert plan.desc["rows"][1] == 0 and plan.desc["rows"][3] == 0
    _check_full(V, b, plan, out, "f32")
    _check_properties(out)


def test_empty_batch(V):
    b = W.uniform_images([], seed=1)
    plan = V.plan_batch(np.zeros((0, 3), dtype=np.int32))
    assert plan.total_rows == 0 and len(plan) == 0
    src = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = V.preprocess(src, plan)
    assert out["pixel_values"].shape == (0, 1536)  # [sum of rows, 1536]
    out = V.ImageProcessor()([])
    assert out["pixel_values"].shape == (0, 1536) and out["image_grid_thw"].shape == (0, 3)
    del b


def test_image_processor_call(V):
    """The processor's call shape: decoded images in, rows and grids out,
    equal to the planned path's rows (and so to the oracle's)."""
    _say("ImageProcessor")
    b = W.uniform_images([(200, 300, 3), (45, 77, 4), (96, 128, 3)], seed=9)
    images = [b.image(i) for i in range(len(b))]
    out = V.ImageProcessor(image_mean=b.mean, image_std=b.std)(images, column_order=True)
    plan, ref = _run(V, b, "f32", merge=True, column=True)
    assert torch.equal(out["pixel_values"], ref["pixel_values"][:plan.total_rows])
    assert torch.equal(out["pixel_values_col"], ref["pixel_values_col"][:plan.total_rows])
    assert np.array_equal(out["image_grid_thw"].numpy(), plan.image_grid_thw)
    _check_full(V, b, plan, out, "f32", column=True)


def test_argument_errors(V):
    b = W.uniform_images([(64, 64, 3)], seed=1)
    plan = V.plan_batch(b.shapes)
    src = V.processor.upload_sources(b.packed, plan)
    rows = torch.empty((plan.total_rows - 1, 1536), device="cuda")
    ws = torch.empty(V.workspace_bytes(1), dtype=torch.uint8, device="cuda")
    with pytest.raises(V.MimoError) as e:
        V.preprocess_batch(plan.desc, src, [0, 0, 0], [1, 1, 1], rows=rows, workspace=ws)
    assert e.value.code == V.MIMO_E_CAPACITY
    rows = torch.empty((plan.total_rows, 1536), device="cuda")
    with pytest.raises(V.MimoError) as e:
        V.preprocess_batch(plan.desc, src, [0, 0, 0], [1, 0, 1], rows=rows, workspace=ws)
    assert e.value.code == V.MIMO_E_INVALID
    with pytest.raises(V.MimoError) as e:
        V.preprocess_batch(plan.desc, src[:100], [0, 0, 0], [1, 1, 1], rows=rows, workspace=ws)
    assert e.value.code == V.MIMO_E_CAPACITY


def test_back_to_back_calls_with_different_batches(V):
    """Two calls in flight on one stream with different plans: the pinned
    descriptor staging must not let the second call clobber the first."""
    _say("back to back")
    b1 = W.uniform_images([(300, 200, 3), (64, 96, 4)], seed=31)
    b2 = W.uniform_images([(31, 700, 3), (500, 500, 3), (5, 9, 4)], seed=32)
    p1, p2 = V.plan_batch(b1.shapes), V.plan_batch(b2.shapes)
    s1, s2 = V.processor.upload_sources(b1.packed, p1), V.processor.upload_sources(b2.packed, p2)
    outs = []
    for _ in range(10):
        outs.append((V.preprocess(s1, p1), V.preprocess(s2, p2)))
    torch.cuda.synchronize()
    _check_full(V, b1, p1, outs[0][0], "f32")
    _check_full(V, b2, p2, outs[-1][1], "f32")
    for o1, o2 in outs[1:]:
        assert torch.equal(o1["pixel_values"], outs[0][0]["pixel_values"])
        assert torch.equal(o2["pixel_values"], outs[0][1]["pixel_values"])


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_output_order_choices_agree(V, out_dtype):
    """Merge-only, column-only and both-orders calls write the same rows; the
    gather kernel maps merge order to the same column order."""
    _say("output order choices", out_dtype)
    b = W.uniform_images(RAGGED_SHAPES[:12] + [(700, 1000, 4), (64, 2048, 3)], seed=41)
    plan_m, out_m = _run(V, b, out_dtype, merge=True, column=False)
    plan_c, out_c = _run(V, b, out_dtype, merge=False, column=True)
    plan_b, out_b = _run(V, b, out_dtype, merge=True, column=True)
    assert torch.equal(out_m["pixel_values"], out_b["pixel_values"])
    assert torch.equal(out_c["pixel_values_col"], out_b["pixel_values_col"])
    _check_properties(out_c)
    ws = torch.empty(V.workspace_bytes(len(plan_m)), dtype=torch.uint8, device="cuda")
    gathered = torch.full_like(out_m["pixel_values"], float("nan"))
    V.column_permute(plan_m.desc, out_m["pixel_values"], gathered, ws)
    torch.cuda.synchronize()
    assert torch.equal(gathered, out_c["pixel_values_col"])
    # column order against the oracle's permutation, image by image
    _check_full(V, b, plan_c, out_c, out_dtype, column=True, images=range(len(b)))


# ------------------------------------------------------ workloads, full size
def test_workload_single_rgb_300x200(V):
    _say("single_rgb_300x200")
    b = W.single_rgb_300x200()
    plan, out = _run(V, b)
    assert plan.total_rows == 216
    _check_full(V, b, plan, out, "f32")
    _check_properties(out)


def test_workload_rgba_64_mixed(V):
    _say("rgba_64_mixed")
    b = W.rgba_64_mixed()
    plan, out = _run(V, b)
    _check_full(V, b, plan, out, "f32")
    _check_properties(out)


def test_workload_subfactor_256(V):
    _say("subfactor_256")
    b = W.subfactor_256()
    plan, out = _run(V, b, column=True)
    # geometry and token counts bit-exact for every image
    for i, (h, w, c) in enumerate(b.shapes):
        g, rows, tok = oracle.image_grid(h, w)
        d = plan.desc[i]
        assert (d["grid_t"], d["grid_h"], d["grid_w"]) == g and d["rows"] == rows, (h, w)
    _check_full(V, b, plan, out, "f32", column=True)
    _check_properties(out)


def _sampled_rows(V, b, plan, out, out_dtype, per_image, seed, column=False):
    m, s = _stats(b)
    rng = np.random.default_rng(seed)
    rows = out["pixel_values"]
    for i in range(len(b)):
        d = plan.desc[i]
        n = int(d["rows"])
        r0 = int(d["row_offset"])
        pick = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, per_image)]))
        gpu = _to_np(rows[torch.from_numpy(r0 + pick).cuda()])
        ref = np.stack([oracle.preprocess_rows(b.image(i), int(d["dst_h"]), int(d["dst_w"]),
                                               m, s, int(r), 1)[0] for r in pick])
        _assert_close(gpu, ref, out_dtype, f"image {i} rows {pick[:4]}...")
        if column:
            perm = oracle.column_permutation(1, int(d["grid_h"]), int(d["grid_w"]))
            dst = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, per_image)]))
            gpu_c = _to_np(out["pixel_values_col"][torch.from_numpy(r0 + dst).cuda()])
            ref_c = np.stack([oracle.preprocess_rows(b.image(i), int(d["dst_h"]), int(d["dst_w"]),
                                                     m, s, int(perm[r]), 1)[0] for r in dst])
            _assert_close(gpu_c, ref_c, out_dtype, f"col image {i}")


def test_workload_large_16_6000x4000_bf16(V):
    _say("large_16_6000x4000 (bf16)")
    b = W.large_16_6000x4000()
    plan, out = _run(V, b, "bf16")
    assert plan.total_rows == 16 * 32120
    assert set(plan.desc["dst_h"]) == {2336} and set(plan.desc["dst_w"]) == {3520}
    _check_properties(out)
    _check_full(V, b, plan, out, "bf16", images=[0, 15])
    _sampled_rows(V, b, plan, out, "bf16", per_image=64, seed=4)


def test_workload_throughput_512_1024(V):
    _say("throughput_512_1024 (merge + column order)")
    b = W.throughput_512_1024()
    plan, out = _run(V, b, "f32", merge=True, column=True)
    assert plan.total_rows == 512 * 4096
    _check_properties(out)
    _check_full(V, b, plan, out, "f32", images=[0, 511], column=True)
    _sampled_rows(V, b, plan, out, "f32", per_image=8, seed=5, column=True)
    # the standalone gather kernel reproduces the fused column-order output
    _say("column_permute gather")
    ws = torch.empty(V.workspace_bytes(len(plan)), dtype=torch.uint8, device="cuda")
    gathered = torch.empty_like(out["pixel_values"])
    V.column_permute(plan.desc, out["pixel_values"], gathered, ws)
    torch.cuda.synchronize()
    assert torch.equal(gathered, out["pixel_values_col"])


def test_side_stream_back_to_back_allocations(V):
    """preprocess on a non-default stream: the outputs and workspace it
    allocates belong to that stream, so allocations made right after on the
    current stream (and overwritten there) cannot take their memory while the
    side stream's table copy and kernel still use it."""
    _say("side stream")
    batch = W.uniform_images([(200, 300, 3), (45, 77, 3), (130, 64, 3)], seed=91)
    plan = V.plan_batch(batch.shapes)
    src = V.processor.upload_sources(batch.packed, plan)
    side = torch.cuda.Stream()
    outs = []
    for rep in range(4):
        out = V.preprocess(src, plan, mean=batch.mean, std=batch.std, column_order=True, stream=side)
        outs.append(out)
        # busy the current stream with fresh allocations of the same sizes,
        # filled with garbage, while the side stream may still be working
        junk = [torch.full((max(plan.total_rows, 1), 1536), 7.0, device="cuda") for _ in range(2)]
        junk.append(torch.full((V.workspace_bytes(len(plan)) + 64,), 255, dtype=torch.uint8, device="cuda"))
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for out in outs:
        _check_properties(out)
        _check_full(V, batch, plan, out, "f32", column=True)
