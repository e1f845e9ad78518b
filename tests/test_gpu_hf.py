"""GPU parity for the stock-HF contrast path: the HIP kernel (through the C
ABI) against the oracle, which is itself pinned bitwise to PIL and to
transformers' Qwen2-VL processor.

Bar: bit-exact.  The path is integer up to a per-byte float32 table (the
resize taps are fixed-point, the rescale and normalisation depend only on
the byte), so float32 rows must equal the oracle's exactly and bf16 rows
must equal the oracle's float32 rounded to nearest even, bit for bit.
Outputs are prefilled with NaN so an unwritten element fails.
"""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MEAN01 = (0.485, 0.456, 0.406)
STD01 = (0.229, 0.224, 0.225)


def _say(*a):
    print("[gpu-hf]", *a, flush=True)


@pytest.fixture(scope="module")
def V():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vision_image_preprocessing_amd as V
    V.load()
    return V


def _run(V, batch, out_dtype="f32", merge=True, column=False, min_pixels=None, max_pixels=None):
    plan = V.plan_batch_hf(batch.shapes, min_pixels=min_pixels, max_pixels=max_pixels, check=False)
    src = V.processor.upload_sources(batch.packed, plan)
    tdtype = torch.float32 if out_dtype == "f32" else torch.bfloat16
    n = max(plan.total_rows, 1)
    rows = torch.full((n, 1536), float("nan"), dtype=tdtype, device="cuda") if merge else None
    rows_col = torch.full((n, 1536), float("nan"), dtype=tdtype, device="cuda") if column else None
    before = V.dispatch_count()
    out = V.preprocess_hf(src, plan, mean=MEAN01, std=STD01, out_dtype=out_dtype, merge_order=merge,
                          column_order=column, rows=rows, rows_col=rows_col)
    torch.cuda.synchronize()
    if plan.total_rows > 0:
        assert V.dispatch_count() == before + 1
    return plan, out


def _check(V, batch, plan, out, out_dtype, items=None, min_pixels=None, max_pixels=None):
    bounds = {}
    if min_pixels is not None:
        bounds["min_pixels"] = min_pixels
    if max_pixels is not None:
        bounds["max_pixels"] = max_pixels
    for i in (range(len(batch)) if items is None else items):
        h, w, c = batch.shapes[i]
        st, oh, ow = oracle.hf_smart_resize_status(h, w, **bounds)
        d = plan.desc[i]
        assert d["status"] == st, (i, batch.shapes[i])
        if st != 0:
            continue
        assert (d["dst_h"], d["dst_w"]) == (oh, ow)
        ref = oracle.hf_preprocess_image(batch.image(i), oh, ow, MEAN01, STD01)
        r0, r1 = int(d["row_offset"]), int(d["row_offset"] + d["rows"])
        orders = [("merge", out["pixel_values"], None), ("col", out["pixel_values_col"],
                                                         oracle.column_permutation(1, oh // 16, ow // 16))]
        for name, t, perm in orders:
            if t is None:
                continue
            want = ref if perm is None else ref[perm]
            got = t[r0:r1]
            if out_dtype == "f32":
                g = got.cpu().numpy()
                assert np.array_equal(g, want), (name, i, batch.shapes[i], float(np.nanmax(np.abs(g - want))))
            else:
                g = got.cpu().view(torch.int16).numpy().astype(np.uint16)
                assert np.array_equal(g, oracle.to_bf16_bits(want)), (name, i, batch.shapes[i])


# (96, 128, 3) and (96, 96, 4) are left at their size (the direct path);
# the rest resize one axis or both.
SHAPES = [(200, 300, 3), (45, 77, 4), (16, 192, 3), (8, 500, 3), (31, 31, 4), (1, 64, 3), (1, 1, 3),
          (96, 128, 3), (96, 200, 4), (300, 128, 3), (513, 257, 3), (1000, 33, 4), (700, 1000, 3),
          (129, 4095, 3), (2, 3, 4), (96, 96, 4)]


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_ragged_batch_bitwise(V, out_dtype):
    _say("ragged", out_dtype)
    b = W.uniform_images(SHAPES, seed=81)
    plan, out = _run(V, b, out_dtype, merge=True, column=True)
    _check(V, b, plan, out, out_dtype)


@pytest.mark.parametrize("seed,out_dtype", [(93, "f32"), (94, "f32"), (95, "bf16")])
def test_random_shapes_bitwise(V, seed, out_dtype):
    """60 random images: sides log-uniform in [1, 700] on each axis, so
    upscales of sides shorter than the tap count, mild and strong
    downscales and sizes the stock geometry leaves alone all occur; RGB and
    RGBA, both orders, every row compared with the oracle bit for bit."""
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(60):
        h, w = (int(np.exp(rng.uniform(0.0, np.log(700.0)))) for _ in range(2))
        shapes.append((max(h, 1), max(w, 1), int(rng.choice([3, 4]))))
    _say("random shapes", seed, out_dtype)
    b = W.uniform_images(shapes, seed=seed)
    plan, out = _run(V, b, out_dtype, merge=True, column=True)
    _check(V, b, plan, out, out_dtype)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_mild_resizes_bitwise(V, out_dtype):
    """A batch of mild up- and downscales under the stock geometry (every
    tile within 64 source columns and band rows, windows of at most 12
    taps) runs the matrix-core instance; same bar.  (The ragged batch above
    runs it too, with identity-size items; the random batches, which hold
    strong downscales, run the dot-product instance.)"""
    _say("mild resizes", out_dtype)
    b = W.uniform_images([(200, 300, 3), (300, 200, 4), (250, 250, 3), (90, 500, 4), (1000, 700, 3),
                          (1000, 1400, 4), (2000, 1500, 3)], seed=88)
    before = V.hf_matrix_dispatch_count()
    plan, out = _run(V, b, out_dtype, merge=True, column=True)
    assert V.hf_matrix_dispatch_count() == before + 1
    _check(V, b, plan, out, out_dtype)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_matrix_core_edge_cases_bitwise(V, out_dtype):
    """The matrix-core instance where its reads run past what a tile needs.
    Sources narrower than a tile's 64-column read (20x30 RGB, 40x21 RGBA,
    33x61) put the rows past a tile's band partly inside the tile's source
    resource. An axis that keeps its length (50x160, 160x53) runs one tap of
    weight 1. 301x157 RGBA has odd rows. The last item's vertical upscale
    (19 -> 64 rows) is the last table in the batch, so the digit planes of
    its last record are read past the record, into the tables' zero tail.
    The instance that ran is checked; same bar."""
    shapes = [(20, 30, 3), (40, 21, 4), (33, 61, 3), (50, 160, 3), (160, 53, 4), (301, 157, 4), (19, 44, 3)]
    _say("matrix-core edge cases", out_dtype)
    b = W.uniform_images(shapes, seed=89)
    before = V.hf_matrix_dispatch_count()
    plan, out = _run(V, b, out_dtype, merge=True, column=True)
    assert V.hf_matrix_dispatch_count() == before + 1
    _check(V, b, plan, out, out_dtype)


def test_column_order_only(V):
    _say("column only")
    b = W.uniform_images(SHAPES[:8], seed=82)
    plan, out = _run(V, b, "f32", merge=False, column=True)
    _check(V, b, plan, out, "f32")


def test_rgba_alpha_is_ignored(V):
    """Two RGBA images with the same RGB bytes and different alpha give the
    same rows (the stock path drops alpha)."""
    _say("alpha ignored")
    b = W.uniform_images([(120, 200, 4), (120, 200, 4)], seed=83)
    first, second = b.image(0), b.image(1)
    second[..., :3] = first[..., :3]
    second[..., 3] = 255 - first[..., 3]
    plan, out = _run(V, b, "f32")
    n = int(plan.desc["rows"][0])
    assert torch.equal(out["pixel_values"][:n], out["pixel_values"][n:2 * n])
    _check(V, b, plan, out, "f32")


def test_strong_downscale_row_groups(V):
    """A small pixel ceiling forces a ~60x downscale: the vertical taps of 32
    output rows no longer fit the LDS band, so the kernel works in smaller
    row groups."""
    _say("strong downscale")
    b = W.uniform_images([(4000, 6000, 3), (3000, 300, 3)], seed=84)
    before = V.hf_matrix_dispatch_count()
    plan, out = _run(V, b, "f32", min_pixels=4096, max_pixels=8192)
    assert plan.desc["dst_h"][0] < 200
    # windows of hundreds of taps: the dot-product instance, not the matrix cores
    assert V.hf_matrix_dispatch_count() == before
    _check(V, b, plan, out, "f32", min_pixels=4096, max_pixels=8192)


def test_large_images(V):
    _say("large 6000x4000")
    b = W.large_16_6000x4000(n=2)
    plan, out = _run(V, b, "bf16")
    _check(V, b, plan, out, "bf16")


def test_back_to_back_and_empty(V):
    _say("back to back")
    b1 = W.uniform_images([(640, 480, 3), (77, 45, 4)], seed=85)
    p1, o1 = _run(V, b1, "f32")
    b2 = W.uniform_images([(64, 64, 3)], seed=86)
    p2, o2 = _run(V, b2, "f32", column=True)
    _check(V, b1, p1, o1, "f32")
    _check(V, b2, p2, o2, "f32")
    plan = V.plan_batch_hf(np.zeros((0, 3), np.int32))
    src = torch.zeros(16, dtype=torch.uint8, device="cuda")
    V.preprocess_hf(src, plan)


def test_contrast_on_gpu(V):
    """The page's shift, measured on the GPU: MiMo and stock rows for the
    same images, in units of the channel standard deviation."""
    _say("contrast")
    b = W.uniform_images([(600, 900, 3), (1080, 1920, 3)], seed=87)
    plan_m = V.plan_batch(b.shapes)
    plan_h = V.plan_batch_hf(b.shapes)
    assert np.array_equal(plan_m.image_grid_thw, plan_h.image_grid_thw)
    src = V.processor.upload_sources(b.packed, plan_m)
    m = V.preprocess(src, plan_m, mean=MEAN01, std=STD01)["pixel_values"]
    h = V.preprocess_hf(src, plan_h, mean=MEAN01, std=STD01)["pixel_values"]
    torch.cuda.synchronize()
    diff = (m - h).abs()
    assert 0.0 < float(diff.mean()) < 0.5
