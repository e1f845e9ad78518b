"""GPU parity for the video frames path: the HIP kernel (through the C ABI)
against the oracle's prepare_video_frames pixel part.

Every clip is planned by the library (mimo_plan_frames with the per-frame
ceiling from mimo_video_max_pixels) and, independently, by the oracle
(video_max_pixels, smart_resize); geometry must agree exactly.  Rows are
compared in full: float32 within 1e-4, bf16 within 1 ulp of the oracle's
float32 value rounded to nearest even.  Outputs are prefilled with NaN so an
unwritten element fails.

Cases: odd and even frame counts (an odd count repeats its last frame),
one-frame items mixed with clips (still images), RGB and RGBA, identity
tiles (resized size equals the source) and bilinear ones, merge-block and
column order, back-to-back calls, and the 8-clip 1280x720 workload in full.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32_TOL = 1e-4


def _say(*a):
    print("[gpu-video]", *a, flush=True)


@pytest.fixture(scope="module")
def V():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vision_image_preprocessing_amd as V
    V.load()
    return V


def _oracle_geometry(b, i):
    """(out_h, out_w) from the oracle alone: the clip's per-frame ceiling,
    then smart_resize."""
    f = b.frame_counts[i]
    h, w, _ = b.shapes[i]
    budget = b.video_budget[i] if b.video_budget is not None else 0
    mx = oracle.video_max_pixels(f, budget) if budget > 0 else oracle.MAX_PIXELS
    return oracle.smart_resize(h, w, max_pixels=mx)


def _run(V, b, out_dtype, merge=True, column=False):
    plan = V.plan_media(b.items, video_budget=b.video_budget)
    src = V.processor.upload_sources(b.packed, plan)
    tdtype = torch.float32 if out_dtype == "f32" else torch.bfloat16
    n = max(plan.total_rows, 1)
    rows = torch.full((n, 1536), float("nan"), dtype=tdtype, device="cuda") if merge else None
    rows_col = torch.full((n, 1536), float("nan"), dtype=tdtype, device="cuda") if column else None
    before = V.dispatch_count()
    out = V.preprocess(src, plan, mean=b.mean, std=b.std, out_dtype=out_dtype, merge_order=merge,
                       column_order=column, rows=rows, rows_col=rows_col)
    torch.cuda.synchronize()
    if plan.total_rows > 0:
        assert V.dispatch_count() == before + 1
    return plan, out


def _to_np(t):
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _assert_close(got, ref, out_dtype, what=""):
    assert got.shape == ref.shape, what
    assert np.isfinite(got).all(), f"{what}: unwritten or non-finite elements"
    if out_dtype == "f32":
        err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        assert err.max() <= F32_TOL, (what, float(err.max()), np.unravel_index(err.argmax(), err.shape))
        # tighter: the resize is the oracle's float32 arithmetic in the same
        # order; only the standardisation differs (a product with the rounded
        # 1/S against a quotient by S), by at most 3 float32 ulps of the value
        bound = 4.0 * 2.0 ** -24 * np.maximum(np.abs(ref.astype(np.float64)), 1.0)
        assert (err <= bound).all(), (what, "beyond 4 ulps", float((err / bound).max()))
    else:
        want = oracle.to_bf16_bits(ref).astype(np.int64)
        have = (got.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)

        def ordered(bits):
            return np.where(bits & 0x8000, -(bits & 0x7FFF), bits)
        ulps = np.abs(ordered(have) - ordered(want))
        assert ulps.max() <= 1, (what, int(ulps.max()))


def _check(V, b, plan, out, out_dtype, items=None, column=False):
    m, s = oracle.stats255(b.mean, b.std)
    idx = list(range(len(b))) if items is None else list(items)
    for i in idx:
        f = b.frame_counts[i]
        oh, ow = _oracle_geometry(b, i)
        d = plan.desc[i]
        gt = -(-f // 2)
        assert (d["dst_h"], d["dst_w"], d["frames"]) == (oh, ow, f), i
        assert (d["grid_t"], d["grid_h"], d["grid_w"]) == (gt, oh // 16, ow // 16), i
        assert d["rows"] == gt * (oh // 16) * (ow // 16), i

    def ref_rows(i):
        d = plan.desc[i]
        return oracle.preprocess_video(b.clip(i), int(d["dst_h"]), int(d["dst_w"]), m, s)

    with ThreadPoolExecutor(max_workers=8) as ex:
        refs = list(ex.map(ref_rows, idx))
    for i, ref in zip(idx, refs):
        d = plan.desc[i]
        r0, r1 = int(d["row_offset"]), int(d["row_offset"] + d["rows"])
        what = f"item {i} {b.items[i]}"
        if out["pixel_values"] is not None:
            _assert_close(_to_np(out["pixel_values"][r0:r1]), ref, out_dtype, what)
        if column:
            perm = oracle.column_permutation(int(d["grid_t"]), int(d["grid_h"]), int(d["grid_w"]))
            _assert_close(_to_np(out["pixel_values_col"][r0:r1]), ref[perm], out_dtype,
                          "col " + what)


MIXED = [
    (2, 64, 96, 3),      # even pair, upscaled (below min_pixels)
    (5, 37, 29, 4),      # odd: last frame repeated; RGBA; sub-factor sides
    (1, 200, 300, 3),    # a still image among clips
    (3, 96, 128, 3),     # identity tiles (96x128 already a multiple of 32)
    (4, 96, 96, 4),      # identity tiles, RGBA
    (6, 120, 200, 3),    # bilinear
    (7, 16, 192, 3),     # sub-factor short side, odd count
    (1, 1, 1, 3),        # one pixel, one frame
    (9, 45, 77, 4),
    (4, 1080, 1920, 3),  # big frames under a clip budget
]
BUDGET = [0, 0, 0, 0, 0, 0, 0, 0, 0, 1 << 22]


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_mixed_clips_and_stills_full(V, out_dtype):
    _say("mixed clips", out_dtype)
    b = W.media_batch(MIXED, seed=61, video_budget=BUDGET)
    plan, out = _run(V, b, out_dtype, merge=True, column=True)
    _check(V, b, plan, out, out_dtype, column=True)
    # the standalone gather kernel reproduces the fused column order
    ws = torch.empty(V.workspace_bytes(len(plan)), dtype=torch.uint8, device="cuda")
    gathered = torch.empty_like(out["pixel_values"])
    V.column_permute(plan.desc, out["pixel_values"], gathered, ws)
    torch.cuda.synchronize()
    assert torch.equal(gathered, out["pixel_values_col"])


@pytest.mark.parametrize("seed,out_dtype", [(71, "f32"), (72, "f32"), (73, "bf16")])
def test_random_clips_full(V, seed, out_dtype):
    """40 random items: 1 to 7 frames (odd counts repeat their last frame),
    sides log-uniform in [1, 400], RGB and RGBA, a quarter of them under a
    clip pixel budget; both orders, every row against the oracle."""
    rng = np.random.default_rng(seed)
    items, budget = [], []
    for _ in range(40):
        h, w = (int(np.exp(rng.uniform(0.0, np.log(400.0)))) for _ in range(2))
        items.append((int(rng.integers(1, 8)), max(h, 1), max(w, 1), int(rng.choice([3, 4]))))
        budget.append(int(1 << 16) if rng.random() < 0.25 else 0)
    # keep the items the geometry accepts (sub-factor shapes whose upscale
    # exceeds the pixel ceiling are refused)
    pre = V.plan_media(items, video_budget=budget, check=False)
    keep = [i for i in range(len(items)) if pre.desc["status"][i] == 0]
    items, budget = [items[i] for i in keep], [budget[i] for i in keep]
    _say("random clips", seed, out_dtype, len(items))
    b = W.media_batch(items, seed=seed, video_budget=budget)
    plan, out = _run(V, b, out_dtype, merge=True, column=True)
    _check(V, b, plan, out, out_dtype, column=True)


def test_video_processor_call(V):
    """Clips and a still through VideoProcessor equal the planned path's
    rows (and so the oracle's)."""
    _say("VideoProcessor")
    items = [(4, 64, 96, 3), (3, 45, 77, 4), (1, 200, 300, 3)]
    b = W.media_batch(items, seed=69, video_budget=[1 << 16, 0, 0])
    arrays = [b.clip(i) for i in range(len(b))]
    out = V.VideoProcessor(image_mean=b.mean, image_std=b.std)(arrays, video_budget=[1 << 16, 0, 0],
                                                              column_order=True)
    plan, ref = _run(V, b, "f32", merge=True, column=True)
    assert torch.equal(out["pixel_values"], ref["pixel_values"][:plan.total_rows])
    assert torch.equal(out["pixel_values_col"], ref["pixel_values_col"][:plan.total_rows])
    assert np.array_equal(out["video_grid_thw"].numpy(), plan.grid_thw)
    _check(V, b, plan, out, "f32", column=True)


def test_clip_strong_downscale_reads_taps_directly(V):
    """Distinct frames whose band exceeds the LDS budget (a 7-10x downscale
    under a small per-frame ceiling) take the direct-read route, frame
    after frame; same bar."""
    _say("clip strong downscale")
    b = W.media_batch([(2, 3000, 2600, 3), (3, 2048, 4000, 4)], seed=68, video_budget=[1 << 17, 1 << 17])
    plan, out = _run(V, b, "f32", merge=True, column=True)
    assert plan.desc["dst_h"][0] * 7 <= 3000  # band far beyond the LDS budget
    _check(V, b, plan, out, "f32", column=True)


def test_column_order_only(V):
    _say("column order only")
    b = W.media_batch(MIXED[:7], seed=62)
    plan, out = _run(V, b, "f32", merge=False, column=True)
    _check(V, b, plan, out, "f32", column=True)


def test_rgba_alpha_extremes_in_clips(V):
    """Transparent, opaque and half alpha in every frame, distinct per frame."""
    _say("rgba clip extremes")
    b = W.media_batch([(5, 64, 96, 4), (2, 33, 70, 4)], seed=63)
    for i in range(len(b)):
        clip = b.clip(i)
        clip[..., 3][:, ::3] = 0
        clip[..., 3][:, 1::3] = 255
    plan, out = _run(V, b, "f32")
    _check(V, b, plan, out, "f32")


def test_frames_are_not_duplicated(V):
    """With distinct frames the two temporal slots differ (the still-image
    duplication must not leak into clips), and a one-frame item keeps them
    equal."""
    _say("temporal slots")
    b = W.media_batch([(2, 96, 128, 3), (1, 96, 128, 3)], seed=64)
    plan, out = _run(V, b, "f32")
    v = out["pixel_values"].view(-1, 3, 2, 256)
    n0 = int(plan.desc[0]["rows"])
    assert not torch.equal(v[:n0, :, 0], v[:n0, :, 1])
    assert torch.equal(v[n0:, :, 0], v[n0:, :, 1])


def test_back_to_back_video_then_images(V):
    _say("back to back")
    b1 = W.media_batch([(6, 120, 200, 3), (3, 45, 77, 4)], seed=65)
    p1, o1 = _run(V, b1, "bf16", column=True)
    b2 = W.media_batch([(1, 300, 200, 3), (1, 64, 64, 4)], seed=66)
    p2, o2 = _run(V, b2, "bf16", column=True)
    _check(V, b1, p1, o1, "bf16", column=True)
    _check(V, b2, p2, o2, "bf16", column=True)


def test_plan_frames_matches_plan_geometry_on_gpu(V):
    """One-frame items through mimo_plan_frames give the same rows as the
    still-image planner on the same bytes."""
    _say("stills via frames planner")
    shapes = [(200, 300, 3), (45, 77, 4), (513, 257, 3)]
    b = W.uniform_images(shapes, seed=67)
    pg = V.plan_batch(b.shapes)
    pf = V.plan_media([(1,) + s for s in shapes])
    assert np.array_equal(pg.desc, pf.desc)
    src = V.processor.upload_sources(b.packed, pg)
    a = V.preprocess(src, pg)["pixel_values"]
    c = V.preprocess(src, pf)["pixel_values"]
    torch.cuda.synchronize()
    assert torch.equal(a, c)


def test_workload_video_8x64_1280x720(V):
    _say("video_8x64_1280x720 (bf16)")
    b = W.video_8x64_1280x720()
    plan, out = _run(V, b, "bf16")
    assert set(plan.desc["dst_h"]) == {512} and set(plan.desc["dst_w"]) == {960}
    assert plan.total_rows == 8 * 32 * 32 * 60
    _check(V, b, plan, out, "bf16")
