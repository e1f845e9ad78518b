"""Host-side checks of the C ABI (no GPU needed).

* the library loads and exports every function include/mimo_pre.h declares;
* the host planner (smart_resize, plan_geometry, column_permutation) is
  bit-exact against the oracle on every workload shape and on random sizes;
* argument validation returns the documented codes before touching a GPU.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads as W
import vision_image_preprocessing_amd as V

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mimo_pre.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mimo_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = V.load()
    names = _declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
        assert name in V._abi.SIGNATURES, name


def test_struct_layouts():
    assert V.IMAGE_DESC_DTYPE.itemsize == 64
    assert ctypes.sizeof(V.MimoParams) == 40
    p = V.default_params()
    assert (p.patch_size, p.merge_size, p.temporal_patch_size) == (16, 2, 2)
    assert (p.min_pixels, p.max_pixels, p.max_aspect) == (8192, 8388608, 200.0)


def _all_workload_shapes():
    shapes = [(200, 300, 3)]
    rng = np.random.default_rng(2)
    for _ in range(64):  # the rgba_64_mixed size recipe
        w = int(rng.integers(640, 1921))
        h = int(rng.integers(480, 1081))
        shapes.append((h, w, 4))
    shapes += [(h, w, 3) for (h, w) in W.subfactor_sizes()]
    shapes += [(4000, 6000, 3), (1024, 1024, 3)]
    return shapes


def test_plan_matches_oracle_on_workload_shapes():
    shapes = _all_workload_shapes()
    desc, total_rows, total_src, code = V.plan_geometry(shapes)
    assert code == 0
    rows = src = 0
    for i, (h, w, c) in enumerate(shapes):
        g, n, tok = oracle.image_grid(h, w)
        oh, ow = oracle.smart_resize(h, w)
        d = desc[i]
        assert (d["grid_t"], d["grid_h"], d["grid_w"]) == g
        assert (d["dst_h"], d["dst_w"]) == (oh, ow)
        assert d["rows"] == n and n // 4 == tok
        assert d["row_offset"] == rows and d["src_offset"] == src
        rows += n
        src += h * w * c
    assert (total_rows, total_src) == (rows, src)


@pytest.mark.parametrize("branch", ["full", "subfactor"])
def test_smart_resize_matches_oracle_random(branch):
    rng = np.random.default_rng(17 if branch == "full" else 18)
    for _ in range(30000):
        if branch == "full":
            s = int(rng.integers(32, 5000))
            l = int(rng.integers(s, min(250 * s, 60000)))
        else:
            s = int(rng.integers(1, 32))
            l = int(rng.integers(s, 12000))
        h, w = (s, l) if rng.random() < 0.5 else (l, s)
        st, oh, ow = oracle.smart_resize_status(h, w)
        if st == 0:
            assert V.smart_resize(h, w) == (oh, ow), (h, w)
        else:
            with pytest.raises(V.MimoError) as e:
                V.smart_resize(h, w)
            assert e.value.code == st, (h, w)


def test_smart_resize_per_call_bounds_match_oracle():
    rng = np.random.default_rng(19)
    for _ in range(20000):
        h = int(rng.integers(1, 5000))
        w = int(rng.integers(1, 5000))
        mn = int(rng.integers(0, 100000))
        mx = int(rng.integers(max(mn, 1), mn + 5_000_000))
        p = V.make_params(mn, mx)
        st, oh, ow = oracle.smart_resize_status(h, w, 32, mn, mx)
        if st == 0:
            assert V.smart_resize(h, w, p) == (oh, ow), (h, w, mn, mx)
        else:
            with pytest.raises(V.MimoError) as e:
                V.smart_resize(h, w, p)
            assert e.value.code == st


def test_get_number_of_image_patches_matches_oracle():
    """The processor's get_number_of_image_patches through the planner: the
    oracle's row count on random sizes and the pages' sub-factor cases, the
    per-call bounds honoured, and a rejected size raising."""
    import oracle
    import vision_image_preprocessing_amd as V

    assert V.get_number_of_image_patches(16, 192) == 48     # 32x384 -> 2 x 24 patches
    assert V.get_number_of_image_patches(8, 500) == 248     # 32x1984 -> 2 x 124 (a tie, to even)
    rng = np.random.default_rng(12)
    for _ in range(300):
        h, w = (int(np.exp(rng.uniform(0.0, np.log(5000.0)))) for _ in range(2))
        st, _, _ = oracle.smart_resize_status(h, w)
        if st != 0:
            continue
        assert V.get_number_of_image_patches(h, w) == oracle.image_grid(h, w)[1], (h, w)
    assert V.get_number_of_image_patches(1000, 1000, max_pixels=65536) == \
        oracle.image_grid(1000, 1000, max_pixels=65536)[1]
    with pytest.raises(V.MimoError):
        V.get_number_of_image_patches(32, 6401)               # beyond the 200:1 aspect guard


def test_image_processor_arguments_without_gpu():
    """The processor's constructor arguments; patch sizes other than the
    kernels' and non-image inputs are refused before any GPU work."""
    import vision_image_preprocessing_amd as V

    p = V.ImageProcessor(16, 2, 2, 8192, 8388608, (0.5, 0.5, 0.5), (0.5, 0.5, 0.5))
    assert p.image_mean == (0.5, 0.5, 0.5) and p.min_pixels == 8192
    with pytest.raises(V.MimoError):
        V.ImageProcessor(patch_size=14)
    with pytest.raises(V.MimoError):
        p([np.zeros((10, 10), np.uint8)])
    with pytest.raises(V.MimoError):
        p([np.zeros((10, 10, 3), np.float32)])


def test_video_processor_arguments_without_gpu():
    """Items that are not uint8 clips or images are refused before any GPU
    work; a clip beyond the geometry raises the planner's error."""
    import vision_image_preprocessing_amd as V

    p = V.VideoProcessor()
    with pytest.raises(V.MimoError):
        p([np.zeros((2, 10, 10), np.uint8)])           # no channel axis
    with pytest.raises(V.MimoError):
        p([np.zeros((2, 10, 10, 3), np.float32)])      # not uint8
    with pytest.raises(V.MimoError):
        p([np.zeros((0, 10, 10, 3), np.uint8)])        # no frames
    with pytest.raises(V.MimoError):
        p([np.zeros((2, 32, 6401, 3), np.uint8)])      # beyond the 200:1 aspect guard


def test_plan_reports_per_image_status():
    shapes = [(64, 64, 3), (32, 6401, 3), (0, 5, 3), (40, 40, 5), (1, 8193, 4), (50, 60, 4)]
    desc, total_rows, total_src, code = V.plan_geometry(shapes, check=False)
    assert code == V.MIMO_E_ASPECT  # first failure
    assert list(desc["status"]) == [0, V.MIMO_E_ASPECT, V.MIMO_E_INVALID, V.MIMO_E_INVALID,
                                    V.MIMO_E_DEGENERATE, 0]
    assert list(desc["rows"][[1, 2, 3, 4]]) == [0, 0, 0, 0]
    assert total_rows == desc["rows"].sum()
    with pytest.raises(V.MimoError):
        V.plan_geometry(shapes)
    assert "item 1" in V.last_error()


def test_column_permutation_matches_oracle():
    rng = np.random.default_rng(23)
    for _ in range(300):
        gt = int(rng.integers(1, 3))
        gh = 2 * int(rng.integers(1, 60))
        gw = 2 * int(rng.integers(1, 60))
        assert np.array_equal(V.column_permutation(gt, gh, gw), oracle.column_permutation(gt, gh, gw))
    with pytest.raises(V.MimoError):
        V.column_permutation(1, 3, 4)


def test_preprocess_argument_validation_without_gpu():
    lib = V.load()
    desc, _, _, _ = V.plan_geometry([(64, 64, 3)])
    m = (ctypes.c_float * 3)(0, 0, 0)
    s = (ctypes.c_float * 3)(1, 1, 1)
    dummy = ctypes.c_void_p(0x1000)
    # no outputs
    assert lib.mimo_preprocess_batch(1, desc.ctypes.data, dummy, 4096, m, s, 0, None, None,
                                     16, dummy, 4096, None) == V.MIMO_E_INVALID
    # bad dtype
    assert lib.mimo_preprocess_batch(1, desc.ctypes.data, dummy, 4096, m, s, 7, dummy, None,
                                     16, dummy, 4096, None) == V.MIMO_E_INVALID
    # empty batch is a no-op
    assert lib.mimo_preprocess_batch(0, None, None, 0, m, s, 0, dummy, None, 0, None, 0,
                                     None) == V.MIMO_OK
    # workspace too small
    assert lib.mimo_preprocess_batch(1, desc.ctypes.data, dummy, 1 << 20, m, s, 0, dummy, None,
                                     16, dummy, 8, None) == V.MIMO_E_CAPACITY
    # in-place permute is rejected
    assert lib.mimo_column_permute(1, desc.ctypes.data, dummy, dummy, 0, 16, dummy, 4096,
                                   None) == V.MIMO_E_INVALID
    assert V.status_string(V.MIMO_E_DEGENERATE).startswith("degenerate")


def test_video_helpers_match_oracle():
    rng = np.random.default_rng(29)
    for _ in range(3000):
        total = int(rng.integers(1, 20000))
        fps_src = float(rng.uniform(5, 120))
        fps = float(rng.uniform(0.1, 8))
        n = V.smart_nframes(total, fps_src, fps, 4, 768)
        assert n == oracle.smart_nframes(total, fps_src, fps, 4, 768), (total, fps_src, fps)
        k = max(n, 1)
        idx, ts = V.sample_frames(total, k, fps_src)
        ridx, rts = oracle.sample_frames(total, k, fps_src)
        assert np.array_equal(idx, ridx) and np.array_equal(ts, rts), (total, k, fps_src)
        total_max = int(rng.integers(1, 1 << 26))
        assert V.video_max_pixels(k, total_max) == oracle.video_max_pixels(k, total_max)


def test_plan_frames_matches_oracle():
    """Per-item ceilings, grid_t = ceil(frames / 2), rows and offsets for a
    mix of stills and videos; one-frame items plan exactly like images."""
    rng = np.random.default_rng(31)
    items, ceilings = [], []
    for i in range(200):
        f = int(rng.integers(1, 40)) if i % 3 else 1
        h = int(rng.integers(8, 2200))
        w = int(rng.integers(8, 2200))
        c = 3 if rng.random() < 0.7 else 4
        items.append((f, h, w, c))
        ceilings.append(oracle.video_max_pixels(f, 1 << 24) if f > 1 else 0)
    desc, total_rows, total_src, code = V.plan_frames(items, ceilings, check=False)
    rows = src = 0
    for i, (f, h, w, c) in enumerate(items):
        mx = ceilings[i] if ceilings[i] > 0 else oracle.MAX_PIXELS
        st, oh, ow = oracle.smart_resize_status(h, w, 32, oracle.MIN_PIXELS, mx)
        d = desc[i]
        assert d["status"] == st, (i, items[i])
        if st:
            assert d["rows"] == 0
            continue
        gt = (f + 1) // 2
        assert (d["dst_h"], d["dst_w"], d["frames"]) == (oh, ow, f)
        assert (d["grid_t"], d["grid_h"], d["grid_w"]) == (gt, oh // 16, ow // 16)
        assert d["rows"] == gt * (oh // 16) * (ow // 16)
        assert d["row_offset"] == rows and d["src_offset"] == src
        rows += int(d["rows"])
        src += f * h * w * c
    assert (total_rows, total_src) == (rows, src)
    stills = [it for it in items if it[0] == 1]
    gdesc, _, _, _ = V.plan_geometry([it[1:] for it in stills], check=False)
    fdesc, _, _, _ = V.plan_frames(stills, check=False)
    assert np.array_equal(gdesc, fdesc)


def test_plan_frames_rejects_bad_frame_counts():
    desc, _, _, code = V.plan_frames([(0, 64, 64, 3), (2, 64, 64, 3), (-3, 64, 64, 3)], check=False)
    assert list(desc["status"]) == [V.MIMO_E_INVALID, 0, V.MIMO_E_INVALID]
    assert code == V.MIMO_E_INVALID


@pytest.mark.parametrize("dim", [8, 16, 32, 40, 64, 128, 256])
def test_rope_inv_freq_matches_oracle(dim):
    for theta in (10000.0, 500.0, 1e6):
        assert np.array_equal(V.rope_inv_freq(dim, theta), oracle.rope_inv_freq(dim, theta)), (dim, theta)
    with pytest.raises(V.MimoError):
        V.rope_inv_freq(7)


def test_chunk_seqlens_match_oracle():
    items = [(1, 200, 300, 3), (5, 64, 96, 3), (1, 1, 8193, 3), (4, 1080, 1920, 3), (3, 37, 29, 4)]
    desc, _, _, _ = V.plan_frames(items, check=False)
    ok = desc["status"] == 0
    thw = np.stack([desc["grid_t"], desc["grid_h"], desc["grid_w"]], axis=1)[ok]
    assert np.array_equal(V.chunk_seqlens(desc), oracle.chunk_seqlens(thw))
    lib = V.load()
    cu = np.empty(2, dtype=np.int32)
    assert lib.mimo_chunk_seqlens(len(desc), desc.ctypes.data, cu.ctypes.data, 2) == V.MIMO_E_CAPACITY


def test_vit_tables_argument_validation_without_gpu():
    lib = V.load()
    desc, _, _, _ = V.plan_geometry([(64, 64, 3)])
    dummy = ctypes.c_void_p(0x1000)
    # bad order, bad rope_dim, no outputs, misaligned table: all rejected before any GPU work
    assert lib.mimo_rotary_tables(1, desc.ctypes.data, 2, 32, 1e4, dummy, None, None, 16, dummy,
                                  4096, None) == V.MIMO_E_INVALID
    assert lib.mimo_rotary_tables(1, desc.ctypes.data, 0, 12, 1e4, dummy, None, None, 16, dummy,
                                  4096, None) == V.MIMO_E_INVALID
    assert lib.mimo_rotary_tables(1, desc.ctypes.data, 0, 32, 1e4, None, None, None, 16, dummy,
                                  4096, None) == V.MIMO_E_INVALID
    assert lib.mimo_rotary_tables(1, desc.ctypes.data, 0, 32, 1e4, None, ctypes.c_void_p(0x1004),
                                  None, 16, dummy, 4096, None) == V.MIMO_E_INVALID
    # capacity below the plan's rows (16 rows for 64x64 -> 128x128... use a tiny capacity)
    assert lib.mimo_rotary_tables(1, desc.ctypes.data, 0, 32, 1e4, dummy, None, None, 1, dummy,
                                  4096, None) == V.MIMO_E_CAPACITY
    assert lib.mimo_window_index(1, desc.ctypes.data, 1, None, None, 16, dummy, 4096,
                                 None) == V.MIMO_E_INVALID
    assert lib.mimo_window_index(1, desc.ctypes.data, 1, dummy, None, 1, dummy, 4096,
                                 None) == V.MIMO_E_CAPACITY
    assert lib.mimo_window_index(1, desc.ctypes.data, 1, dummy, None, 1 << 20, dummy, 8,
                                 None) == V.MIMO_E_CAPACITY
    # an empty batch is a no-op
    assert lib.mimo_rotary_tables(0, None, 0, 32, 1e4, dummy, None, None, 0, None, 0,
                                  None) == V.MIMO_OK


def test_hf_plan_matches_oracle():
    rng = np.random.default_rng(57)
    shapes = [(16, 192, 3), (8, 500, 3), (31, 31, 4), (1, 64, 3), (1, 1, 3), (4000, 6000, 3),
              (1, 8193, 3), (200, 300, 4)]
    shapes += [(int(rng.integers(1, 3000)), int(rng.integers(1, 3000)), 3) for _ in range(500)]
    desc, total_rows, total_src, _ = V.plan_hf(shapes, check=False)
    rows = src = 0
    for i, (h, w, c) in enumerate(shapes):
        st, oh, ow = oracle.hf_smart_resize_status(h, w)
        d = desc[i]
        assert d["status"] == st, (h, w)
        if st == 0:
            assert (d["dst_h"], d["dst_w"]) == (oh, ow), (h, w)
            assert (d["grid_t"], d["grid_h"], d["grid_w"], d["rows"]) == (1, oh // 16, ow // 16, oh * ow // 256)
            assert d["row_offset"] == rows
            rows += int(d["rows"])
        assert d["src_offset"] == src
        src += h * w * c
    assert (total_rows, total_src) == (rows, src)
    assert V.hf_smart_resize(16, 192) == oracle.hf_smart_resize(16, 192) == (32, 320)


def test_hf_argument_validation_without_gpu():
    lib = V.load()
    desc, _, _, _ = V.plan_hf([(64, 64, 3)])
    m = (ctypes.c_float * 3)(0.5, 0.5, 0.5)
    s = (ctypes.c_float * 3)(0.2, 0.2, 0.2)
    bad_s = (ctypes.c_float * 3)(0.2, 0.0, 0.2)
    dummy = ctypes.c_void_p(0x1000)
    ws = V.hf_workspace_bytes(desc)
    assert lib.mimo_preprocess_hf_batch(1, desc.ctypes.data, dummy, 4096, m, s, 0, None, None,
                                        1 << 20, dummy, ws, None) == V.MIMO_E_INVALID
    assert lib.mimo_preprocess_hf_batch(1, desc.ctypes.data, dummy, 4096, m, bad_s, 0, dummy, None,
                                        1 << 20, dummy, ws, None) == V.MIMO_E_INVALID
    assert lib.mimo_preprocess_hf_batch(1, desc.ctypes.data, dummy, 1 << 20, m, s, 0, dummy, None,
                                        1 << 20, dummy, 16, None) == V.MIMO_E_CAPACITY
    assert lib.mimo_preprocess_hf_batch(1, desc.ctypes.data, dummy, 16, m, s, 0, dummy, None,
                                        1 << 20, dummy, ws, None) == V.MIMO_E_CAPACITY


def test_hf_extreme_vertical_downscale_is_refused_before_launch():
    lib = V.load()
    p = V.make_params(4096, 8192)
    desc, _, _, _ = V.plan_hf([(20000, 20000, 3)], p)
    assert desc["dst_h"][0] == 64  # a ~312x downscale: about 1250 taps per output row
    m = (ctypes.c_float * 3)(0.5, 0.5, 0.5)
    s = (ctypes.c_float * 3)(0.2, 0.2, 0.2)
    dummy = ctypes.c_void_p(0x1000)
    st = lib.mimo_preprocess_hf_batch(1, desc.ctypes.data, dummy, 20000 * 20000 * 3, m, s, 0, dummy,
                                      None, 1 << 20, dummy, V.hf_workspace_bytes(desc), None)
    assert st == V.MIMO_E_UNSUPPORTED
    assert "downscale" in V.last_error()


def test_stats255_matches_oracle():
    for mean, std in (((0.485, 0.456, 0.406), (0.229, 0.224, 0.225)),
                      (W.CLIP_MEAN, W.CLIP_STD), ((0.0, 0.5, 1.0), (1e-3, 1.0, 3.5))):
        m, s = V._abi.stats255(mean, std)
        om, os_ = oracle.stats255(mean, std)
        assert np.array_equal(np.asarray(m, np.float32), om)
        assert np.array_equal(np.asarray(s, np.float32), os_)
    for bad in (((0.5, 0.5, 0.5), (0.2, 0.0, 0.2)), ((0.5, float("nan"), 0.5), (0.2, 0.2, 0.2)),
                ((0.5, 0.5, 0.5), (0.2, -1.0, 0.2)), ((0.5, 0.5, 0.5), (0.2, 0.2, float("inf")))):
        with pytest.raises(V.MimoError) as e:
            V._abi.stats255(*bad)
        assert e.value.code == V.MIMO_E_INVALID


def test_binding_refuses_misshaped_tensors_before_any_launch():
    """Every entry point that takes device tensors checks their shape, dtype
    and contiguity (then their device) in the binding: a flat or narrow
    output would otherwise make the library believe it holds far more rows
    than it does.  Host tensors stand in here: the shape checks come first,
    and a well-shaped host tensor fails the device check."""
    torch = pytest.importorskip("torch")
    desc, _, _, _ = V.plan_geometry([(64, 64, 3)])
    f32, bf16 = torch.float32, torch.bfloat16
    rows = torch.zeros((4, 1536), dtype=f32)
    ws = torch.zeros(V.workspace_bytes(1), dtype=torch.uint8)
    src = torch.zeros(64 * 64 * 3, dtype=torch.uint8)
    m, s = (1.0, 1.0, 1.0), (1.0, 1.0, 1.0)

    def refused(fn, *a, **k):
        with pytest.raises(V.MimoError) as e:
            fn(*a, **k)
        assert e.value.code == V.MIMO_E_INVALID
        return str(e.value)

    # preprocess_batch
    refused(V.preprocess_batch, desc, src, m, s, rows=torch.zeros(4 * 1536, dtype=f32), workspace=ws)
    refused(V.preprocess_batch, desc, src, m, s, rows=torch.zeros((4, 768), dtype=f32), workspace=ws)
    refused(V.preprocess_batch, desc, src, m, s, rows=torch.zeros((1536, 4), dtype=f32).t(), workspace=ws)
    refused(V.preprocess_batch, desc, src, m, s, rows=torch.zeros((4, 1536), dtype=torch.float16),
            workspace=ws)
    refused(V.preprocess_batch, desc, src, m, s, rows=rows, rows_col=torch.zeros((4, 1536), dtype=bf16),
            workspace=ws)
    refused(V.preprocess_batch, desc, src.float(), m, s, rows=rows, workspace=ws)
    refused(V.preprocess_batch, desc, src, m, s, rows=rows, workspace=None)
    assert "GPU" in refused(V.preprocess_batch, desc, src, m, s, rows=rows, workspace=ws)
    # column_permute
    refused(V.column_permute, desc, rows, torch.zeros(4 * 1536, dtype=f32), ws)
    refused(V.column_permute, desc, rows, torch.zeros((4, 1536), dtype=bf16), ws)
    refused(V.column_permute, desc, rows.view(8, 768), rows.clone().view(8, 768), ws)
    assert "GPU" in refused(V.column_permute, desc, rows, rows.clone(), ws)
    # patch_embed
    w = torch.zeros((256, 1536), dtype=bf16)
    refused(V.patch_embed, rows, w)                                      # float32 rows
    refused(V.patch_embed, rows.to(bf16), torch.zeros((256, 1000), dtype=bf16))
    refused(V.patch_embed, rows.to(bf16), w.float())
    refused(V.patch_embed, rows.to(bf16), w, bias=torch.zeros(255))
    refused(V.patch_embed, rows.to(bf16), w, out=torch.zeros((4, 128), dtype=f32))
    refused(V.patch_embed, rows.to(bf16), w, out=torch.zeros((3, 256), dtype=f32))
    assert "GPU" in refused(V.patch_embed, rows.to(bf16), w, out=torch.zeros((4, 256), dtype=f32))
    # fold_patch_weights
    refused(V.fold_patch_weights, torch.zeros((256, 768), dtype=bf16))
    refused(V.fold_patch_weights, w, torch.zeros((128, 768), dtype=bf16))
    # preprocess_hf_batch
    hdesc, _, _, _ = V.plan_hf([(64, 64, 3)])
    refused(V.preprocess_hf_batch, hdesc, src, m, s, rows=torch.zeros(4 * 1536, dtype=f32), workspace=ws)
    refused(V.preprocess_hf_batch, hdesc, src, m, s, rows=None, workspace=ws)
    assert "GPU" in refused(V.preprocess_hf_batch, hdesc, src, m, s, rows=rows, workspace=ws)
    # rotary tables and window index
    refused(V.rotary_tables, desc, ws, pos=torch.zeros((4, 2), dtype=torch.int64))
    refused(V.rotary_tables, desc, ws, cos=torch.zeros((4, 16), dtype=f32), rope_dim=32)
    refused(V.window_index, desc, ws, index=torch.zeros((1, 1), dtype=torch.int64))
    refused(V.window_index, desc, ws, index=torch.zeros(1, dtype=torch.int32))


def test_noalloc_refuses_too_many_images_before_any_device_work():
    """mimo_preprocess_batch_noalloc checks the image count against its
    static scratch first: the pointers are never touched (these are not
    device addresses) and nothing is enqueued."""
    lib = V.load()
    n = V._abi.NOALLOC_MAX_IMAGES + 1
    m = (ctypes.c_float * 3)(0.0, 0.0, 0.0)
    s = (ctypes.c_float * 3)(1.0, 1.0, 1.0)
    before = V.dispatch_count()
    code = lib.mimo_preprocess_batch_noalloc(n, 0x1000, 0x2000, 1 << 20, m, s, V.MIMO_F32, 0x3000,
                                             None, 1 << 20, None)
    assert code == V.MIMO_E_CAPACITY and V.dispatch_count() == before
    assert "8192" in V.last_error()
