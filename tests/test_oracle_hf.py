"""Pins for the oracle's stock-HF contrast path (CPU only).

The processing page describes the stock Qwen2-VL processor's pixels (PIL
bicubic with antialias and a uint8 round trip, 0-1 normalisation, alpha
dropped, per-side clamping in smart_resize).  Both libraries it names are
installed, so the oracle is pinned to them directly:

* the resize bitwise against PIL's Image.resize(BICUBIC) on upscales,
  downscales, mixed, one-axis and identity cases;
* smart_resize against transformers' Qwen2-VL smart_resize (PIL backend)
  on random sizes, sub-factor ones included;
* the whole pixel path bitwise against transformers'
  Qwen2VLImageProcessorPil configured with patch 16, merge 2, temporal 2,
  the MiMo pixel bounds and ImageNet statistics, RGB and RGBA inputs;
* the page's example that 16x192 gets a different grid from the MiMo path.
"""
import numpy as np
import pytest
from PIL import Image

import oracle

IMAGENET_MEAN = (0.485, 0.456, 0.406)
IMAGENET_STD = (0.229, 0.224, 0.225)


def _hf_module():
    return pytest.importorskip("transformers.models.qwen2_vl.image_processing_pil_qwen2_vl")


def test_pil_bicubic_bitwise():
    rng = np.random.default_rng(51)
    cases = [(7, 9, 13, 5), (100, 150, 64, 96), (64, 96, 100, 150), (31, 31, 96, 96),
             (1, 64, 32, 320), (17, 300, 17, 128), (300, 17, 128, 17), (40, 40, 40, 40),
             (1, 1, 96, 96), (2000, 3000, 1168, 1760)]
    cases += [tuple(int(v) for v in rng.integers(1, 300, 4)) for _ in range(120)]
    for h, w, oh, ow in cases:
        for c, mode in ((3, "RGB"), (1, "L")):
            img = rng.integers(0, 256, (h, w, c), dtype=np.uint8)
            pil = Image.fromarray(img[..., 0] if c == 1 else img, mode)
            ref = np.asarray(pil.resize((ow, oh), Image.BICUBIC)).reshape(oh, ow, c)
            assert np.array_equal(oracle.pil_resize_bicubic(img, oh, ow), ref), (h, w, oh, ow, mode)


def test_hf_smart_resize_matches_transformers():
    hf = _hf_module().smart_resize
    rng = np.random.default_rng(52)
    sizes = [(16, 192), (8, 500), (31, 31), (1, 64), (1, 1), (4000, 6000), (1, 8193), (1, 8192)]
    sizes += [(int(rng.integers(1, 40)), int(rng.integers(1, 3000))) for _ in range(3000)]
    sizes += [(int(rng.integers(1, 9000)), int(rng.integers(1, 9000))) for _ in range(3000)]
    for h, w in sizes:
        try:
            want = hf(h, w, factor=32, min_pixels=8192, max_pixels=8388608)
        except ValueError:
            want = None
        st, oh, ow = oracle.hf_smart_resize_status(h, w)
        if want is None:
            assert st == oracle.E_ASPECT, (h, w)
        else:
            assert st == 0 and (oh, ow) == tuple(want), (h, w, want, (oh, ow))


def test_hf_smart_resize_random_bounds_match_transformers():
    """Smaller pixel ceilings reach the per-side clamp of the shrink branch
    (a side that floors to zero becomes one factor)."""
    hf = _hf_module().smart_resize
    rng = np.random.default_rng(55)
    clamped = 0
    for _ in range(4000):
        h, w = int(rng.integers(1, 400)), int(rng.integers(1, 20000))
        if rng.random() < 0.5:
            h, w = w, h
        mn = int(rng.integers(0, 5000))
        mx = int(rng.integers(max(mn, 1024), 200000))
        try:
            want = hf(h, w, factor=32, min_pixels=mn, max_pixels=mx)
        except ValueError:
            want = None
        st, oh, ow = oracle.hf_smart_resize_status(h, w, 32, mn, mx)
        if want is None:
            assert st == oracle.E_ASPECT, (h, w)
            continue
        assert st == 0 and (oh, ow) == tuple(want), (h, w, mn, mx, want, (oh, ow))
        beta = np.sqrt(h * w / mx)
        clamped += int(round(h / 32) * round(w / 32) * 1024 > mx and min(np.floor(h / beta / 32), np.floor(w / beta / 32)) == 0)
    assert clamped > 20  # the clamp was exercised


def test_page_example_grids_differ():
    # the page: tiny inputs such as 16x192 get a different grid under the stock rules
    assert oracle.hf_smart_resize(16, 192) != oracle.smart_resize(16, 192)
    # and images with both sides >= the factor get the same one
    rng = np.random.default_rng(53)
    for _ in range(500):
        h, w = int(rng.integers(32, 5000)), int(rng.integers(32, 5000))
        if max(h, w) / min(h, w) <= 200:
            assert oracle.hf_smart_resize(h, w) == oracle.smart_resize(h, w), (h, w)


def _hf_processor():
    mod = _hf_module()
    return mod.Qwen2VLImageProcessorPil(patch_size=16, merge_size=2, temporal_patch_size=2,
                                        min_pixels=8192, max_pixels=8388608,
                                        image_mean=list(IMAGENET_MEAN), image_std=list(IMAGENET_STD))


@pytest.mark.parametrize("h,w,c", [(200, 300, 3), (45, 77, 4), (513, 257, 3), (64, 64, 3), (16, 192, 3),
                                   (1000, 33, 4), (96, 128, 3), (700, 1000, 4)])
def test_pixel_path_matches_transformers(h, w, c):
    rng = np.random.default_rng(h * 7 + w)
    img = rng.integers(0, 256, (h, w, c), dtype=np.uint8)
    proc = _hf_processor()
    pil = Image.fromarray(img, "RGBA" if c == 4 else "RGB")
    out = proc(images=[pil], return_tensors="np")
    oh, ow = oracle.hf_smart_resize(h, w)
    assert list(out["image_grid_thw"][0]) == [1, oh // 16, ow // 16]
    got = oracle.hf_preprocess_image(img, oh, ow, IMAGENET_MEAN, IMAGENET_STD)
    assert np.array_equal(got, out["pixel_values"]), (h, w, c)


def test_contrast_with_the_mimo_path():
    """The page's distribution shift: on a non-identity resize the stock
    pixels differ from the MiMo ones by a fraction of a standard deviation."""
    rng = np.random.default_rng(54)
    img = rng.integers(0, 256, (600, 900, 3), dtype=np.uint8)
    oh, ow = oracle.smart_resize(600, 900)
    assert (oh, ow) == oracle.hf_smart_resize(600, 900)
    m, s = oracle.stats255(IMAGENET_MEAN, IMAGENET_STD)
    mimo = oracle.preprocess_image(img, oh, ow, m, s)
    hf = oracle.hf_preprocess_image(img, oh, ow, IMAGENET_MEAN, IMAGENET_STD)
    diff = np.abs(mimo - hf)
    assert 0.0 < diff.mean() < 0.5 and diff.max() < 3.0
