"""Pins for the oracle's pixel arithmetic (CPU only).

* flatten: PIL compositing onto white, on all 65,536 (value, alpha) pairs;
* resize: torch CPU F.interpolate(bilinear, align_corners=False, no
  antialias) -- the routine the pages name -- and a float64 evaluation of
  the half-pixel bilinear definition within a derived rounding bound;
* standardise: closed forms (mean 0 / std 1 is the identity; a constant
  image maps to (v - mean) / std);
* bf16: torch's float32 -> bfloat16 conversion (round to nearest even).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

Image = pytest.importorskip("PIL.Image")


# ----------------------------------------------------------------- flatten
def _all_pairs():
    c = np.repeat(np.arange(256, dtype=np.uint8), 256)
    a = np.tile(np.arange(256, dtype=np.uint8), 256)
    rgba = np.stack([c, c, c, a], axis=-1).reshape(256, 256, 4)
    return rgba


def test_flatten_matches_pil_alpha_composite_all_pairs():
    rgba = _all_pairs()
    im = Image.fromarray(rgba, "RGBA")
    white = Image.new("RGBA", im.size, (255, 255, 255, 255))
    ref = np.asarray(Image.alpha_composite(white, im).convert("RGB"))
    got = oracle.flatten_rgba(rgba)
    assert np.array_equal(got, ref)


def test_flatten_matches_pil_paste_with_mask_all_pairs():
    rgba = _all_pairs()
    im = Image.fromarray(rgba, "RGBA")
    bg = Image.new("RGB", im.size, (255, 255, 255))
    bg.paste(im, mask=im.split()[3])
    got = oracle.flatten_rgba(rgba)
    assert np.array_equal(got, np.asarray(bg))


def test_flatten_special_alphas():
    rng = np.random.default_rng(0)
    rgba = rng.integers(0, 256, (50, 40, 4), dtype=np.uint8)
    rgba[..., 3] = 0
    assert (oracle.flatten_rgba(rgba) == 255).all()
    rgba[..., 3] = 255
    assert np.array_equal(oracle.flatten_rgba(rgba), rgba[..., :3])


# ------------------------------------------------------------------ resize
RESIZE_SHAPES = [
    (200, 300, 192, 288),      # 300x200 RGB workload
    (16, 192, 32, 384),        # pages' sub-factor case
    (8, 500, 32, 1984),
    (31, 31, 96, 96),
    (1, 64, 32, 2048),
    (480, 640, 480, 640),      # identity
    (700, 1000, 704, 992),     # mild down/up per axis
    (1080, 1920, 1088, 1920),
    (777, 1333, 768, 1344),
    (37, 29, 64, 96),          # upscale, odd sizes
    (513, 257, 96, 64),        # strong downscale
]


def _torch_resize(planar, oh, ow):
    t = torch.from_numpy(planar)[None]
    return F.interpolate(t, size=(oh, ow), mode="bilinear", align_corners=False,
                         antialias=False)[0].numpy()


@pytest.mark.parametrize("h,w,oh,ow", RESIZE_SHAPES)
def test_resize_matches_torch_interpolate(h, w, oh, ow):
    rng = np.random.default_rng(h * 7919 + w)
    planar = rng.integers(0, 256, (3, h, w)).astype(np.float32)
    got = oracle.resize_bilinear(planar, oh, ow)
    ref = _torch_resize(planar, oh, ow)
    # bitwise on this host; the same recipe is torch's float32 arithmetic
    assert np.array_equal(got, ref), float(np.abs(got - ref).max())


def test_resize_matches_torch_at_large_downscale_one_plane():
    """6000x4000 -> 3520x2336, the large-image workload's target."""
    rng = np.random.default_rng(5)
    planar = rng.integers(0, 256, (1, 4000, 6000)).astype(np.float32)
    got = oracle.resize_bilinear(planar, 2336, 3520)
    ref = _torch_resize(planar, 2336, 3520)
    assert np.array_equal(got, ref)


def _exact_bilinear_f64(planar, oh, ow):
    """Half-pixel bilinear in float64 (align_corners=False definition):
    source coordinate (d + 0.5) * n_in / n_out - 0.5, clamped below at 0."""
    c, h, w = planar.shape

    def axis(n_in, n_out):
        d = np.arange(n_out, dtype=np.float64)
        s = np.maximum((d + 0.5) * n_in / n_out - 0.5, 0.0)
        i0 = np.minimum(np.floor(s).astype(np.int64), n_in - 1)
        i1 = np.minimum(i0 + 1, n_in - 1)
        l1 = s - i0
        return i0, i1, 1.0 - l1, l1

    y0, y1, ly0, ly1 = axis(h, oh)
    x0, x1, lx0, lx1 = axis(w, ow)
    p = planar.astype(np.float64)
    top = p[:, y0][:, :, x0] * lx0 + p[:, y0][:, :, x1] * lx1
    bot = p[:, y1][:, :, x0] * lx0 + p[:, y1][:, :, x1] * lx1
    return top * ly0[:, None] + bot * ly1[:, None]


@pytest.mark.parametrize("h,w,oh,ow", RESIZE_SHAPES)
def test_resize_within_float32_rounding_bound_of_exact(h, w, oh, ow):
    """The float32 recipe differs from exact arithmetic only by coordinate
    and weight rounding.  Per axis the source coordinate carries at most
    ~3 ulps of n_in (scale rounding amplified by d + 0.5, plus the fma
    rounding), so a weight moves by <= 3 * n_in * 2^-24; with values in
    [0, 255] the output moves by <= 255 * (ex + ey) plus a few ulps of 255."""
    rng = np.random.default_rng(h + 31 * w)
    planar = rng.integers(0, 256, (3, h, w)).astype(np.float32)
    got = oracle.resize_bilinear(planar, oh, ow).astype(np.float64)
    ref = _exact_bilinear_f64(planar, oh, ow)
    ex = 3.0 * w * 2.0 ** -24
    ey = 3.0 * h * 2.0 ** -24
    bound = 255.0 * (ex + ey) + 4 * 255.0 * 2.0 ** -24
    assert np.abs(got - ref).max() <= bound


def test_resize_identity_and_constant():
    rng = np.random.default_rng(3)
    planar = rng.integers(0, 256, (3, 64, 96)).astype(np.float32)
    assert np.array_equal(oracle.resize_bilinear(planar, 64, 96), planar)
    const = np.full((3, 50, 70), 137.0, dtype=np.float32)
    for oh, ow in ((32, 64), (96, 160), (50, 70), (7, 300)):
        assert (oracle.resize_bilinear(const, oh, ow) == 137.0).all()


def test_resize_power_of_two_upscale_is_exact():
    """x2 upscale: weights are 1/4 and 3/4, so every product and sum of
    8-bit values is exact in float32 and equals the rational definition."""
    rng = np.random.default_rng(9)
    planar = rng.integers(0, 256, (3, 16, 24)).astype(np.float32)
    got = oracle.resize_bilinear(planar, 32, 48)
    assert np.array_equal(got.astype(np.float64), _exact_bilinear_f64(planar, 32, 48))


# ------------------------------------------------------------- standardise
def test_standardise_closed_forms():
    # mean 0, std 1 leaves the resized values unchanged
    rng = np.random.default_rng(4)
    img = rng.integers(0, 256, (64, 64, 3), dtype=np.uint8)
    rows = oracle.preprocess_image(img, 64, 64, [0, 0, 0], [1, 1, 1])
    assert set(np.unique(rows)).issubset(set(range(256)))
    # a constant image v maps to (v - M) / S per channel, in every element
    m, s = oracle.stats255((0.485, 0.456, 0.406), (0.229, 0.224, 0.225))
    const = np.full((40, 70, 3), 200, dtype=np.uint8)
    oh, ow = oracle.smart_resize(40, 70)
    rows = oracle.preprocess_image(const, oh, ow, m, s)
    for c in range(3):
        expect = np.float32((np.float32(200.0) - m[c]) / s[c])
        assert (rows[:, c * 512:(c + 1) * 512] == expect).all()


# -------------------------------------------------------------------- bf16
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(200000) * 3).astype(np.float32)
    # exact ties: low 16 bits 0x8000, kept mantissa bits random (both
    # parities of the last kept bit), exponents from 2^-8 to 2^8
    kept = rng.integers(0, 128, 4000, dtype=np.uint32) << 16
    expo = rng.integers(119, 136, 4000, dtype=np.uint32) << 23
    ties = (expo | kept | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    got = oracle.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
