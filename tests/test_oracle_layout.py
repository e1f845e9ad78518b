"""Pins for the oracle's row layout, temporal duplication and column
permutation (CPU only).

* layout: a coded image whose pixel values name their own coordinates,
  decoded element by element against the pages' description of a row
  ((c, tt, py, px)) and of the row order ((t, block row, block col, mh, mw));
* the whole oracle pipeline against an independent torch composition:
  PIL flatten, torch float cast, F.interpolate, standardise, repeat to two
  frames, and a tensor reshape/permute patchify;
* column permutation: brute-force sort of the unit coordinates, bijection,
  unit grouping, involution on square block grids, identity on a single
  block row or column.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

Image = pytest.importorskip("PIL.Image")

P, M, T = 16, 2, 2


def test_coded_image_decodes_to_its_coordinates():
    h = w = 64
    y, x = np.mgrid[0:h, 0:w]
    img = np.stack([x, y, (x + 7 * y) % 256], axis=-1).astype(np.uint8)
    rows = oracle.preprocess_image(img, h, w, [0, 0, 0], [1, 1, 1])
    gh, gw = h // P, w // P
    bw = gw // M
    assert rows.shape == (gh * gw, 3 * T * P * P) == (16, 1536)
    for r in range(rows.shape[0]):
        # row order (block row, block col, mh, mw)
        block, k = divmod(r, M * M)
        br, bc = divmod(block, bw)
        mh, mw = divmod(k, M)
        for e in range(rows.shape[1]):
            # element order (c, tt, py, px)
            c, rest = divmod(e, T * P * P)
            tt, rest = divmod(rest, P * P)
            py, px = divmod(rest, P)
            yy = (br * M + mh) * P + py
            xx = (bc * M + mw) * P + px
            want = (xx, yy, (xx + 7 * yy) % 256)[c]
            assert rows[r, e] == want, (r, e)


def test_two_frames_are_identical():
    rng = np.random.default_rng(1)
    img = rng.integers(0, 256, (45, 77, 3), dtype=np.uint8)
    oh, ow = oracle.smart_resize(45, 77)
    m, s = oracle.stats255((0.485, 0.456, 0.406), (0.229, 0.224, 0.225))
    rows = oracle.preprocess_image(img, oh, ow, m, s)
    r = rows.reshape(-1, 3, T, P * P)
    assert np.array_equal(r[:, :, 0], r[:, :, 1])


def _torch_pipeline(img_u8, oh, ow, mean255, std255):
    """Independent formulation with library ops (PIL, torch)."""
    if img_u8.shape[-1] == 4:
        im = Image.fromarray(img_u8, "RGBA")
        white = Image.new("RGBA", im.size, (255, 255, 255, 255))
        img_u8 = np.asarray(Image.alpha_composite(white, im).convert("RGB"))
    x = torch.from_numpy(np.ascontiguousarray(img_u8)).permute(2, 0, 1).float()[None]
    x = F.interpolate(x, size=(oh, ow), mode="bilinear", align_corners=False,
                      antialias=False)[0]
    mean = torch.from_numpy(np.asarray(mean255, dtype=np.float32))[:, None, None]
    std = torch.from_numpy(np.asarray(std255, dtype=np.float32))[:, None, None]
    x = (x - mean) / std
    frames = x[None].repeat(T, 1, 1, 1)  # [T, C, H, W]
    gh, gw = oh // P, ow // P
    p = frames.reshape(1, T, 3, gh // M, M, P, gw // M, M, P)
    # -> (t, block row, block col, mh, mw, c, tt, py, px)
    p = p.permute(0, 3, 6, 4, 7, 2, 1, 5, 8)
    return p.reshape(gh * gw, 3 * T * P * P).numpy()


@pytest.mark.parametrize("hwc", [(200, 300, 3), (16, 192, 3), (8, 500, 3), (31, 31, 3),
                                 (1, 64, 3), (97, 61, 4), (480, 640, 4), (33, 1000, 3)])
def test_pipeline_matches_torch_composition(hwc):
    rng = np.random.default_rng(sum(hwc))
    img = rng.integers(0, 256, hwc, dtype=np.uint8)
    oh, ow = oracle.smart_resize(hwc[0], hwc[1])
    m, s = oracle.stats255((0.48145466, 0.4578275, 0.40821073),
                           (0.26862954, 0.26130258, 0.27577711))
    got = oracle.preprocess_image(img, oh, ow, m, s)
    ref = _torch_pipeline(img, oh, ow, m, s)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref), float(np.abs(got - ref).max())


def test_rows_route_equals_image_route():
    """The one-element-at-a-time route (for sampling big batches) gives the
    same bits as the materialised route."""
    rng = np.random.default_rng(2)
    for hwc in ((200, 300, 3), (77, 91, 4), (8, 500, 3)):
        img = rng.integers(0, 256, hwc, dtype=np.uint8)
        oh, ow = oracle.smart_resize(hwc[0], hwc[1])
        m, s = oracle.stats255((0.485, 0.456, 0.406), (0.229, 0.224, 0.225))
        full = oracle.preprocess_image(img, oh, ow, m, s)
        part = oracle.preprocess_rows(img, oh, ow, m, s, 3, full.shape[0] - 5)
        assert np.array_equal(full[3:full.shape[0] - 2], part)


# ------------------------------------------------------------- permutation
def _brute_force_perm(gt, gh, gw, m=M):
    bh, bw = gh // m, gw // m
    units = [(t, br, bc) for t in range(gt) for br in range(bh) for bc in range(bw)]
    src_index = {u: i for i, u in enumerate(units)}
    order = sorted(units, key=lambda u: (u[0], u[2], u[1]))  # (t, block col, block row)
    perm = []
    for u in order:
        perm.extend(src_index[u] * m * m + k for k in range(m * m))
    return np.asarray(perm, dtype=np.int64)


@pytest.mark.parametrize("gt,gh,gw", [(1, 2, 2), (1, 4, 6), (1, 6, 4), (2, 4, 8), (1, 12, 18),
                                      (1, 2, 24), (1, 146, 220), (3, 10, 2)])
def test_permutation_brute_force(gt, gh, gw):
    assert np.array_equal(oracle.column_permutation(gt, gh, gw), _brute_force_perm(gt, gh, gw))


def test_permutation_properties():
    rng = np.random.default_rng(6)
    for _ in range(200):
        gh = 2 * int(rng.integers(1, 40))
        gw = 2 * int(rng.integers(1, 40))
        perm = oracle.column_permutation(1, gh, gw)
        n = gh * gw
        assert np.array_equal(np.sort(perm), np.arange(n))  # bijection
        g = perm.reshape(-1, 4)
        assert (g - g[:, :1] == np.arange(4)).all()  # unit kept together, k kept
        assert (g[:, 0] % 4 == 0).all()
        if gh == gw:  # square block grid: transpose of units is an involution
            assert np.array_equal(perm[perm], np.arange(n))
        if gh == 2 or gw == 2:  # one block row or column: identity
            assert np.array_equal(perm, np.arange(n))
