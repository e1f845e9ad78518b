"""Pins for the oracle's patch embedding (CPU only).

* torch's float64 conv3d with kernel = stride = (2, 16, 16) on the rows
  viewed as [n, 3, 2, 16, 16] patches (the definition of
  MiMoVisionPatchEmbed), on rows the pixel path produced from an image;
* a one-hot weight selects single row elements exactly; scaling by 2 is
  exact; the bias adds up to float64 rounding.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle


def _image_rows(seed, h=96, w=160):
    rng = np.random.default_rng(seed)
    img = rng.integers(0, 256, (h, w, 3), dtype=np.uint8)
    m, s = oracle.stats255((0.485, 0.456, 0.406), (0.229, 0.224, 0.225))
    oh, ow = oracle.smart_resize(h, w)
    return oracle.preprocess_image(img, oh, ow, m, s)


def test_patch_embed_is_the_conv3d():
    rows = _image_rows(1)
    rng = np.random.default_rng(2)
    e = 48
    w = rng.normal(0, 0.02, (e, 3, 2, 16, 16)).astype(np.float32)
    bias = rng.normal(0, 0.1, e).astype(np.float32)
    got = oracle.patch_embed(rows, w.reshape(e, -1), bias)
    x = torch.from_numpy(rows.astype(np.float64)).view(-1, 3, 2, 16, 16)
    ref = F.conv3d(x, torch.from_numpy(w.astype(np.float64)), torch.from_numpy(bias.astype(np.float64)),
                   stride=(2, 16, 16)).view(-1, e).numpy()
    assert got.shape == ref.shape
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_patch_embed_exact_cases():
    rows = _image_rows(3)
    k = rows.shape[1]
    pick = np.array([0, 1, 255, 256, 511, 512, 1023, 1535])
    w = np.zeros((pick.size, k), np.float32)
    w[np.arange(pick.size), pick] = 1.0
    assert np.array_equal(oracle.patch_embed(rows, w), rows[:, pick].astype(np.float64))
    rng = np.random.default_rng(4)
    w = rng.normal(0, 0.02, (16, k)).astype(np.float32)
    base = oracle.patch_embed(rows, w)
    assert np.array_equal(oracle.patch_embed(2 * rows, w), 2 * base)
    bias = rng.normal(0, 1, 16).astype(np.float32)
    # the bias seeds the float64 sum, so it moves results by rounding only
    assert np.abs(oracle.patch_embed(rows, w, bias) - bias.astype(np.float64) - base).max() <= 1e-12
