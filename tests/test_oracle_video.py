"""Pins for the oracle's video-frame functions (CPU only).

* sample_frames: numpy's unique(int64(linspace(...))) and float32 division,
  the expression the cortiq page prints;
* smart_nframes, video_max_pixels: hand-derived cases from the printed
  formulas, and properties (even, bounded);
* the frames pixel path: one frame reduces to the image path; several
  frames match an independent torch composition (F.interpolate on the frame
  stack, standardise, and a reshape/permute patchify with real temporal
  pairs); odd counts repeat the last frame.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

P, M, T = 16, 2, 2


def test_sample_frames_matches_numpy_linspace():
    rng = np.random.default_rng(3)
    cases = [(100, 8, 30.0), (10, 10, 24.0), (5, 9, 25.0), (1, 1, 30.0), (7, 1, 29.97)]
    cases += [(int(rng.integers(1, 5000)), int(rng.integers(1, 300)), float(rng.uniform(1, 120)))
              for _ in range(300)]
    for total, n, fps in cases:
        idx, ts = oracle.sample_frames(total, n, fps)
        ref_idx = np.unique(np.linspace(0, total - 1, n).astype(np.int64))
        ref_ts = ref_idx.astype(np.float32) / np.float32(fps)
        assert np.array_equal(idx, ref_idx), (total, n, fps)
        assert np.array_equal(ts, ref_ts), (total, n, fps)


def test_smart_nframes_cases():
    # 300 frames at 30 fps sampled at 2 fps: 20 frames (even, inside [4, 768])
    assert oracle.smart_nframes(300, 30.0, 2.0, 4, 768) == 20
    # 45 frames at 30 fps at 2 fps: 3.0 -> clamped up to min 4
    assert oracle.smart_nframes(45, 30.0, 2.0, 4, 768) == 4
    # 3 frames: min 4 exceeds total -> at most 3 -> floored to even 2
    assert oracle.smart_nframes(3, 30.0, 2.0, 4, 768) == 2
    # 100000 frames: capped at max 768
    assert oracle.smart_nframes(100000, 30.0, 2.0, 4, 768) == 768
    # 301 frames at 30 fps at 2 fps: 20.07 -> floored to even 20
    assert oracle.smart_nframes(301, 30.0, 2.0, 4, 768) == 20
    # 315 at 30 fps at 2 fps: 21.0 -> floored to even 20
    assert oracle.smart_nframes(315, 30.0, 2.0, 4, 768) == 20
    rng = np.random.default_rng(4)
    for _ in range(2000):
        total = int(rng.integers(1, 20000))
        fps_src = float(rng.uniform(5, 120))
        fps = float(rng.uniform(0.1, 8))
        n = oracle.smart_nframes(total, fps_src, fps, 4, 768)
        assert n % 2 == 0 and 0 <= n <= min(total, 768)
        if total >= 4:
            assert n >= 4


def test_video_max_pixels_cases():
    # max(min, min(total*T//n, max)): 16777216*2//32 = 1048576
    assert oracle.video_max_pixels(32, 16777216) == 1048576
    # per-frame share above max_pixels is capped
    assert oracle.video_max_pixels(1, 16777216) == 8388608
    # below min_pixels is raised to min
    assert oracle.video_max_pixels(4096, 1000) == 8192
    # floor division: 1000*2//3 = 666 < min -> 8192; 10**7*2//3 = 6666666
    assert oracle.video_max_pixels(3, 10 ** 7) == 6666666


def _torch_video(frames_u8, oh, ow, mean255, std255):
    n = frames_u8.shape[0]
    pad = (-n) % T
    if pad:
        frames_u8 = np.concatenate([frames_u8, np.repeat(frames_u8[-1:], pad, axis=0)])
    x = torch.from_numpy(np.ascontiguousarray(frames_u8)).permute(0, 3, 1, 2).float()
    x = F.interpolate(x, size=(oh, ow), mode="bilinear", align_corners=False, antialias=False)
    mean = torch.from_numpy(np.asarray(mean255, dtype=np.float32))[None, :, None, None]
    std = torch.from_numpy(np.asarray(std255, dtype=np.float32))[None, :, None, None]
    x = (x - mean) / std  # [n_pad, C, H, W]
    gt, gh, gw = x.shape[0] // T, oh // P, ow // P
    p = x.reshape(gt, T, 3, gh // M, M, P, gw // M, M, P)
    p = p.permute(0, 3, 6, 4, 7, 2, 1, 5, 8)  # (t, br, bc, mh, mw, c, tt, py, px)
    return p.reshape(gt * gh * gw, 3 * T * P * P).numpy()


@pytest.mark.parametrize("n,h,w", [(1, 40, 70), (2, 64, 96), (5, 37, 29), (6, 120, 200), (4, 16, 192)])
def test_video_matches_torch_composition(n, h, w):
    rng = np.random.default_rng(n * 100 + h)
    frames = rng.integers(0, 256, (n, h, w, 3), dtype=np.uint8)
    oh, ow = oracle.smart_resize(h, w)
    m, s = oracle.stats255((0.485, 0.456, 0.406), (0.229, 0.224, 0.225))
    got = oracle.preprocess_video(frames, oh, ow, m, s)
    ref = _torch_video(frames, oh, ow, m, s)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


def test_single_frame_is_the_image_path():
    rng = np.random.default_rng(8)
    for hwc in ((200, 300, 3), (45, 77, 4)):
        img = rng.integers(0, 256, hwc, dtype=np.uint8)
        oh, ow = oracle.smart_resize(hwc[0], hwc[1])
        m, s = oracle.stats255((0.485, 0.456, 0.406), (0.229, 0.224, 0.225))
        assert np.array_equal(oracle.preprocess_video(img[None], oh, ow, m, s),
                              oracle.preprocess_image(img, oh, ow, m, s))


def test_frames_pair_into_temporal_slots():
    """Slot tt of temporal patch t holds frame 2t+tt; an odd count repeats the
    last frame in the last pair."""
    rng = np.random.default_rng(9)
    n, h, w = 5, 64, 64
    frames = rng.integers(0, 256, (n, h, w, 4), dtype=np.uint8)
    m, s = oracle.stats255((0.485, 0.456, 0.406), (0.229, 0.224, 0.225))
    rows = oracle.preprocess_video(frames, h, w, m, s).reshape(3, 16, 3, T, P * P)
    for t in range(3):
        for tt in range(T):
            f = min(2 * t + tt, n - 1)
            single = oracle.preprocess_image(frames[f], h, w, m, s).reshape(16, 3, T, P * P)
            assert np.array_equal(rows[t, :, :, tt], single[:, :, 0])
