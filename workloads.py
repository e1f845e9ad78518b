"""Seeded synthetic input batches for the MiMo-V2 image pixel path.

This module only draws inputs: image sizes, uint8 pixel content and the
normalisation statistics as printed.  It holds none of the method's
arithmetic (no geometry, resampling, standardisation or layout), and it is
shared by the tests, the smoke check and the benchmark so that the HIP path
and the oracle see the same bytes.

All randomness is NumPy PCG64 (``numpy.random.default_rng(seed)``).

Image sizes in the workload names are written width x height (display
notation); arrays are uint8 [height, width, channels].

Workloads:

* ``single_rgb_300x200``  -- one 300x200 RGB image, uniform pixels.
* ``rgba_64_mixed``       -- 64 RGBA images, W ~ U{640..1920}, H ~ U{480..1080};
  RGB = linear ramps + N(0, 20^2) noise, rounded and clipped; alpha 25% 0,
  25% 255, 50% U{0..255}.
* ``subfactor_256``       -- 256 RGB images with a short side below 32:
  16x192, 8x500, 31x31, 1x64 (height x width) plus 252 random sizes with
  short side U{1..31}, long side U{short..4096}, orientation a fair coin.
* ``large_16_6000x4000``  -- 16 RGB 6000x4000 images of 4-octave value noise
  (lattices 512/256/128/64 px, amplitudes 1/2^k, smoothstep-interpolated),
  scaled to [0, 255].
* ``throughput_512_1024`` -- 512 RGB 1024x1024 images, uniform pixels.
* ``video_8x64_1280x720`` -- 8 already-sampled RGB clips of 64 frames,
  1280x720: each clip pans across one 4-octave value-noise field (8 px to
  the right per frame) with N(0, 4^2) per-frame sensor noise, rounded and
  clipped; a 2^24-pixel budget per clip (per-frame ceiling from the sampled
  count), bf16 rows.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# ImageNet statistics: the MimoV2ImageProcessor defaults on the processing page.
IMAGENET_MEAN = (0.485, 0.456, 0.406)
IMAGENET_STD = (0.229, 0.224, 0.225)
# OpenAI CLIP statistics.  The processing page says MiMo-V2.5 checkpoints
# declare CLIP values but does not print them; these are the published CLIP
# preprocessing constants, supplied from outside the pages.
CLIP_MEAN = (0.48145466, 0.4578275, 0.40821073)
CLIP_STD = (0.26862954, 0.26130258, 0.27577711)


@dataclass
class Batch:
    """Items packed back to back in one flat buffer, in batch order: a still
    image is uint8 [h, w, c] (row-major), a clip is its frames [f, h, w, c]
    one after another."""

    name: str
    shapes: list  # [(h, w, c)]
    packed: np.ndarray  # uint8, flat
    offsets: np.ndarray  # int64 [n], byte offset of each item
    mean: tuple
    std: tuple
    out_dtype: str  # "f32" or "bf16"
    column_order: bool = False
    notes: dict = field(default_factory=dict)
    frames: list | None = None  # frames per item (None: all stills)
    video_budget: list | None = None  # per-item total pixel budget of a clip (0: none)

    def __len__(self):
        return len(self.shapes)

    @property
    def frame_counts(self) -> list:
        return list(self.frames) if self.frames is not None else [1] * len(self.shapes)

    @property
    def items(self) -> list:
        """(frames, h, w, c) per item."""
        return [(f, h, w, c) for f, (h, w, c) in zip(self.frame_counts, self.shapes)]

    @property
    def is_media(self) -> bool:
        return self.frames is not None

    def image(self, i: int) -> np.ndarray:
        h, w, c = self.shapes[i]
        o = int(self.offsets[i])
        return self.packed[o:o + h * w * c].reshape(h, w, c)

    def clip(self, i: int) -> np.ndarray:
        f = self.frame_counts[i]
        h, w, c = self.shapes[i]
        o = int(self.offsets[i])
        return self.packed[o:o + f * h * w * c].reshape(f, h, w, c)

    @property
    def src_bytes(self) -> int:
        return int(self.packed.size)


def _pack(shapes, frames=None):
    frames = frames if frames is not None else [1] * len(shapes)
    sizes = np.array([f * h * w * c for f, (h, w, c) in zip(frames, shapes)], dtype=np.int64)
    offsets = np.zeros(len(shapes), dtype=np.int64)
    if len(shapes) > 1:
        offsets[1:] = np.cumsum(sizes)[:-1]
    total = int(sizes.sum())
    return offsets, total


def _from_images(name, images, **kw) -> Batch:
    shapes = [tuple(int(v) for v in im.shape) for im in images]
    offsets, total = _pack(shapes)
    packed = np.empty(total, dtype=np.uint8)
    for im, o in zip(images, offsets):
        packed[o:o + im.size] = im.reshape(-1)
    return Batch(name=name, shapes=shapes, packed=packed, offsets=offsets, **kw)


def _image_rngs(seed: int, n: int):
    """One independent generator per image, so that a thread pool can draw
    images in any order and still give the same bytes."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _pool_map(fn, items):
    workers = max(1, min(16, os.cpu_count() or 1, len(items)))
    if workers == 1:
        return [fn(it) for it in items]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def _uniform_batch(name, shapes, seed, **kw) -> Batch:
    """Uniform U{0..255} pixels for every image, drawn in one go."""
    rng = np.random.default_rng(seed)
    offsets, total = _pack(shapes)
    packed = rng.integers(0, 256, size=total, dtype=np.uint8)
    return Batch(name=name, shapes=shapes, packed=packed, offsets=offsets, **kw)


def single_rgb_300x200(seed: int = 1) -> Batch:
    return _uniform_batch("single_rgb_300x200", [(200, 300, 3)], seed,
                          mean=IMAGENET_MEAN, std=IMAGENET_STD, out_dtype="f32")


def _ramp_noise_rgba(rng, h, w):
    y = np.arange(h, dtype=np.float32)[:, None]
    x = np.arange(w, dtype=np.float32)[None, :]
    r = np.broadcast_to(255.0 * x / max(w - 1, 1), (h, w))
    g = np.broadcast_to(255.0 * y / max(h - 1, 1), (h, w))
    b = 255.0 * (x + y) / max(w + h - 2, 1)
    rgb = np.stack([r, g, b], axis=-1)
    rgb = rgb + rng.normal(0.0, 20.0, size=(h, w, 3)).astype(np.float32)
    rgb = np.clip(np.rint(rgb), 0, 255).astype(np.uint8)
    # alpha: 25% fully transparent, 25% opaque, 50% uniform
    kind = rng.random((h, w))
    alpha = rng.integers(0, 256, size=(h, w), dtype=np.uint8)
    alpha[kind < 0.25] = 0
    alpha[(kind >= 0.25) & (kind < 0.5)] = 255
    return np.concatenate([rgb, alpha[..., None]], axis=-1)


def rgba_64_mixed(seed: int = 2, n: int = 64) -> Batch:
    rng = np.random.default_rng(seed)
    sizes = []
    for _ in range(n):
        w = int(rng.integers(640, 1921))
        h = int(rng.integers(480, 1081))
        sizes.append((h, w))
    rngs = _image_rngs(seed, n)
    images = _pool_map(lambda i: _ramp_noise_rgba(rngs[i], *sizes[i]), list(range(n)))
    return _from_images("rgba_64_mixed", images, mean=CLIP_MEAN, std=CLIP_STD,
                        out_dtype="f32")


def subfactor_sizes(seed: int = 3, n: int = 256):
    """(h, w) sizes: the four fixed cases, then random short/long sides."""
    fixed = [(16, 192), (8, 500), (31, 31), (1, 64)]
    rng = np.random.default_rng(seed)
    sizes = list(fixed)
    while len(sizes) < n:
        short = int(rng.integers(1, 32))
        long = int(rng.integers(short, 4097))
        if rng.random() < 0.5:
            sizes.append((short, long))
        else:
            sizes.append((long, short))
    return sizes


def subfactor_256(seed: int = 3, n: int = 256) -> Batch:
    shapes = [(h, w, 3) for (h, w) in subfactor_sizes(seed, n)]
    return _uniform_batch("subfactor_256", shapes, seed + 1000,
                          mean=IMAGENET_MEAN, std=IMAGENET_STD, out_dtype="f32")


def _smoothstep(t):
    return t * t * (3.0 - 2.0 * t)


def _value_noise(rng, h, w, lattices=(512, 256, 128, 64)):
    """Sum of octaves of lattice value noise in [0, 1] (smoothstep blend)."""
    acc = np.zeros((h, w), dtype=np.float32)
    total_amp = 0.0
    for k, cell in enumerate(lattices):
        amp = 0.5 ** k
        gh, gw = h // cell + 2, w // cell + 2
        grid = rng.random((gh, gw), dtype=np.float32)
        ys = np.arange(h, dtype=np.float32) / cell
        xs = np.arange(w, dtype=np.float32) / cell
        yi = ys.astype(np.int64)
        xi = xs.astype(np.int64)
        ty = _smoothstep(ys - yi)[:, None]
        tx = _smoothstep(xs - xi)[None, :]
        # blend lattice columns first at lattice-row resolution, then rows
        left = grid[:, xi]
        right = grid[:, xi + 1]
        horiz = left + (right - left) * tx  # [gh, w]
        top = horiz[yi]
        bot = horiz[yi + 1]
        acc += amp * (top + (bot - top) * ty)
        total_amp += amp
    return acc / total_amp


def large_16_6000x4000(seed: int = 4, n: int = 16, h: int = 4000, w: int = 6000) -> Batch:
    shapes = [(h, w, 3)] * n
    offsets, total = _pack(shapes)
    packed = np.empty(total, dtype=np.uint8)
    rngs = _image_rngs(seed, n)

    def one(i):
        img = packed[offsets[i]:offsets[i] + h * w * 3].reshape(h, w, 3)
        for c in range(3):
            v = _value_noise(rngs[i], h, w)
            lo, hi = float(v.min()), float(v.max())
            img[..., c] = np.clip(np.rint((v - lo) * (255.0 / max(hi - lo, 1e-6))), 0, 255)

    _pool_map(one, list(range(n)))
    return Batch(name="large_16_6000x4000", shapes=shapes, packed=packed, offsets=offsets,
                 mean=IMAGENET_MEAN, std=IMAGENET_STD, out_dtype="bf16")


def throughput_512_1024(seed: int = 5, n: int = 512, side: int = 1024) -> Batch:
    return _uniform_batch("throughput_512_1024", [(side, side, 3)] * n, seed,
                          mean=IMAGENET_MEAN, std=IMAGENET_STD, out_dtype="f32",
                          column_order=True)


def _panning_clip(rng, frames, h, w, step=8, sigma=4.0):
    """One clip: a window sliding `step` px right per frame over a wider
    3-channel value-noise field, plus per-frame Gaussian noise."""
    fw = w + step * (frames - 1)
    field_ = np.stack([_value_noise(rng, h, fw) for _ in range(3)], axis=-1) * 255.0
    out = np.empty((frames, h, w, 3), dtype=np.uint8)
    for f in range(frames):
        x0 = f * step
        v = field_[:, x0:x0 + w] + rng.normal(0.0, sigma, size=(h, w, 3)).astype(np.float32)
        out[f] = np.clip(np.rint(v), 0, 255)
    return out


def video_clips(name, clips, frames, h, w, seed, total_max=1 << 24,
                out_dtype="bf16") -> Batch:
    """`clips` RGB clips of `frames` already-sampled frames each, with a
    total pixel budget of `total_max` per clip (the caller's video budget; the
    per-frame ceiling derived from it belongs to the method)."""
    shapes = [(h, w, 3)] * clips
    counts = [frames] * clips
    offsets, total = _pack(shapes, counts)
    packed = np.empty(total, dtype=np.uint8)
    rngs = _image_rngs(seed, clips)
    size = frames * h * w * 3

    def one(i):
        packed[offsets[i]:offsets[i] + size] = _panning_clip(rngs[i], frames, h, w).reshape(-1)

    _pool_map(one, list(range(clips)))
    return Batch(name=name, shapes=shapes, packed=packed, offsets=offsets, mean=IMAGENET_MEAN,
                 std=IMAGENET_STD, out_dtype=out_dtype, frames=counts,
                 video_budget=[total_max] * clips)


def video_8x64_1280x720(seed: int = 6) -> Batch:
    return video_clips("video_8x64_1280x720", 8, 64, 720, 1280, seed)


def media_batch(items, seed: int, video_budget=None, name="custom_media") -> Batch:
    """Uniform pixels for (frames, h, w, c) items (tests); video_budget: the
    total pixel budget per item (0: none), one value or one per item."""
    items = [tuple(int(v) for v in it) for it in items]
    shapes = [it[1:] for it in items]
    counts = [it[0] for it in items]
    rng = np.random.default_rng(seed)
    offsets, total = _pack(shapes, counts)
    packed = rng.integers(0, 256, size=total, dtype=np.uint8)
    vb = None
    if video_budget is not None:
        vb = [int(v) for v in np.broadcast_to(video_budget, (len(items),))]
    return Batch(name=name, shapes=shapes, packed=packed, offsets=offsets, mean=IMAGENET_MEAN,
                 std=IMAGENET_STD, out_dtype="f32", frames=counts, video_budget=vb)


WORKLOADS = {
    "single_rgb_300x200": single_rgb_300x200,
    "rgba_64_mixed": rgba_64_mixed,
    "subfactor_256": subfactor_256,
    "large_16_6000x4000": large_16_6000x4000,
    "throughput_512_1024": throughput_512_1024,
    "video_8x64_1280x720": video_8x64_1280x720,
}


def uniform_images(shapes, seed: int) -> Batch:
    """Uniform pixels for an arbitrary list of (h, w, c) shapes (tests)."""
    return _uniform_batch("custom", [tuple(s) for s in shapes], seed,
                          mean=IMAGENET_MEAN, std=IMAGENET_STD, out_dtype="f32")
