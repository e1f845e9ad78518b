"""Batch helper over the C ABI: plan a batch, place its packed uint8 sources
in device memory, allocate outputs with torch, and run the fused kernel.

This is the equivalent of MimoV2ImageProcessor.__call__ (processing page):
images in, ``pixel_values`` [total_patches, 1536] and ``image_grid_thw``
[n, 3] out, in input order.  Decoding is out of scope: images arrive as
uint8 HWC arrays (RGB or RGBA).
"""
from __future__ import annotations

import contextlib
import functools
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from . import _abi

# MimoV2ImageProcessor defaults (processing page): ImageNet statistics.
IMAGENET_MEAN = (0.485, 0.456, 0.406)
IMAGENET_STD = (0.229, 0.224, 0.225)


@functools.lru_cache(maxsize=64)
def _stats255_cached(mean: tuple, std: tuple):
    m, s = _abi.stats255(mean, std)
    return tuple(m), tuple(s)


def stats255(mean, std):
    """Statistics in 0-255 units (mimo_stats255): float32(255 * v), the
    product formed in float64.  Cached per (mean, std)."""
    return _stats255_cached(tuple(float(v) for v in mean), tuple(float(v) for v in std))


def _on_stream(torch, stream, tensors):
    """The context a call runs in: with a caller's stream, that stream is
    made current, so the outputs and workspace allocated here belong to it in
    torch's caching allocator, and the caller's tensors are marked as used on
    it (their memory is not handed out again before its work has run)."""
    if stream is None:
        return contextlib.nullcontext()
    for t in tensors:
        if t is not None:
            t.record_stream(stream)
    return torch.cuda.stream(stream)


@dataclass
class BatchPlan:
    desc: np.ndarray          # IMAGE_DESC_DTYPE [n]
    total_rows: int
    total_src_bytes: int
    _grid: np.ndarray = None  # image_grid_thw, formed on first use

    @property
    def src_capacity(self) -> int:
        """Device bytes for the packed sources: the kernels read whole
        16-byte words, so the buffer is padded to a multiple of 16."""
        return max(16, (self.total_src_bytes + 15) // 16 * 16)

    @property
    def grid_thw(self) -> np.ndarray:
        """(grid_t, grid_h, grid_w) per item: image_grid_thw / video_grid_thw."""
        return self.image_grid_thw

    @property
    def image_grid_thw(self) -> np.ndarray:
        if self._grid is None:
            self._grid = np.stack([self.desc["grid_t"], self.desc["grid_h"], self.desc["grid_w"]],
                                  axis=1).astype(np.int64)
        return self._grid

    def __len__(self):
        return int(self.desc.shape[0])


def plan_batch(shapes, min_pixels=None, max_pixels=None, check: bool = True) -> BatchPlan:
    """Plans images given as (height, width, channels) tuples."""
    params = _abi.make_params(min_pixels, max_pixels)
    desc, rows, src, _ = _abi.plan_geometry(np.asarray(shapes, dtype=np.int32).reshape(-1, 3),
                                            params, check=check)
    return BatchPlan(desc=desc, total_rows=rows, total_src_bytes=src)


def plan_media(items, max_pixels=None, min_pixels=None, video_budget=None,
               check: bool = True) -> BatchPlan:
    """Plans still images and already-sampled clips given as (frames, height,
    width, channels) tuples (prepare_video_frames, inference page).

    max_pixels: one resized-area ceiling for every item, or one per item.
    video_budget: a clip's total pixel budget (one value or one per item; 0
    for none); where it is set, the item's ceiling is the per-frame share
    mimo_video_max_pixels gives for its sampled frame count.
    """
    params = _abi.make_params(min_pixels, None)
    items = np.asarray(items, dtype=np.int32).reshape(-1, 4)
    n = items.shape[0]
    ceilings = np.zeros(n, dtype=np.int64)
    if max_pixels is not None:
        ceilings[:] = np.broadcast_to(np.asarray(max_pixels, dtype=np.int64), (n,))
    if video_budget is not None:
        budget = np.broadcast_to(np.asarray(video_budget, dtype=np.int64), (n,))
        vparams = _abi.make_params(min_pixels, max_pixels if np.isscalar(max_pixels) else None)
        for i in range(n):
            if budget[i] > 0 and items[i, 0] > 0:
                ceilings[i] = _abi.video_max_pixels(int(items[i, 0]), int(budget[i]), vparams)
    desc, rows, src, _ = _abi.plan_frames(items, ceilings, params, check=check)
    return BatchPlan(desc=desc, total_rows=rows, total_src_bytes=src)


_STAGE_BYTES = 64 << 20          # one pinned staging chunk
_DIRECT_BYTES = 8 << 20          # smaller uploads copy straight from pageable memory
_stage_lock = threading.Lock()
_stages = {}                     # device index -> two pinned uint8 tensors of _STAGE_BYTES


def _pinned_stages(torch, index):
    """The device's two staging chunks (callers hold _stage_lock)."""
    if index not in _stages:
        _stages[index] = [torch.empty(_STAGE_BYTES, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
    return _stages[index]


def upload_sources(packed: np.ndarray, plan: BatchPlan, device="cuda"):
    """Copies packed uint8 images (back to back, batch order) into a padded
    device buffer; returns when the copy is done.

    Large batches go through two reusable pinned chunks: host threads fill
    one while the other's DMA copy runs, instead of one copy from pageable
    memory (which the runtime stages through a small buffer of its own).
    The chunks (128 MB of pinned host memory per device) are allocated on
    the first large upload and kept for the life of the process; large
    uploads from several threads take turns.
    """
    import torch
    dev = torch.device(device)
    if dev.type == "cuda" and dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    flat = np.ascontiguousarray(packed).reshape(-1)
    n = int(flat.size)
    buf = torch.empty(plan.src_capacity, dtype=torch.uint8, device=dev)
    if plan.src_capacity > n:
        buf[n:].zero_()
    if n == 0:
        return buf
    if n <= _DIRECT_BYTES:
        buf[:n].copy_(torch.from_numpy(flat))
        return buf
    stream = torch.cuda.current_stream(dev)
    done = [None, None]
    parts = 8
    # one chunked upload at a time: concurrent callers would share the chunks
    with _stage_lock, ThreadPoolExecutor(max_workers=parts) as pool:
        stages = _pinned_stages(torch, dev.index)
        for i, off in enumerate(range(0, n, _STAGE_BYTES)):
            k = i & 1
            if done[k] is not None:
                done[k].synchronize()      # this chunk's previous copy has run
            m = min(_STAGE_BYTES, n - off)
            host = stages[k].numpy()
            step = (m + parts - 1) // parts
            list(pool.map(lambda j: np.copyto(host[j:min(j + step, m)], flat[off + j:off + min(j + step, m)]),
                          range(0, m, step)))
            buf[off:off + m].copy_(stages[k][:m], non_blocking=True)
            done[k] = torch.cuda.Event()
            done[k].record(stream)
        for ev in done:
            if ev is not None:
                ev.synchronize()
    return buf


def preprocess(src_dev, plan: BatchPlan, mean=IMAGENET_MEAN, std=IMAGENET_STD,
               out_dtype: str = "f32", merge_order: bool = True, column_order: bool = False,
               stream=None, rows=None, rows_col=None, workspace=None):
    """Runs the fused pixel path on a planned batch.

    Returns a dict with ``pixel_values`` (merge-block order, or None),
    ``pixel_values_col`` (column order, or None) and ``image_grid_thw``.
    Preallocated ``rows`` / ``rows_col`` / ``workspace`` tensors may be
    passed to keep allocation out of a timed loop.
    """
    import torch
    dev = src_dev.device
    tdtype = {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    n_rows = max(plan.total_rows, 1)
    own_rows, own_col = merge_order and rows is None, column_order and rows_col is None
    with _on_stream(torch, stream, (src_dev, rows, rows_col, workspace)):
        if own_rows:
            rows = torch.empty((n_rows, _abi.ROW_LEN), dtype=tdtype, device=dev)
        if own_col:
            rows_col = torch.empty((n_rows, _abi.ROW_LEN), dtype=tdtype, device=dev)
        if workspace is None:
            workspace = torch.empty(max(_abi.workspace_bytes(len(plan)), 16), dtype=torch.uint8,
                                    device=dev)
        m255, s255 = stats255(mean, std)
        _abi.preprocess_batch(plan.desc, src_dev, m255, s255,
                              rows=rows if merge_order else None,
                              rows_col=rows_col if column_order else None,
                              workspace=workspace, stream=stream)
    # outputs allocated here hold at least one row (the library takes no null
    # output); hand back exactly the plan's rows
    if own_rows:
        rows = rows[:plan.total_rows]
    if own_col:
        rows_col = rows_col[:plan.total_rows]
    return {
        "pixel_values": rows if merge_order else None,
        "pixel_values_col": rows_col if column_order else None,
        "image_grid_thw": torch.from_numpy(plan.image_grid_thw),
    }


class ImageProcessor:
    """MimoV2ImageProcessor's call shape (NeMo Automodel
    "mimo_v2_flash.processing"): decoded images in, ``pixel_values`` and
    ``image_grid_thw`` out, in one kernel launch.

    The constructor takes the processor's arguments, in its order.  Images
    are uint8 arrays [height, width, 3 or 4] (RGB, or RGBA flattened onto
    white); decoding them is the caller's.  Defaults are the processor's:
    patch 16, temporal 2, merge 2, 8192..8388608 pixels, ImageNet
    statistics; other patch sizes raise MimoError (MIMO_E_UNSUPPORTED), as
    does a size the geometry rejects (its own code).
    """

    def __init__(self, patch_size: int = 16, temporal_patch_size: int = 2, merge_size: int = 2,
                 min_pixels=None, max_pixels=None, image_mean=IMAGENET_MEAN, image_std=IMAGENET_STD,
                 out_dtype: str = "f32", device="cuda"):
        if (patch_size, temporal_patch_size, merge_size) != (16, 2, 2):
            raise _abi.MimoError(_abi.MIMO_E_UNSUPPORTED,
                                 "ImageProcessor: the kernels are built for patch 16, temporal 2, merge 2")
        self.image_mean, self.image_std = tuple(image_mean), tuple(image_std)
        self.min_pixels, self.max_pixels = min_pixels, max_pixels
        self.out_dtype, self.device = out_dtype, device

    def __call__(self, images, min_pixels=None, max_pixels=None, column_order: bool = False):
        images = [np.asarray(im) for im in images]
        for im in images:
            if im.dtype != np.uint8 or im.ndim != 3 or im.shape[2] not in (3, 4):
                raise _abi.MimoError(_abi.MIMO_E_INVALID,
                                     "ImageProcessor: images must be uint8 [height, width, 3 or 4]")
        plan = plan_batch([im.shape for im in images],
                          self.min_pixels if min_pixels is None else min_pixels,
                          self.max_pixels if max_pixels is None else max_pixels)
        packed = (np.concatenate([np.ascontiguousarray(im).reshape(-1) for im in images])
                  if images else np.zeros(0, dtype=np.uint8))
        src = upload_sources(packed, plan, self.device)
        return preprocess(src, plan, mean=self.image_mean, std=self.image_std, out_dtype=self.out_dtype,
                          column_order=column_order)


class VideoProcessor:
    """The frames path of docs.rs "cortiq_engine::mimo_vision"
    (prepare_video_frames) on the GPU: already-sampled clips, and still
    images among them, in; ``pixel_values`` and ``video_grid_thw`` out, in
    one kernel launch.

    Each item is a uint8 array [frames, height, width, 3 or 4], or an image
    [height, width, 3 or 4] (one frame).  Frames 2t and 2t + 1 form
    temporal patch t; an odd count repeats its last frame.  ``video_budget``
    (a clip's total pixels, per call or per item; 0 for none) sets each
    clip's per-frame ceiling as mimo_video_max_pixels does.  Sampling frames
    out of a longer video is the caller's (smart_nframes, sample_frames).
    """

    def __init__(self, min_pixels=None, max_pixels=None, image_mean=IMAGENET_MEAN, image_std=IMAGENET_STD,
                 out_dtype: str = "f32", device="cuda"):
        self.image_mean, self.image_std = tuple(image_mean), tuple(image_std)
        self.min_pixels, self.max_pixels = min_pixels, max_pixels
        self.out_dtype, self.device = out_dtype, device

    def __call__(self, items, video_budget=None, column_order: bool = False):
        arrays = []
        for it in items:
            a = np.asarray(it)
            if a.ndim == 3:
                a = a[None]
            if a.dtype != np.uint8 or a.ndim != 4 or a.shape[0] < 1 or a.shape[3] not in (3, 4):
                raise _abi.MimoError(_abi.MIMO_E_INVALID, "VideoProcessor: items must be uint8 "
                                                          "[frames, height, width, 3 or 4] or [height, width, 3 or 4]")
            arrays.append(a)
        plan = plan_media([a.shape for a in arrays], max_pixels=self.max_pixels, min_pixels=self.min_pixels,
                          video_budget=video_budget)
        packed = (np.concatenate([np.ascontiguousarray(a).reshape(-1) for a in arrays])
                  if arrays else np.zeros(0, dtype=np.uint8))
        src = upload_sources(packed, plan, self.device)
        out = preprocess(src, plan, mean=self.image_mean, std=self.image_std, out_dtype=self.out_dtype,
                         column_order=column_order)
        out["video_grid_thw"] = out.pop("image_grid_thw")
        return out


def vit_tables(plan: BatchPlan, device="cuda", column: bool = False, rope_dim: int = 32,
               theta: float = _abi.ROPE_THETA, stream=None, workspace=None):
    """The ViT index tables of a planned batch (vision page,
    MiMoVisionTransformer._rotary_positions / _get_window_index; cortiq
    module conventions), for rows in merge-block order or, with column=True,
    column order:

    ``rotary_pos`` int32 [rows, 2] (h, w); ``rope_cos`` / ``rope_sin``
    float32 [rows, rope_dim] (h half, then w half); ``window_index`` /
    ``window_inverse`` int64 [rows / 4] (the identity for merge-block order);
    ``cu_seqlens`` int32 [chunks + 1] (one chunk per temporal slice).
    """
    import torch
    n_rows = max(plan.total_rows, 1)
    units = max(plan.total_rows // 4, 1)
    with _on_stream(torch, stream, (workspace,)):
        if workspace is None:
            workspace = torch.empty(max(_abi.workspace_bytes(len(plan)), 16), dtype=torch.uint8,
                                    device=device)
        pos = torch.empty((n_rows, 2), dtype=torch.int32, device=device)
        cos = torch.empty((n_rows, rope_dim), dtype=torch.float32, device=device)
        sin = torch.empty((n_rows, rope_dim), dtype=torch.float32, device=device)
        index = torch.empty(units, dtype=torch.int64, device=device)
        inverse = torch.empty(units, dtype=torch.int64, device=device)
        _abi.rotary_tables(plan.desc, workspace, pos=pos, cos=cos, sin=sin, column=column,
                           rope_dim=rope_dim, theta=theta, stream=stream)
        _abi.window_index(plan.desc, workspace, index=index, inverse=inverse, column_major=column,
                          stream=stream)
    rows = plan.total_rows
    return {
        "rotary_pos": pos[:rows], "rope_cos": cos[:rows], "rope_sin": sin[:rows],
        "window_index": index[:rows // 4], "window_inverse": inverse[:rows // 4],
        "cu_seqlens": torch.from_numpy(_abi.chunk_seqlens(plan.desc)),
    }


def plan_batch_hf(shapes, min_pixels=None, max_pixels=None, check: bool = True) -> BatchPlan:
    """Plans images with the stock Qwen2-VL geometry (the contrast path)."""
    params = _abi.make_params(min_pixels, max_pixels)
    desc, rows, src, _ = _abi.plan_hf(np.asarray(shapes, dtype=np.int32).reshape(-1, 3), params,
                                      check=check)
    return BatchPlan(desc=desc, total_rows=rows, total_src_bytes=src)


def preprocess_hf(src_dev, plan: BatchPlan, mean=IMAGENET_MEAN, std=IMAGENET_STD,
                  out_dtype: str = "f32", merge_order: bool = True, column_order: bool = False,
                  stream=None, rows=None, rows_col=None, workspace=None):
    """The stock processor's pixels for a plan from plan_batch_hf (processing page,
    module docstring: PIL antialiased bicubic to bytes, 0-1 statistics, alpha
    dropped); same outputs as preprocess()."""
    import torch
    dev = src_dev.device
    tdtype = {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    n_rows = max(plan.total_rows, 1)
    own_rows, own_col = merge_order and rows is None, column_order and rows_col is None
    with _on_stream(torch, stream, (src_dev, rows, rows_col, workspace)):
        if own_rows:
            rows = torch.empty((n_rows, _abi.ROW_LEN), dtype=tdtype, device=dev)
        if own_col:
            rows_col = torch.empty((n_rows, _abi.ROW_LEN), dtype=tdtype, device=dev)
        if workspace is None:
            workspace = torch.empty(max(_abi.hf_workspace_bytes(plan.desc), 16), dtype=torch.uint8,
                                    device=dev)
        _abi.preprocess_hf_batch(plan.desc, src_dev, mean, std, rows=rows if merge_order else None,
                                 rows_col=rows_col if column_order else None, workspace=workspace,
                                 stream=stream)
    # outputs allocated here hold at least one row (the library takes no null
    # output); hand back exactly the plan's rows
    if own_rows:
        rows = rows[:plan.total_rows]
    if own_col:
        rows_col = rows_col[:plan.total_rows]
    return {
        "pixel_values": rows if merge_order else None,
        "pixel_values_col": rows_col if column_order else None,
        "image_grid_thw": torch.from_numpy(plan.image_grid_thw),
    }


def prepare_pixel_embed_weights(w, bias=None, mean=IMAGENET_MEAN, std=IMAGENET_STD, stream=None):
    """The patch-embedding weight (bf16 [E, 1536], Conv3d (c, tt, py, px)
    order) and bias, prepared for embed_pixels with these statistics:
    (w_pixels bf16 [E, 768], bias_pixels float32 [E])."""
    m255, s255 = stats255(mean, std)
    return _abi.prepare_pixel_embed(w, m255, s255, bias=bias, stream=stream)


def embed_pixels(src_dev, plan: BatchPlan, w_pixels, bias_pixels, out_dtype: str = "bf16", out=None,
                 workspace=None, stream=None):
    """Still images straight to their patch embeddings (vision page,
    MiMoVisionPatchEmbed, over the processing page's pixels) in one kernel
    launch: out [total_rows, E], rows in merge-block order, as
    patch_embed(preprocess(...)) would give with the folded weight, but
    without writing the pixel rows."""
    import torch
    dev = src_dev.device
    e = w_pixels.shape[0]
    with _on_stream(torch, stream, (src_dev, w_pixels, bias_pixels, out, workspace)):
        if out is None:
            tdtype = {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
            out = torch.empty((max(plan.total_rows, 1), e), dtype=tdtype, device=dev)
        if workspace is None:
            workspace = torch.empty(max(_abi.workspace_bytes(len(plan)), 16), dtype=torch.uint8,
                                    device=dev)
        _abi.pixel_embed(plan.desc, src_dev, w_pixels, bias_pixels, out, workspace, stream=stream)
    return out[:plan.total_rows]
