"""MI355X-native MiMo-V2 image pixel path.

The pixel path of the pages (NeMo Automodel ``mimo_v2_flash.processing``,
class ``MimoV2ImageProcessor``; docs.rs ``cortiq_engine::mimo_vision``):
RGBA flattened onto white, cast to 0-255 float, bilinear resize
(align_corners=False, no antialias) to the smart_resize target, per-channel
standardisation in 0-255 units, two identical frames, Conv3d patch rows of
1536 values in merge-block order, and optionally the column-order
permutation.  All of it runs in hand-written HIP kernels for gfx950 behind
the C ABI in ``include/mimo_pre.h``; this package is the ctypes binding plus
a batch helper that allocates torch device buffers.
"""
from __future__ import annotations

from ._abi import (  # noqa: F401
    IMAGE_DESC_DTYPE, MIMO_BF16, MIMO_E_ASPECT, MIMO_E_CAPACITY, MIMO_E_DEGENERATE,
    MIMO_E_HIP, MIMO_E_INVALID, MIMO_E_TOO_LARGE, MIMO_E_UNSUPPORTED, MIMO_F32, MIMO_OK,
    ROW_LEN, LibraryNotBuilt, MimoError, MimoParams, column_permutation, column_permute,
    chunk_seqlens, default_params, dispatch_count, fold_patch_weights, get_number_of_image_patches,
    hf_matrix_dispatch_count,
    hf_smart_resize,
    hf_workspace_bytes, last_error, load, make_params, patch_embed, plan_frames, plan_geometry,
    plan_hf,
    pixel_embed, prepare_pixel_embed, preprocess_batch_noalloc,
    preprocess_hf_batch, preprocess_batch, rope_inv_freq, rotary_tables, sample_frames,
    set_launch_events, smart_nframes, smart_resize, status_string, video_max_pixels,
    window_index, workspace_bytes,
)
from .processor import (  # noqa: F401
    BatchPlan, ImageProcessor, VideoProcessor, embed_pixels, plan_batch, plan_batch_hf, plan_media,
    prepare_pixel_embed_weights, preprocess, preprocess_hf, stats255, vit_tables,
)
