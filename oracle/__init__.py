"""Plain CPU oracle of the MiMo-V2 image pixel path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``vision_image_preprocessing_amd``) never imports it, and the two share no
code: the C source here (``oracle.c``) is compiled by gcc on its own, with
``-ffp-contract=off`` so that the only fused multiply-adds are the explicit
``fmaf`` calls that reproduce torch's float32 resize arithmetic.

Each wrapper below names the passage of the pages it follows; the C source
carries the step-by-step definitions.  Pages:

* NeMo Automodel, ``mimo_v2_flash.processing`` (module docstring,
  ``MimoV2ImageProcessor``, ``smart_resize``, ``_to_rgb``,
  ``get_number_of_image_patches``);
* docs.rs ``cortiq_engine::mimo_vision`` (module conventions,
  ``resize_bilinear``, ``column_permutation``, ``smart_resize``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

OK = 0
E_INVALID = -1
E_ASPECT = -2
E_DEGENERATE = -3
E_NOMEM = -4

# Defaults of MimoV2ImageProcessor (processing page, class signature).
PATCH = 16
TEMPORAL = 2
MERGE = 2
MIN_PIXELS = 8192
MAX_PIXELS = 8388608
# Aspect guard of the Qwen2-VL smart_resize the processing page defers to.
MAX_ASPECT = 200.0

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-Wextra", _SRC, "-lm", "-o", tmp,
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
        ):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_smart_resize.argtypes = [i64, i64, i64, i64, i64, ctypes.c_double,
                                            ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.oracle_smart_resize.restype = ctypes.c_int
        lib.oracle_image_grid.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_double,
                                          p, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.oracle_image_grid.restype = ctypes.c_int
        lib.oracle_flatten_rgba.argtypes = [p, i64, p]
        lib.oracle_flatten_rgba.restype = None
        lib.oracle_resize_bilinear.argtypes = [p, i64, i64, i64, p, i64, i64]
        lib.oracle_resize_bilinear.restype = None
        lib.oracle_to_bf16.argtypes = [p, i64, p]
        lib.oracle_to_bf16.restype = None
        lib.oracle_preprocess_image.argtypes = [p, i64, i64, i64, i64, i64, i64, i64, i64,
                                                p, p, p]
        lib.oracle_preprocess_image.restype = ctypes.c_int
        lib.oracle_preprocess_rows.argtypes = [p, i64, i64, i64, i64, i64, i64, i64, i64,
                                               p, p, i64, i64, p]
        lib.oracle_preprocess_rows.restype = ctypes.c_int
        lib.oracle_column_permutation.argtypes = [i64, i64, i64, i64, p]
        lib.oracle_column_permutation.restype = ctypes.c_int
        lib.oracle_video_max_pixels.argtypes = [i64, i64, i64, i64, i64]
        lib.oracle_video_max_pixels.restype = i64
        lib.oracle_smart_nframes.argtypes = [i64, ctypes.c_double, ctypes.c_double, i64, i64]
        lib.oracle_smart_nframes.restype = i64
        lib.oracle_sample_frames.argtypes = [i64, i64, ctypes.c_double, p, p]
        lib.oracle_sample_frames.restype = i64
        lib.oracle_preprocess_video.argtypes = [p, i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                                p, p, p]
        lib.oracle_preprocess_video.restype = ctypes.c_int
        lib.oracle_rotary_positions.argtypes = [i64, i64, i64, i64, ctypes.c_int, p]
        lib.oracle_rotary_positions.restype = ctypes.c_int
        lib.oracle_rope_inv_freq.argtypes = [i64, ctypes.c_double, p]
        lib.oracle_rope_inv_freq.restype = ctypes.c_int
        lib.oracle_rope_tables.argtypes = [p, i64, i64, p, p, p, p]
        lib.oracle_rope_tables.restype = ctypes.c_int
        lib.oracle_window_index.argtypes = [i64, p, i64, ctypes.c_int, p]
        lib.oracle_window_index.restype = ctypes.c_int
        lib.oracle_chunk_seqlens.argtypes = [i64, p, p]
        lib.oracle_chunk_seqlens.restype = i64
        lib.oracle_patch_embed.argtypes = [p, i64, i64, p, i64, p, p]
        lib.oracle_patch_embed.restype = ctypes.c_int
        lib.oracle_hf_smart_resize.argtypes = [i64, i64, i64, i64, i64, ctypes.c_double,
                                               ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.oracle_hf_smart_resize.restype = ctypes.c_int
        lib.oracle_pil_resize_bicubic.argtypes = [p, i64, i64, i64, i64, i64, p]
        lib.oracle_pil_resize_bicubic.restype = ctypes.c_int
        lib.oracle_hf_preprocess_image.argtypes = [p, i64, i64, i64, i64, i64, i64, i64, i64,
                                                   p, p, p]
        lib.oracle_hf_preprocess_image.restype = ctypes.c_int
        _lib = lib
        return lib


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle status {code}")
        self.code = code


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def smart_resize(height: int, width: int, factor: int = PATCH * MERGE,
                 min_pixels: int = MIN_PIXELS, max_pixels: int = MAX_PIXELS,
                 max_aspect: float = MAX_ASPECT):
    """processing page, ``smart_resize``: (resized_height, resized_width).

    Raises OracleError with code E_INVALID, E_ASPECT or E_DEGENERATE.
    """
    lib = _load()
    oh, ow = ctypes.c_int64(), ctypes.c_int64()
    st = lib.oracle_smart_resize(height, width, factor, min_pixels, max_pixels,
                                 float(max_aspect), ctypes.byref(oh), ctypes.byref(ow))
    if st != OK:
        raise OracleError(st, f"smart_resize({height}, {width})")
    return oh.value, ow.value


def smart_resize_status(height, width, factor=PATCH * MERGE, min_pixels=MIN_PIXELS,
                        max_pixels=MAX_PIXELS, max_aspect=MAX_ASPECT):
    """Like smart_resize but returns (status, h, w) instead of raising."""
    lib = _load()
    oh, ow = ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib.oracle_smart_resize(height, width, factor, min_pixels, max_pixels,
                                 float(max_aspect), ctypes.byref(oh), ctypes.byref(ow))
    return st, oh.value, ow.value


def image_grid(height, width, patch=PATCH, merge=MERGE, min_pixels=MIN_PIXELS,
               max_pixels=MAX_PIXELS, max_aspect=MAX_ASPECT):
    """get_number_of_image_patches and the image_grid_thw entry.

    Returns ((grid_t, grid_h, grid_w), rows, tokens) with rows = gt*gh*gw
    patches and tokens = rows / merge**2.
    """
    lib = _load()
    g = np.zeros(3, dtype=np.int64)
    rows, tokens = ctypes.c_int64(), ctypes.c_int64()
    st = lib.oracle_image_grid(height, width, patch, merge, min_pixels, max_pixels,
                               float(max_aspect), _ptr(g), ctypes.byref(rows),
                               ctypes.byref(tokens))
    if st != OK:
        raise OracleError(st, f"image_grid({height}, {width})")
    return tuple(int(v) for v in g), rows.value, tokens.value


def flatten_rgba(rgba: np.ndarray) -> np.ndarray:
    """_to_rgb: RGBA [..., 4] uint8 flattened onto white -> RGB [..., 3] uint8."""
    rgba = np.ascontiguousarray(rgba, dtype=np.uint8)
    assert rgba.shape[-1] == 4
    npix = rgba.size // 4
    out = np.empty(rgba.shape[:-1] + (3,), dtype=np.uint8)
    _load().oracle_flatten_rgba(_ptr(rgba), npix, _ptr(out))
    return out


def resize_bilinear(planar: np.ndarray, out_h: int, out_w: int) -> np.ndarray:
    """resize_bilinear: planar float32 [C, H, W] -> [C, out_h, out_w]."""
    planar = np.ascontiguousarray(planar, dtype=np.float32)
    c, h, w = planar.shape
    out = np.empty((c, out_h, out_w), dtype=np.float32)
    _load().oracle_resize_bilinear(_ptr(planar), c, h, w, _ptr(out), out_h, out_w)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def _stats(mean255, std255):
    m = np.ascontiguousarray(np.asarray(mean255, dtype=np.float32).reshape(3))
    s = np.ascontiguousarray(np.asarray(std255, dtype=np.float32).reshape(3))
    return m, s


def preprocess_image(hwc: np.ndarray, out_h: int, out_w: int, mean255, std255,
                     patch: int = PATCH, merge: int = MERGE,
                     temporal: int = TEMPORAL) -> np.ndarray:
    """_process_one / prepare_image for one uint8 HWC image (C = 3 or 4).

    Returns float32 rows [(out_h/patch)*(out_w/patch), 3*temporal*patch*patch]
    in merge-block order.
    """
    hwc = np.ascontiguousarray(hwc, dtype=np.uint8)
    h, w, c = hwc.shape
    m, s = _stats(mean255, std255)
    rows = (out_h // patch) * (out_w // patch)
    out = np.empty((rows, 3 * temporal * patch * patch), dtype=np.float32)
    st = _load().oracle_preprocess_image(_ptr(hwc), h, w, c, out_h, out_w, patch, merge,
                                         temporal, _ptr(m), _ptr(s), _ptr(out))
    if st != OK:
        raise OracleError(st, "preprocess_image")
    return out


def preprocess_rows(hwc: np.ndarray, out_h: int, out_w: int, mean255, std255,
                    row_begin: int, row_count: int, patch: int = PATCH,
                    merge: int = MERGE, temporal: int = TEMPORAL) -> np.ndarray:
    """Rows [row_begin, row_begin+row_count) of preprocess_image, computed
    one element at a time (for sampling large batches)."""
    hwc = np.ascontiguousarray(hwc, dtype=np.uint8)
    h, w, c = hwc.shape
    m, s = _stats(mean255, std255)
    out = np.empty((row_count, 3 * temporal * patch * patch), dtype=np.float32)
    st = _load().oracle_preprocess_rows(_ptr(hwc), h, w, c, out_h, out_w, patch, merge,
                                        temporal, _ptr(m), _ptr(s), row_begin, row_count,
                                        _ptr(out))
    if st != OK:
        raise OracleError(st, "preprocess_rows")
    return out


def column_permutation(grid_t: int, grid_h: int, grid_w: int, merge: int = MERGE) -> np.ndarray:
    """cortiq column_permutation: perm[dst] = src, int64 [gt*gh*gw]."""
    perm = np.empty(grid_t * grid_h * grid_w, dtype=np.int64)
    st = _load().oracle_column_permutation(grid_t, grid_h, grid_w, merge, _ptr(perm))
    if st != OK:
        raise OracleError(st, "column_permutation")
    return perm


def stats255(mean, std):
    """Statistics in 0-255 units as float32: 255*mean and 255*std formed in
    float64 and rounded once (the processor's 0-255 normalisation)."""
    m = np.asarray([255.0 * float(v) for v in mean], dtype=np.float64).astype(np.float32)
    s = np.asarray([255.0 * float(v) for v in std], dtype=np.float64).astype(np.float32)
    return m, s


# ------------------------------------------------------------------ video
def video_max_pixels(n_sampled: int, total_max: int, temporal: int = TEMPORAL,
                     min_pixels: int = MIN_PIXELS, max_pixels: int = MAX_PIXELS) -> int:
    """cortiq video_max_pixels: per-frame pixel ceiling for n sampled frames."""
    v = _load().oracle_video_max_pixels(n_sampled, total_max, temporal, min_pixels, max_pixels)
    if v < 0:
        raise OracleError(v, "video_max_pixels")
    return int(v)


def smart_nframes(total: int, fps_src: float, fps: float, min_frames: int, max_frames: int) -> int:
    """cortiq smart_nframes: even frame count for `total` frames sampled at fps."""
    v = _load().oracle_smart_nframes(total, float(fps_src), float(fps), min_frames, max_frames)
    if v < 0:
        raise OracleError(v, "smart_nframes")
    return int(v)


def sample_frames(total: int, n: int, fps_src: float):
    """cortiq sample_frames: (indices int64, timestamps float32)."""
    idx = np.empty(max(n, 1), dtype=np.int64)
    ts = np.empty(max(n, 1), dtype=np.float32)
    k = _load().oracle_sample_frames(total, n, float(fps_src), _ptr(idx), _ptr(ts))
    if k < 0:
        raise OracleError(int(k), "sample_frames")
    return idx[:k].copy(), ts[:k].copy()


def preprocess_video(frames: np.ndarray, out_h: int, out_w: int, mean255, std255,
                     patch: int = PATCH, merge: int = MERGE, temporal: int = TEMPORAL) -> np.ndarray:
    """prepare_video_frames (pixel part) for uint8 frames [n, H, W, C]:
    rows [ceil(n/T)*(out_h/patch)*(out_w/patch), 3*T*patch*patch]."""
    frames = np.ascontiguousarray(frames, dtype=np.uint8)
    n, h, w, c = frames.shape
    m, s = _stats(mean255, std255)
    gt = -(-n // temporal)
    rows = gt * (out_h // patch) * (out_w // patch)
    out = np.empty((rows, 3 * temporal * patch * patch), dtype=np.float32)
    st = _load().oracle_preprocess_video(_ptr(frames), n, h, w, c, out_h, out_w, patch, merge,
                                         temporal, _ptr(m), _ptr(s), _ptr(out))
    if st != OK:
        raise OracleError(st, "preprocess_video")
    return out


# ------------------------------------------------------- ViT index tables
ROPE_THETA = 10000.0


def rotary_positions(grid_t: int, grid_h: int, grid_w: int, column: bool = False,
                     merge: int = MERGE) -> np.ndarray:
    """vision page, MiMoVisionTransformer._rotary_positions: int32 [rows, 2]
    (h, w) patch coordinates of every row, in merge-block order or, with
    column=True, in column order."""
    rows = grid_t * grid_h * grid_w
    pos = np.empty((rows, 2), dtype=np.int32)
    st = _load().oracle_rotary_positions(grid_t, grid_h, grid_w, merge, int(bool(column)), _ptr(pos))
    if st != OK:
        raise OracleError(st, "rotary_positions")
    return pos


def rope_inv_freq(dim: int, theta: float = ROPE_THETA) -> np.ndarray:
    """vision page, MiMoVisionRotaryEmbedding(dim, theta) inv_freq: float32 [dim/2]."""
    inv = np.empty(dim // 2, dtype=np.float32)
    st = _load().oracle_rope_inv_freq(dim, float(theta), _ptr(inv))
    if st != OK:
        raise OracleError(st, "rope_inv_freq")
    return inv


def rope_tables(pos: np.ndarray, dim: int, theta: float = ROPE_THETA):
    """Rotary angles (float32 [rows, dim]: h half, then w half) and their
    cosine and sine in float64, for int32 [rows, 2] positions."""
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    rows = pos.shape[0]
    inv = rope_inv_freq(dim, theta)
    angle = np.empty((rows, dim), dtype=np.float32)
    c = np.empty((rows, dim), dtype=np.float64)
    s = np.empty((rows, dim), dtype=np.float64)
    st = _load().oracle_rope_tables(_ptr(pos), rows, dim, _ptr(inv), _ptr(angle), _ptr(c), _ptr(s))
    if st != OK:
        raise OracleError(st, "rope_tables")
    return angle, c, s


def window_index(grid_thw, column_major: bool, merge: int = MERGE) -> np.ndarray:
    """vision page, MiMoVisionTransformer._get_window_index(grid_thw,
    column_major): int64 [units], index[dst] = src over the batch's merge
    units."""
    thw = np.ascontiguousarray(np.asarray(grid_thw, dtype=np.int64).reshape(-1, 3))
    units = int(sum(t * (h // merge) * (w // merge) for t, h, w in thw))
    index = np.empty(max(units, 1), dtype=np.int64)
    st = _load().oracle_window_index(thw.shape[0], _ptr(thw), merge, int(bool(column_major)),
                                      _ptr(index))
    if st != OK:
        raise OracleError(st, "window_index")
    return index[:units]


def chunk_seqlens(grid_thw) -> np.ndarray:
    """Cumulative rows per attention chunk (one chunk per temporal slice of
    every item): int64 [chunks + 1]."""
    thw = np.ascontiguousarray(np.asarray(grid_thw, dtype=np.int64).reshape(-1, 3))
    cu = np.empty(int(thw[:, 0].sum()) + 1 if thw.size else 1, dtype=np.int64)
    k = _load().oracle_chunk_seqlens(thw.shape[0], _ptr(thw), _ptr(cu))
    if k < 0:
        raise OracleError(int(k), "chunk_seqlens")
    return cu[:k + 1]


# ------------------------------------------------------------ patch embedding
def patch_embed(rows: np.ndarray, w: np.ndarray, bias=None) -> np.ndarray:
    """vision page, MiMoVisionPatchEmbed: the Conv3d (kernel = stride =
    (T, P, P)) on rows [n, C*T*P*P] with weight [E, C, T, P, P] given
    flattened [E, C*T*P*P]; float64 [n, E]."""
    rows = np.ascontiguousarray(rows, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(w.shape[0], -1)
    n, k = rows.shape
    e = w.shape[0]
    assert w.shape[1] == k
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((n, e), dtype=np.float64)
    st = _load().oracle_patch_embed(_ptr(rows), n, k, _ptr(w), e, _ptr(b) if b is not None else None,
                                    _ptr(out))
    if st != OK:
        raise OracleError(st, "patch_embed")
    return out


# ------------------------------------------------- stock-HF contrast path
def hf_smart_resize_status(height: int, width: int, factor: int = PATCH * MERGE,
                           min_pixels: int = MIN_PIXELS, max_pixels: int = MAX_PIXELS,
                           max_aspect: float = MAX_ASPECT):
    """processing page, module docstring: the stock Qwen2-VL smart_resize
    (each side clamped on its own, no short-side upscale): (status, h, w)."""
    oh, ow = ctypes.c_int64(0), ctypes.c_int64(0)
    st = _load().oracle_hf_smart_resize(height, width, factor, min_pixels, max_pixels,
                                        float(max_aspect), ctypes.byref(oh), ctypes.byref(ow))
    return st, oh.value, ow.value


def hf_smart_resize(height: int, width: int, **kw):
    st, oh, ow = hf_smart_resize_status(height, width, **kw)
    if st != OK:
        raise OracleError(st, f"hf_smart_resize({height}, {width})")
    return oh, ow


def pil_resize_bicubic(img: np.ndarray, out_h: int, out_w: int) -> np.ndarray:
    """PIL's 8-bit antialiased bicubic resize of uint8 [h, w, c]."""
    img = np.ascontiguousarray(img, dtype=np.uint8)
    h, w, c = img.shape
    out = np.empty((out_h, out_w, c), dtype=np.uint8)
    st = _load().oracle_pil_resize_bicubic(_ptr(img), h, w, c, out_h, out_w, _ptr(out))
    if st != OK:
        raise OracleError(st, "pil_resize_bicubic")
    return out


def hf_preprocess_image(hwc: np.ndarray, out_h: int, out_w: int, mean01, std01,
                        patch: int = PATCH, merge: int = MERGE, temporal: int = TEMPORAL) -> np.ndarray:
    """The stock processor's pixel path for one image (alpha dropped, PIL
    bicubic to uint8, 0-1 rescale, float32 normalise): float32 rows in
    merge-block order."""
    hwc = np.ascontiguousarray(hwc, dtype=np.uint8)
    h, w, c = hwc.shape
    m = np.ascontiguousarray(np.asarray(mean01, dtype=np.float32))
    s = np.ascontiguousarray(np.asarray(std01, dtype=np.float32))
    rows = np.empty(((out_h // patch) * (out_w // patch), 3 * temporal * patch * patch), dtype=np.float32)
    st = _load().oracle_hf_preprocess_image(_ptr(hwc), h, w, c, out_h, out_w, patch, merge, temporal,
                                            _ptr(m), _ptr(s), _ptr(rows))
    if st != OK:
        raise OracleError(st, "hf_preprocess_image")
    return rows
