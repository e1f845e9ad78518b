"""ctypes binding of libmimopre.so (the C ABI declared in include/mimo_pre.h).

Argument marshalling only: every step of the pixel path runs in the HIP
library.  PyTorch supplies device memory (``data_ptr()``) and the current
HIP stream.  Importing this module does not need a GPU; loading the library
fails loudly if it has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

from .build import LIB_PATH

MIMO_OK = 0
MIMO_E_INVALID = -1
MIMO_E_ASPECT = -2
MIMO_E_DEGENERATE = -3
MIMO_E_UNSUPPORTED = -4
MIMO_E_CAPACITY = -5
MIMO_E_HIP = -6
MIMO_E_TOO_LARGE = -7

MIMO_F32 = 0
MIMO_BF16 = 1

ROW_LEN = 1536  # 3 channels x 2 frames x 16 x 16
MIMO_ORDER_MERGE = 0
MIMO_ORDER_COLUMN = 1
MIMO_ROPE_DIM_MAX = 256
ROPE_THETA = 10000.0

# mimo_image_desc, 64 bytes (include/mimo_pre.h)
IMAGE_DESC_DTYPE = np.dtype([
    ("src_offset", "<i8"), ("row_offset", "<i8"), ("rows", "<i8"),
    ("src_h", "<i4"), ("src_w", "<i4"), ("channels", "<i4"),
    ("dst_h", "<i4"), ("dst_w", "<i4"),
    ("grid_t", "<i4"), ("grid_h", "<i4"), ("grid_w", "<i4"),
    ("status", "<i4"), ("frames", "<i4"),
])
assert IMAGE_DESC_DTYPE.itemsize == 64


class MimoParams(ctypes.Structure):
    """mimo_params: processor knobs (patch, merge, temporal, pixel bounds,
    aspect guard)."""
    _fields_ = [
        ("patch_size", ctypes.c_int32),
        ("merge_size", ctypes.c_int32),
        ("temporal_patch_size", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("min_pixels", ctypes.c_int64),
        ("max_pixels", ctypes.c_int64),
        ("max_aspect", ctypes.c_double),
    ]


class MimoError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{message} [status {code}]")
        self.code = code


class LibraryNotBuilt(RuntimeError):
    pass


# exported symbol -> (argtypes, restype)
_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "mimo_default_params": ([_P], None),
    "mimo_smart_resize": ([_I64, _I64, _P, _P, _P], ctypes.c_int),
    "mimo_plan_geometry": ([_I32, _P, _P, _P, _P, _P], ctypes.c_int),
    "mimo_plan_frames": ([_I32, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "mimo_video_max_pixels": ([_I64, _I64, _P], _I64),
    "mimo_smart_nframes": ([_I64, ctypes.c_double, ctypes.c_double, _I64, _I64], _I64),
    "mimo_sample_frames": ([_I64, _I64, ctypes.c_double, _P, _P], _I64),
    "mimo_workspace_bytes": ([_I32], _SZ),
    "mimo_stats255": ([_P, _P, _P, _P], ctypes.c_int),
    "mimo_preprocess_batch": ([_I32, _P, _P, _I64, _P, _P, _I32, _P, _P, _I64, _P, _SZ, _P],
                              ctypes.c_int),
    "mimo_preprocess_batch_noalloc": ([_I32, _P, _P, _I64, _P, _P, _I32, _P, _P, _I64, _P],
                                      ctypes.c_int),
    "mimo_column_permutation": ([_I64, _I64, _I64, _I64, _P], ctypes.c_int),
    "mimo_column_permute": ([_I32, _P, _P, _P, _I32, _I64, _P, _SZ, _P], ctypes.c_int),
    "mimo_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "mimo_last_error": ([], ctypes.c_char_p),
    "mimo_dispatch_count": ([], _I64),
    "mimo_hf_matrix_dispatch_count": ([], _I64),
    "mimo_set_launch_events": ([_P, _P], ctypes.c_int),
    "mimo_rope_inv_freq": ([_I32, ctypes.c_double, _P], ctypes.c_int),
    "mimo_rotary_tables": ([_I32, _P, _I32, _I32, ctypes.c_double, _P, _P, _P, _I64, _P, _SZ, _P],
                           ctypes.c_int),
    "mimo_window_index": ([_I32, _P, _I32, _P, _P, _I64, _P, _SZ, _P], ctypes.c_int),
    "mimo_chunk_seqlens": ([_I32, _P, _P, _I64], _I64),
    "mimo_fold_patch_weights": ([_I32, _P, _P, _P], ctypes.c_int),
    "mimo_hf_smart_resize": ([_I64, _I64, _P, ctypes.POINTER(_I64), ctypes.POINTER(_I64)], ctypes.c_int),
    "mimo_plan_hf": ([_I32, _P, _P, _P, _P, _P], ctypes.c_int),
    "mimo_hf_workspace_bytes": ([_I32, _P], _SZ),
    "mimo_preprocess_hf_batch": ([_I32, _P, _P, _I64, _P, _P, _I32, _P, _P, _I64, _P, _SZ, _P],
                                 ctypes.c_int),
    "mimo_patch_embed": ([_I64, _P, _I32, _P, _I32, _P, _I32, _P, _P], ctypes.c_int),
    "mimo_prepare_pixel_embed": ([_I32, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "mimo_pixel_embed": ([_I32, _P, _P, _I64, _I32, _P, _P, _I32, _P, _I64, _P, _SZ, _P], ctypes.c_int),
}

_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Loads the in-tree HIP library; raises LibraryNotBuilt if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(
                f"{LIB_PATH} is missing: build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
        # torch ships its own HIP runtime under the same sonames as the
        # system's; whichever loads first serves the whole process.  The
        # device memory handed to the library comes from torch, so torch's
        # runtime must be the one: import torch before opening the library
        # (loaded first, the library would pull in the system runtime and
        # torch would then find no device).
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
        return lib


def _check(code: int, what: str):
    if code != MIMO_OK:
        raise MimoError(code, f"{what}: {last_error() or status_string(code)}")


def status_string(code: int) -> str:
    return load().mimo_status_string(code).decode()


def last_error() -> str:
    return load().mimo_last_error().decode()


def dispatch_count() -> int:
    return int(load().mimo_dispatch_count())


def hf_matrix_dispatch_count() -> int:
    """mimo_hf_matrix_dispatch_count: contrast launches that ran the
    matrix-core instance."""
    return int(load().mimo_hf_matrix_dispatch_count())


def set_launch_events(start=None, stop=None):
    """mimo_set_launch_events: torch.cuda.Event pair recorded right around
    each later kernel launch on this thread (None, None to stop).  The events
    must already exist (record them once first)."""
    h = lambda e: None if e is None else ctypes.c_void_p(int(e.cuda_event))
    if start is not None and (not start.cuda_event or not stop.cuda_event):
        raise MimoError(MIMO_E_INVALID, "set_launch_events: record the events once first")
    _check(load().mimo_set_launch_events(h(start), h(stop)), "set_launch_events")


def default_params() -> MimoParams:
    p = MimoParams()
    load().mimo_default_params(ctypes.byref(p))
    return p


def make_params(min_pixels=None, max_pixels=None, **kw) -> MimoParams:
    """Defaults with per-call pixel-bound overrides (MimoV2ImageProcessor
    __call__ accepts min_pixels / max_pixels per call)."""
    p = default_params()
    if min_pixels is not None:
        p.min_pixels = int(min_pixels)
    if max_pixels is not None:
        p.max_pixels = int(max_pixels)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def smart_resize(height: int, width: int, params: MimoParams | None = None):
    """mimo_smart_resize -> (resized_height, resized_width)."""
    oh, ow = ctypes.c_int64(), ctypes.c_int64()
    code = load().mimo_smart_resize(int(height), int(width),
                                    ctypes.byref(params) if params is not None else None,
                                    ctypes.byref(oh), ctypes.byref(ow))
    _check(code, "smart_resize")
    return oh.value, ow.value


def plan_geometry(hwc, params: MimoParams | None = None, check: bool = True):
    """mimo_plan_geometry over an [n, 3] (height, width, channels) table.

    Returns (desc, total_rows, total_src_bytes, status) where desc is a
    structured numpy array of IMAGE_DESC_DTYPE.  With check=True a failing
    image raises MimoError; otherwise per-image codes are in desc['status'].
    """
    hwc = np.ascontiguousarray(np.asarray(hwc, dtype=np.int32).reshape(-1, 3))
    n = hwc.shape[0]
    desc = np.zeros(n, dtype=IMAGE_DESC_DTYPE)
    total_rows, total_src = ctypes.c_int64(), ctypes.c_int64()
    code = load().mimo_plan_geometry(n, hwc.ctypes.data,
                                     ctypes.byref(params) if params is not None else None,
                                     desc.ctypes.data, ctypes.byref(total_rows),
                                     ctypes.byref(total_src))
    if check:
        _check(code, "plan_geometry")
    return desc, total_rows.value, total_src.value, code


def get_number_of_image_patches(height: int, width: int, min_pixels=None, max_pixels=None) -> int:
    """The processor's get_number_of_image_patches (NeMo Automodel
    "mimo_v2_flash.processing"): patches (= rows, grid_h * grid_w) of one
    image of that size, from mimo_plan_geometry; raises MimoError for a size
    the geometry rejects."""
    desc, _, _, _ = plan_geometry([(int(height), int(width), 3)], make_params(min_pixels, max_pixels))
    return int(desc["rows"][0])


def plan_frames(fhwc, max_pixels=None, params: MimoParams | None = None, check: bool = True):
    """mimo_plan_frames over an [n, 4] (frames, height, width, channels)
    table; max_pixels: optional per-item resized-area ceilings ([n] int64,
    <= 0 for the default).  Returns (desc, total_rows, total_src_bytes,
    status) like plan_geometry."""
    fhwc = np.ascontiguousarray(np.asarray(fhwc, dtype=np.int32).reshape(-1, 4))
    n = fhwc.shape[0]
    mp = None
    if max_pixels is not None:
        mp = np.ascontiguousarray(np.asarray(max_pixels, dtype=np.int64).reshape(n))
    desc = np.zeros(n, dtype=IMAGE_DESC_DTYPE)
    total_rows, total_src = ctypes.c_int64(), ctypes.c_int64()
    code = load().mimo_plan_frames(n, fhwc.ctypes.data, mp.ctypes.data if mp is not None else None,
                                   ctypes.byref(params) if params is not None else None,
                                   desc.ctypes.data, ctypes.byref(total_rows),
                                   ctypes.byref(total_src))
    if check:
        _check(code, "plan_frames")
    return desc, total_rows.value, total_src.value, code


def video_max_pixels(n_sampled: int, total_max: int, params: MimoParams | None = None) -> int:
    """mimo_video_max_pixels: per-frame pixel ceiling for n sampled frames."""
    v = load().mimo_video_max_pixels(int(n_sampled), int(total_max),
                                     ctypes.byref(params) if params is not None else None)
    if v < 0:
        _check(int(v), "video_max_pixels")
    return int(v)


def smart_nframes(total: int, fps_src: float, fps: float, min_frames: int, max_frames: int) -> int:
    """mimo_smart_nframes: even frame count for a video of `total` frames."""
    v = load().mimo_smart_nframes(int(total), float(fps_src), float(fps), int(min_frames),
                                  int(max_frames))
    if v < 0:
        _check(int(v), "smart_nframes")
    return int(v)


def sample_frames(total: int, n: int, fps_src: float):
    """mimo_sample_frames: (indices int64, timestamps float32)."""
    idx = np.empty(max(int(n), 1), dtype=np.int64)
    ts = np.empty(max(int(n), 1), dtype=np.float32)
    k = load().mimo_sample_frames(int(total), int(n), float(fps_src), idx.ctypes.data, ts.ctypes.data)
    if k < 0:
        _check(int(k), "sample_frames")
    return idx[:k].copy(), ts[:k].copy()


def workspace_bytes(n: int) -> int:
    return int(load().mimo_workspace_bytes(int(n)))


def stats255(mean, std):
    """mimo_stats255: the processor's 0-1 statistics in 0-255 units, as the
    float32 lists (mean255, std255) that preprocess_batch takes."""
    m01 = (ctypes.c_double * 3)(*[float(v) for v in mean])
    s01 = (ctypes.c_double * 3)(*[float(v) for v in std])
    m255, s255 = (ctypes.c_float * 3)(), (ctypes.c_float * 3)()
    _check(load().mimo_stats255(m01, s01, m255, s255), "stats255")
    return list(m255), list(s255)


def column_permutation(grid_t: int, grid_h: int, grid_w: int, merge: int = 2) -> np.ndarray:
    """mimo_column_permutation: perm[dst] = src (int64)."""
    perm = np.empty(int(grid_t) * int(grid_h) * int(grid_w), dtype=np.int64)
    code = load().mimo_column_permutation(grid_t, grid_h, grid_w, merge, perm.ctypes.data)
    _check(code, "column_permutation")
    return perm


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(int(stream.cuda_stream))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MIMO_F32
    if t.dtype == torch.bfloat16:
        return MIMO_BF16
    raise MimoError(MIMO_E_INVALID, f"output dtype {t.dtype} is not float32 or bfloat16")


def _require(ok: bool, what):
    """Raises MimoError(MIMO_E_INVALID) unless ok; `what` is the message or a
    callable that makes it (formatted only on failure)."""
    if not ok:
        raise MimoError(MIMO_E_INVALID, what() if callable(what) else what)


def _check_matrix(t, what: str, width: int, dtypes):
    """t must be a contiguous 2-D tensor [capacity, width] of one of dtypes."""
    if t.dim() == 2 and t.shape[1] == width and t.dtype in dtypes and t.is_contiguous():
        return
    raise MimoError(MIMO_E_INVALID,
                    f"{what}: need a contiguous [capacity, {width}] tensor of "
                    f"{' or '.join(str(d) for d in dtypes)}, got {tuple(t.shape)} {t.dtype}"
                    + ("" if t.is_contiguous() else " (not contiguous)"))


def _check_bytes(t, what: str):
    """t must be a contiguous uint8 tensor (its numel is its size in bytes)."""
    import torch
    if t.dtype == torch.uint8 and t.dim() == 1 and t.is_contiguous():
        return
    raise MimoError(MIMO_E_INVALID, f"{what}: need a contiguous 1-D uint8 tensor, got {tuple(t.shape)} {t.dtype}")


def _check_device(tensors, what: str):
    """Every tensor lives on one GPU (checked after shapes and dtypes, so
    mis-shaped host tensors are reported as such)."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        d = t.device
        if d.type != "cuda" or (dev is not None and d != dev):
            devs = sorted({str(x.device) for x in tensors if x is not None})
            raise MimoError(MIMO_E_INVALID, f"{what}: every tensor must be on one GPU, got {devs}")
        dev = d


_ROW_DTYPES = None  # (torch.float32, torch.bfloat16), set on first use


def _row_dtypes():
    global _ROW_DTYPES
    if _ROW_DTYPES is None:
        import torch
        _ROW_DTYPES = (torch.float32, torch.bfloat16)
    return _ROW_DTYPES


def _out_tensors(rows, rows_col, what: str):
    """Checks the pixel-path outputs: one or two contiguous [capacity, 1536]
    tensors of one dtype (float32 or bfloat16); returns (dtype code,
    capacity)."""
    dts = _row_dtypes()
    if rows is None and rows_col is None:
        raise MimoError(MIMO_E_INVALID, f"{what}: both outputs are None")
    first = rows if rows is not None else rows_col
    _check_matrix(first, what + " output", ROW_LEN, dts)
    cap = first.shape[0]
    if rows is not None and rows_col is not None:
        _check_matrix(rows_col, what + " output", ROW_LEN, dts)
        _require(rows_col.dtype == first.dtype, lambda: f"{what}: the two outputs differ in dtype")
        cap = min(cap, rows_col.shape[0])
    return (MIMO_F32 if first.dtype == dts[0] else MIMO_BF16), cap


def preprocess_batch(desc: np.ndarray, src, mean255, std255, rows=None, rows_col=None,
                     workspace=None, stream=None):
    """mimo_preprocess_batch.  src: uint8 device tensor (packed images,
    length >= packed size rounded up to 16); rows / rows_col: float32 or
    bfloat16 device tensors [capacity, 1536] (either may be None);
    workspace: uint8 device tensor of >= workspace_bytes(n) bytes.
    Enqueues on `stream` (default: torch's current stream)."""
    desc = np.ascontiguousarray(desc, dtype=IMAGE_DESC_DTYPE)
    n = desc.shape[0]
    code_dtype, cap = _out_tensors(rows, rows_col, "preprocess_batch")
    out = rows if rows is not None else rows_col
    _check_bytes(src, "preprocess_batch: src")
    _require(workspace is not None, "preprocess_batch: workspace is None")
    _check_bytes(workspace, "preprocess_batch: workspace")
    _check_device([src, rows, rows_col, workspace], "preprocess_batch")
    m = (ctypes.c_float * 3)(*[float(v) for v in mean255])
    s = (ctypes.c_float * 3)(*[float(v) for v in std255])
    code = load().mimo_preprocess_batch(
        n, desc.ctypes.data, src.data_ptr(), src.numel(), m, s, code_dtype,
        rows.data_ptr() if rows is not None else None,
        rows_col.data_ptr() if rows_col is not None else None,
        cap, workspace.data_ptr(), workspace.numel(), _stream_handle(stream, out.device))
    _check(code, "preprocess_batch")


NOALLOC_MAX_IMAGES = 8192  # MIMO_NOALLOC_MAX_IMAGES


def preprocess_batch_noalloc(desc: np.ndarray, src, mean255, std255, rows=None, rows_col=None,
                             stream=None):
    """mimo_preprocess_batch_noalloc: preprocess_batch with the descriptor
    tables in the library's static device scratch (no workspace, nothing
    allocated); at most NOALLOC_MAX_IMAGES images.  Calls that overlap on
    one GPU race on the scratch."""
    desc = np.ascontiguousarray(desc, dtype=IMAGE_DESC_DTYPE)
    n = desc.shape[0]
    code_dtype, cap = _out_tensors(rows, rows_col, "preprocess_batch_noalloc")
    out = rows if rows is not None else rows_col
    _check_bytes(src, "preprocess_batch_noalloc: src")
    _check_device([src, rows, rows_col], "preprocess_batch_noalloc")
    m = (ctypes.c_float * 3)(*[float(v) for v in mean255])
    s = (ctypes.c_float * 3)(*[float(v) for v in std255])
    code = load().mimo_preprocess_batch_noalloc(
        n, desc.ctypes.data, src.data_ptr(), src.numel(), m, s, code_dtype,
        rows.data_ptr() if rows is not None else None,
        rows_col.data_ptr() if rows_col is not None else None,
        cap, _stream_handle(stream, out.device))
    _check(code, "preprocess_batch_noalloc")


def column_permute(desc: np.ndarray, rows_in, rows_out, workspace, stream=None):
    """mimo_column_permute: merge-order rows -> column-order rows (gather)."""
    import torch
    desc = np.ascontiguousarray(desc, dtype=IMAGE_DESC_DTYPE)
    n = desc.shape[0]
    for t, name in ((rows_in, "rows_in"), (rows_out, "rows_out")):
        _check_matrix(t, "column_permute: " + name, ROW_LEN, (torch.float32, torch.bfloat16))
    _require(rows_in.dtype == rows_out.dtype, "column_permute: rows_in and rows_out differ in dtype")
    code_dtype = _dtype_code(rows_in)
    _check_bytes(workspace, "column_permute: workspace")
    _check_device([rows_in, rows_out, workspace], "column_permute")
    cap = min(rows_in.shape[0], rows_out.shape[0])
    code = load().mimo_column_permute(n, desc.ctypes.data, rows_in.data_ptr(), rows_out.data_ptr(),
                                      code_dtype, cap, workspace.data_ptr(), workspace.numel(),
                                      _stream_handle(stream, rows_in.device))
    _check(code, "column_permute")


def rope_inv_freq(rope_dim: int, theta: float = ROPE_THETA) -> np.ndarray:
    """mimo_rope_inv_freq: float32 [rope_dim / 2]."""
    inv = np.empty(max(int(rope_dim) // 2, 1), dtype=np.float32)
    _check(load().mimo_rope_inv_freq(int(rope_dim), float(theta), inv.ctypes.data), "rope_inv_freq")
    return inv[:int(rope_dim) // 2]


def rotary_tables(desc: np.ndarray, workspace, pos=None, cos=None, sin=None, column=False,
                  rope_dim: int = 32, theta: float = ROPE_THETA, stream=None):
    """mimo_rotary_tables: fills the given device tensors (pos int32 [rows, 2],
    cos / sin float32 [rows, rope_dim]) for the rows in merge-block order, or
    column order with column=True."""
    import torch
    desc = np.ascontiguousarray(desc, dtype=IMAGE_DESC_DTYPE)
    outs = [t for t in (pos, cos, sin) if t is not None]
    _require(bool(outs), "rotary_tables: no output given")
    if pos is not None:
        _check_matrix(pos, "rotary_tables: pos", 2, (torch.int32,))
    for t, name in ((cos, "cos"), (sin, "sin")):
        if t is not None:
            _check_matrix(t, "rotary_tables: " + name, int(rope_dim), (torch.float32,))
    _check_bytes(workspace, "rotary_tables: workspace")
    _check_device(outs + [workspace], "rotary_tables")
    cap = min(t.shape[0] for t in outs)
    dev = outs[0].device
    code = load().mimo_rotary_tables(
        desc.shape[0], desc.ctypes.data, MIMO_ORDER_COLUMN if column else MIMO_ORDER_MERGE,
        int(rope_dim), float(theta),
        pos.data_ptr() if pos is not None else None,
        cos.data_ptr() if cos is not None else None,
        sin.data_ptr() if sin is not None else None,
        cap, workspace.data_ptr(), workspace.numel(), _stream_handle(stream, dev))
    _check(code, "rotary_tables")


def window_index(desc: np.ndarray, workspace, index=None, inverse=None, column_major=True,
                 stream=None):
    """mimo_window_index: fills int64 device tensors [units] (index[dst] = src,
    inverse[src] = dst)."""
    import torch
    desc = np.ascontiguousarray(desc, dtype=IMAGE_DESC_DTYPE)
    outs = [t for t in (index, inverse) if t is not None]
    _require(bool(outs), "window_index: no output given")
    for t in outs:
        _require(t.dim() == 1 and t.dtype == torch.int64 and t.is_contiguous(),
                 f"window_index: need contiguous 1-D int64 outputs, got {tuple(t.shape)} {t.dtype}")
    _check_bytes(workspace, "window_index: workspace")
    _check_device(outs + [workspace], "window_index")
    cap = min(t.shape[0] for t in outs)
    dev = outs[0].device
    code = load().mimo_window_index(
        desc.shape[0], desc.ctypes.data, int(bool(column_major)),
        index.data_ptr() if index is not None else None,
        inverse.data_ptr() if inverse is not None else None,
        cap, workspace.data_ptr(), workspace.numel(), _stream_handle(stream, dev))
    _check(code, "window_index")


def chunk_seqlens(desc: np.ndarray) -> np.ndarray:
    """mimo_chunk_seqlens: int32 [chunks + 1] cumulative rows per chunk."""
    desc = np.ascontiguousarray(desc, dtype=IMAGE_DESC_DTYPE)
    ok = desc["status"] == MIMO_OK
    cu = np.empty(int(desc["grid_t"][ok].sum()) + 1, dtype=np.int32)
    k = load().mimo_chunk_seqlens(desc.shape[0], desc.ctypes.data, cu.ctypes.data, cu.shape[0])
    if k < 0:
        _check(int(k), "chunk_seqlens")
    return cu[:k + 1]


def fold_patch_weights(w, w_folded=None, stream=None):
    """mimo_fold_patch_weights: bf16 [E, 1536] -> bf16 [E, 768] (device tensors)."""
    import torch
    _check_matrix(w, "fold_patch_weights: w", ROW_LEN, (torch.bfloat16,))
    e = w.shape[0]
    if w_folded is None:
        w_folded = torch.empty((e, ROW_LEN // 2), dtype=torch.bfloat16, device=w.device)
    _check_matrix(w_folded, "fold_patch_weights: w_folded", ROW_LEN // 2, (torch.bfloat16,))
    _require(w_folded.shape[0] == e, "fold_patch_weights: w_folded must have w's row count")
    _check_device([w, w_folded], "fold_patch_weights")
    _check(load().mimo_fold_patch_weights(e, w.data_ptr(), w_folded.data_ptr(),
                                          _stream_handle(stream, w.device)), "fold_patch_weights")
    return w_folded


def patch_embed(rows, w, bias=None, out=None, out_dtype: str = "bf16", stream=None):
    """mimo_patch_embed: rows bf16 [n, 1536] x w bf16 [E, 1536] (or folded
    [E, 768]) -> out [n, E] (+ bias float32 [E])."""
    import torch
    _check_matrix(rows, "patch_embed: rows", ROW_LEN, (torch.bfloat16,))
    _require(w.dim() == 2 and w.shape[1] in (ROW_LEN, ROW_LEN // 2),
             f"patch_embed: w must be [E, 1536] or folded [E, 768], got {tuple(w.shape)}")
    _check_matrix(w, "patch_embed: w", int(w.shape[1]), (torch.bfloat16,))
    n, e = rows.shape[0], w.shape[0]
    folded = int(w.shape[1] == ROW_LEN // 2)
    if bias is not None:
        _require(bias.dim() == 1 and bias.shape[0] == e and bias.dtype == torch.float32
                 and bias.is_contiguous(), f"patch_embed: bias must be contiguous float32 [{e}]")
    if out is None:
        _require(out_dtype in ("f32", "bf16"), f"patch_embed: out_dtype {out_dtype!r} is not f32 or bf16")
        tdtype = {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
        out = torch.empty((n, e), dtype=tdtype, device=rows.device)
    _check_matrix(out, "patch_embed: out", e, (torch.float32, torch.bfloat16))
    _require(out.shape[0] == n, f"patch_embed: out must be [{n}, {e}], got {tuple(out.shape)}")
    _check_device([rows, w, bias, out], "patch_embed")
    code = load().mimo_patch_embed(n, rows.data_ptr(), e, w.data_ptr(), folded,
                                   bias.data_ptr() if bias is not None else None,
                                   _dtype_code(out), out.data_ptr(),
                                   _stream_handle(stream, rows.device))
    _check(code, "patch_embed")
    return out


def hf_smart_resize(h: int, w: int, params: MimoParams | None = None):
    """mimo_hf_smart_resize: the stock Qwen2-VL geometry."""
    oh, ow = ctypes.c_int64(), ctypes.c_int64()
    _check(load().mimo_hf_smart_resize(int(h), int(w), ctypes.byref(params) if params else None,
                                       ctypes.byref(oh), ctypes.byref(ow)), "hf_smart_resize")
    return oh.value, ow.value


def plan_hf(hwc, params: MimoParams | None = None, check: bool = True):
    """mimo_plan_hf over an [n, 3] (height, width, channels) table."""
    hwc = np.ascontiguousarray(np.asarray(hwc, dtype=np.int32).reshape(-1, 3))
    n = hwc.shape[0]
    desc = np.zeros(n, dtype=IMAGE_DESC_DTYPE)
    total_rows, total_src = ctypes.c_int64(), ctypes.c_int64()
    code = load().mimo_plan_hf(n, hwc.ctypes.data, ctypes.byref(params) if params else None,
                               desc.ctypes.data, ctypes.byref(total_rows), ctypes.byref(total_src))
    if check:
        _check(code, "plan_hf")
    return desc, total_rows.value, total_src.value, code


def hf_workspace_bytes(desc: np.ndarray) -> int:
    desc = np.ascontiguousarray(desc, dtype=IMAGE_DESC_DTYPE)
    return int(load().mimo_hf_workspace_bytes(desc.shape[0], desc.ctypes.data))


def preprocess_hf_batch(desc: np.ndarray, src, mean01, std01, rows=None, rows_col=None,
                        workspace=None, stream=None):
    """mimo_preprocess_hf_batch on device tensors (src uint8, rows / rows_col
    float32 or bf16 [capacity, 1536], workspace uint8)."""
    desc = np.ascontiguousarray(desc, dtype=IMAGE_DESC_DTYPE)
    n = desc.shape[0]
    code_dtype, cap = _out_tensors(rows, rows_col, "preprocess_hf_batch")
    out = rows if rows is not None else rows_col
    _check_bytes(src, "preprocess_hf_batch: src")
    _require(workspace is not None, "preprocess_hf_batch: workspace is None")
    _check_bytes(workspace, "preprocess_hf_batch: workspace")
    _check_device([src, rows, rows_col, workspace], "preprocess_hf_batch")
    m = (ctypes.c_float * 3)(*[float(v) for v in mean01])
    s = (ctypes.c_float * 3)(*[float(v) for v in std01])
    code = load().mimo_preprocess_hf_batch(
        n, desc.ctypes.data, src.data_ptr(), src.numel(), m, s, code_dtype,
        rows.data_ptr() if rows is not None else None,
        rows_col.data_ptr() if rows_col is not None else None,
        cap, workspace.data_ptr(), workspace.numel(), _stream_handle(stream, out.device))
    _check(code, "preprocess_hf_batch")


def prepare_pixel_embed(w, mean255, std255, bias=None, w_pixels=None, bias_pixels=None, stream=None):
    """mimo_prepare_pixel_embed: the patch-embedding weight bf16 [E, 1536]
    (and float32 bias [E], or None) -> (w_pixels bf16 [E, 768] in the
    source's (py, px, c) order with the two frames' halves summed and the
    standardisation folded in, bias_pixels float32 [E]) for mimo_pixel_embed
    with these statistics (0-255 units)."""
    import torch
    _check_matrix(w, "prepare_pixel_embed: w", ROW_LEN, (torch.bfloat16,))
    e = w.shape[0]
    if bias is not None:
        _require(bias.dim() == 1 and bias.shape[0] == e and bias.dtype == torch.float32
                 and bias.is_contiguous(), f"prepare_pixel_embed: bias must be contiguous float32 [{e}]")
    if w_pixels is None:
        w_pixels = torch.empty((e, ROW_LEN // 2), dtype=torch.bfloat16, device=w.device)
    if bias_pixels is None:
        bias_pixels = torch.empty(e, dtype=torch.float32, device=w.device)
    _check_matrix(w_pixels, "prepare_pixel_embed: w_pixels", ROW_LEN // 2, (torch.bfloat16,))
    _require(w_pixels.shape[0] == e and bias_pixels.dim() == 1 and bias_pixels.shape[0] == e
             and bias_pixels.dtype == torch.float32 and bias_pixels.is_contiguous(),
             "prepare_pixel_embed: outputs must be bf16 [E, 768] and float32 [E]")
    _check_device([w, bias, w_pixels, bias_pixels], "prepare_pixel_embed")
    m = (ctypes.c_float * 3)(*[float(v) for v in mean255])
    s = (ctypes.c_float * 3)(*[float(v) for v in std255])
    _check(load().mimo_prepare_pixel_embed(e, w.data_ptr(), bias.data_ptr() if bias is not None else None,
                                           m, s, w_pixels.data_ptr(), bias_pixels.data_ptr(),
                                           _stream_handle(stream, w.device)), "prepare_pixel_embed")
    return w_pixels, bias_pixels


def pixel_embed(desc: np.ndarray, src, w_pixels, bias_pixels, out, workspace, stream=None):
    """mimo_pixel_embed: the still images of a plan straight to their patch
    embeddings out [rows, E] (merge-block row order), from the packed uint8
    sources, with weights from prepare_pixel_embed."""
    import torch
    desc = np.ascontiguousarray(desc, dtype=IMAGE_DESC_DTYPE)
    _check_bytes(src, "pixel_embed: src")
    _check_matrix(w_pixels, "pixel_embed: w_pixels", ROW_LEN // 2, (torch.bfloat16,))
    e = w_pixels.shape[0]
    _require(bias_pixels.dim() == 1 and bias_pixels.shape[0] == e and bias_pixels.dtype == torch.float32
             and bias_pixels.is_contiguous(), f"pixel_embed: bias_pixels must be contiguous float32 [{e}]")
    _check_matrix(out, "pixel_embed: out", e, (torch.float32, torch.bfloat16))
    _check_bytes(workspace, "pixel_embed: workspace")
    _check_device([src, w_pixels, bias_pixels, out, workspace], "pixel_embed")
    code = load().mimo_pixel_embed(desc.shape[0], desc.ctypes.data, src.data_ptr(), src.numel(), e,
                                   w_pixels.data_ptr(), bias_pixels.data_ptr(), _dtype_code(out),
                                   out.data_ptr(), out.shape[0], workspace.data_ptr(), workspace.numel(),
                                   _stream_handle(stream, out.device))
    _check(code, "pixel_embed")
