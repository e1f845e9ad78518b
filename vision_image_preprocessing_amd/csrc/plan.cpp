// plan.cpp -- host-side geometry of the MiMo-V2 pixel path: smart_resize,
// the per-image plan of a batch, and the column permutation indices; the
// stock Qwen2-VL geometry of the contrast path.
//
// Pages: NeMo Automodel "mimo_v2_flash.processing" (smart_resize,
// get_number_of_image_patches, MimoV2ImageProcessor defaults, and the module
// docstring on the stock processor) and docs.rs "cortiq_engine::mimo_vision"
// (smart_resize, column_permutation).
#include <algorithm>
#include <cfenv>
#include <cmath>
#include <cstring>
#include <string>

#include "internal.h"

namespace mimo {

namespace {
thread_local std::string g_last_error;
}

int set_error(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

void clear_error() { g_last_error.clear(); }

namespace {

bool params_ok(const mimo_params &p) {
    return p.patch_size > 0 && p.merge_size > 0 && p.temporal_patch_size > 0 &&
           p.reserved0 == 0 && p.min_pixels >= 0 && p.max_pixels > 0 &&
           p.min_pixels <= p.max_pixels && p.max_aspect > 0.0;
}

// Nearest integer with ties to even -- the rounding of Python's round(),
// which the Qwen2-VL smart_resize applies to side / factor.  nearbyint()
// rounds in the current mode, which is round-to-nearest-even by default.
double round_ties_even(double v) {
    const int mode = std::fegetround();
    if (mode != FE_TONEAREST) std::fesetround(FE_TONEAREST);
    const double r = std::nearbyint(v);
    if (mode != FE_TONEAREST) std::fesetround(mode);
    return r;
}

// smart_resize with factor f.  Sides are carried as float64 the way the
// Python routine carries them; a short side below f is first scaled to f
// (the long side by the same ratio, one float64 rounding) and that branch
// skips the aspect guard; a shrink that floors a side to zero is rejected.
int smart_resize_impl(int64_t h, int64_t w, int64_t f, int64_t min_px, int64_t max_px,
                      double max_aspect, int64_t *oh, int64_t *ow) {
    const int64_t lo = std::min(h, w);
    const int64_t hi = std::max(h, w);
    double sh, sw;
    if (lo < f) {
        sh = double(h * f) / double(lo);
        sw = double(w * f) / double(lo);
    } else {
        if (double(hi) / double(lo) > max_aspect) return MIMO_E_ASPECT;
        sh = double(h);
        sw = double(w);
    }
    const double fd = double(f);
    double th = round_ties_even(sh / fd) * fd;
    double tw = round_ties_even(sw / fd) * fd;
    if (th * tw > double(max_px)) {
        const double beta = std::sqrt(sh * sw / double(max_px));
        th = std::floor(sh / beta / fd) * fd;
        tw = std::floor(sw / beta / fd) * fd;
        if (th < fd || tw < fd) return MIMO_E_DEGENERATE;
    } else if (th * tw < double(min_px)) {
        const double beta = std::sqrt(double(min_px) / (sh * sw));
        th = std::ceil(sh * beta / fd) * fd;
        tw = std::ceil(sw * beta / fd) * fd;
    }
    *oh = int64_t(th);
    *ow = int64_t(tw);
    return MIMO_OK;
}

// The stock Qwen2-VL smart_resize: no short-side upscale; each side is
// rounded to the factor; a shrink floors each side and clamps it to at
// least one factor on its own, a grow ceils; the aspect guard always applies.
int stock_smart_resize_impl(int64_t h, int64_t w, int64_t f, int64_t min_px, int64_t max_px,
                            double max_aspect, int64_t *oh, int64_t *ow) {
    const double hd = double(h), wd = double(w), fd = double(f);
    if (std::max(hd, wd) / std::min(hd, wd) > max_aspect) return MIMO_E_ASPECT;
    double th = round_ties_even(hd / fd) * fd;
    double tw = round_ties_even(wd / fd) * fd;
    if (th * tw > double(max_px)) {
        const double beta = std::sqrt(hd * wd / double(max_px));
        th = std::max(fd, std::floor(hd / beta / fd) * fd);
        tw = std::max(fd, std::floor(wd / beta / fd) * fd);
    } else if (th * tw < double(min_px)) {
        const double beta = std::sqrt(double(min_px) / (hd * wd));
        th = std::ceil(hd * beta / fd) * fd;
        tw = std::ceil(wd * beta / fd) * fd;
    }
    *oh = int64_t(th);
    *ow = int64_t(tw);
    return MIMO_OK;
}

}  // namespace
}  // namespace mimo

using namespace mimo;

extern "C" {

int mimo_hf_smart_resize(int64_t h, int64_t w, const mimo_params *params, int64_t *out_h,
                         int64_t *out_w) {
    clear_error();
    mimo_params def;
    mimo_default_params(&def);
    const mimo_params &p = params ? *params : def;
    if (!out_h || !out_w) return set_error(MIMO_E_INVALID, "hf_smart_resize: null output pointer");
    if (!params_ok(p)) return set_error(MIMO_E_INVALID, "hf_smart_resize: invalid parameters");
    if (h < 1 || w < 1) return set_error(MIMO_E_INVALID, "hf_smart_resize: sides must be >= 1");
    if (h > (int64_t(1) << 31) || w > (int64_t(1) << 31))
        return set_error(MIMO_E_TOO_LARGE, "hf_smart_resize: side above 2^31");
    int64_t oh = 0, ow = 0;
    const int st = stock_smart_resize_impl(h, w, int64_t(p.patch_size) * p.merge_size, p.min_pixels,
                                           p.max_pixels, p.max_aspect, &oh, &ow);
    if (st != MIMO_OK)
        return set_error(st, "hf_smart_resize: aspect ratio of " + std::to_string(h) + "x" +
                                 std::to_string(w) + " exceeds max_aspect");
    *out_h = oh;
    *out_w = ow;
    return MIMO_OK;
}

void mimo_default_params(mimo_params *p) {
    if (!p) return;
    std::memset(p, 0, sizeof(*p));
    p->patch_size = 16;
    p->merge_size = 2;
    p->temporal_patch_size = 2;
    p->min_pixels = 8192;
    p->max_pixels = 8388608;
    p->max_aspect = 200.0;
}

int mimo_smart_resize(int64_t h, int64_t w, const mimo_params *params, int64_t *out_h,
                      int64_t *out_w) {
    clear_error();
    mimo_params def;
    mimo_default_params(&def);
    const mimo_params &p = params ? *params : def;
    if (!out_h || !out_w) return set_error(MIMO_E_INVALID, "smart_resize: null output pointer");
    if (!params_ok(p)) return set_error(MIMO_E_INVALID, "smart_resize: invalid parameters");
    if (h < 1 || w < 1)
        return set_error(MIMO_E_INVALID, "smart_resize: sides must be >= 1, got " +
                                             std::to_string(h) + "x" + std::to_string(w));
    const int64_t f = int64_t(p.patch_size) * p.merge_size;
    // keep h*f and h*w exact in int64 / float64
    if (h > (int64_t(1) << 31) || w > (int64_t(1) << 31))
        return set_error(MIMO_E_TOO_LARGE, "smart_resize: side above 2^31");
    int64_t oh = 0, ow = 0;
    const int st = smart_resize_impl(h, w, f, p.min_pixels, p.max_pixels, p.max_aspect, &oh, &ow);
    if (st == MIMO_E_ASPECT)
        return set_error(st, "smart_resize: aspect ratio of " + std::to_string(h) + "x" +
                                 std::to_string(w) + " exceeds max_aspect");
    if (st == MIMO_E_DEGENERATE)
        return set_error(st, "smart_resize: shrinking " + std::to_string(h) + "x" +
                                 std::to_string(w) + " to max_pixels floors a side to zero");
    *out_h = oh;
    *out_w = ow;
    return MIMO_OK;
}

}  // extern "C"

namespace mimo {
namespace {

// Plans n items (still images or videos).  item(i) gives frames, h, w, c;
// ceiling(i) the resized-area ceiling for item i; resize is the geometry
// (smart_resize_impl, or the stock rules of the contrast path).
template <typename Item, typename Ceiling, typename Resize>
int plan_items(int32_t n, Item item, Ceiling ceiling, const mimo_params &p, mimo_image_desc *out,
               int64_t *total_rows, int64_t *total_src_bytes, Resize resize) {
    const int64_t patch = p.patch_size;
    const int64_t merge = p.merge_size;
    const int64_t temporal = p.temporal_patch_size;
    int first_error = MIMO_OK;
    std::string first_msg;
    int64_t src_off = 0, row_off = 0;
    for (int32_t i = 0; i < n; ++i) {
        int32_t f, h, w, c;
        item(i, f, h, w, c);
        mimo_image_desc d;
        std::memset(&d, 0, sizeof(d));
        d.src_h = h;
        d.src_w = w;
        d.channels = c;
        d.frames = f;
        d.src_offset = src_off;
        d.row_offset = row_off;
        const int64_t max_px = ceiling(i);
        int st = MIMO_OK;
        std::string msg;
        if (f < 1 || h < 1 || w < 1 || (c != 3 && c != 4) || max_px < p.min_pixels) {
            st = MIMO_E_INVALID;
            msg = "item " + std::to_string(i) + ": bad shape or pixel ceiling";
        } else if (h > kMaxSide || w > kMaxSide) {
            st = MIMO_E_TOO_LARGE;
            msg = "item " + std::to_string(i) + ": side above 2^23 - 1";
        } else {
            int64_t oh = 0, ow = 0;
            st = resize(h, w, patch * merge, p.min_pixels, max_px, p.max_aspect, &oh, &ow);
            const int64_t grid_t = (f + temporal - 1) / temporal;
            if (st == MIMO_OK && (oh > kMaxSide || ow > kMaxSide ||
                                  grid_t * (oh / patch) * (ow / patch) > kMaxRowsPerImage)) {
                st = MIMO_E_TOO_LARGE;
                msg = "item " + std::to_string(i) + ": resized side above 2^23 - 1 or more than 2^24 rows";
            } else if (st != MIMO_OK) {
                msg = "item " + std::to_string(i) + ": " + mimo_status_string(st);
            } else {
                d.dst_h = int32_t(oh);
                d.dst_w = int32_t(ow);
                d.grid_t = int32_t(grid_t);
                d.grid_h = int32_t(oh / patch);
                d.grid_w = int32_t(ow / patch);
                d.rows = int64_t(d.grid_t) * d.grid_h * d.grid_w;
            }
        }
        d.status = st;
        if (st != MIMO_OK && first_error == MIMO_OK) {
            first_error = st;
            first_msg = msg;
        }
        if (f > 0 && h > 0 && w > 0 && c > 0) src_off += int64_t(f) * h * w * c;
        row_off += d.rows;
        out[i] = d;
    }
    if (total_rows) *total_rows = row_off;
    if (total_src_bytes) *total_src_bytes = src_off;
    if (first_error != MIMO_OK) return set_error(first_error, "plan: " + first_msg);
    return MIMO_OK;
}

}  // namespace
}  // namespace mimo

extern "C" {

int mimo_plan_geometry(int32_t n, const int32_t *hwc, const mimo_params *params,
                       mimo_image_desc *out, int64_t *total_rows, int64_t *total_src_bytes) {
    clear_error();
    if (n < 0 || (n > 0 && (!hwc || !out)))
        return set_error(MIMO_E_INVALID, "plan_geometry: bad n or null pointer");
    mimo_params def;
    mimo_default_params(&def);
    const mimo_params &p = params ? *params : def;
    if (!params_ok(p)) return set_error(MIMO_E_INVALID, "plan_geometry: invalid parameters");
    return plan_items(
        n,
        [&](int32_t i, int32_t &f, int32_t &h, int32_t &w, int32_t &c) {
            f = 1;
            h = hwc[3 * i];
            w = hwc[3 * i + 1];
            c = hwc[3 * i + 2];
        },
        [&](int32_t) { return p.max_pixels; }, p, out, total_rows, total_src_bytes,
        smart_resize_impl);
}

int mimo_plan_hf(int32_t n, const int32_t *hwc, const mimo_params *params, mimo_image_desc *out,
                 int64_t *total_rows, int64_t *total_src_bytes) {
    clear_error();
    if (n < 0 || (n > 0 && (!hwc || !out)))
        return set_error(MIMO_E_INVALID, "plan_hf: bad n or null pointer");
    mimo_params def;
    mimo_default_params(&def);
    const mimo_params &p = params ? *params : def;
    if (!params_ok(p)) return set_error(MIMO_E_INVALID, "plan_hf: invalid parameters");
    return plan_items(
        n,
        [&](int32_t i, int32_t &f, int32_t &h, int32_t &w, int32_t &c) {
            f = 1;
            h = hwc[3 * i];
            w = hwc[3 * i + 1];
            c = hwc[3 * i + 2];
        },
        [&](int32_t) { return p.max_pixels; }, p, out, total_rows, total_src_bytes,
        stock_smart_resize_impl);
}

int mimo_plan_frames(int32_t n, const int32_t *fhwc, const int64_t *max_pixels,
                     const mimo_params *params, mimo_image_desc *out, int64_t *total_rows,
                     int64_t *total_src_bytes) {
    clear_error();
    if (n < 0 || (n > 0 && (!fhwc || !out)))
        return set_error(MIMO_E_INVALID, "plan_frames: bad n or null pointer");
    mimo_params def;
    mimo_default_params(&def);
    const mimo_params &p = params ? *params : def;
    if (!params_ok(p)) return set_error(MIMO_E_INVALID, "plan_frames: invalid parameters");
    return plan_items(
        n,
        [&](int32_t i, int32_t &f, int32_t &h, int32_t &w, int32_t &c) {
            f = fhwc[4 * i];
            h = fhwc[4 * i + 1];
            w = fhwc[4 * i + 2];
            c = fhwc[4 * i + 3];
        },
        [&](int32_t i) {
            return (max_pixels && max_pixels[i] > 0) ? max_pixels[i] : p.max_pixels;
        },
        p, out, total_rows, total_src_bytes, smart_resize_impl);
}

int64_t mimo_video_max_pixels(int64_t n_sampled, int64_t total_max, const mimo_params *params) {
    clear_error();
    mimo_params def;
    mimo_default_params(&def);
    const mimo_params &p = params ? *params : def;
    if (n_sampled < 1 || total_max < 0 || !params_ok(p))
        return set_error(MIMO_E_INVALID, "video_max_pixels: n_sampled >= 1, total_max >= 0");
    // floor division of non-negative values
    const int64_t share = total_max * p.temporal_patch_size / n_sampled;
    return std::max(p.min_pixels, std::min(share, p.max_pixels));
}

int64_t mimo_smart_nframes(int64_t total, double fps_src, double fps, int64_t min_frames,
                           int64_t max_frames) {
    clear_error();
    if (total < 1 || !(fps_src > 0.0) || !(fps > 0.0) || min_frames > max_frames)
        return set_error(MIMO_E_INVALID, "smart_nframes: bad arguments");
    const double want = double(total) / fps_src * fps;
    const double clamped = std::min(std::min(std::max(want, double(min_frames)), double(max_frames)),
                                    double(total));
    return int64_t(std::floor(clamped / 2.0)) * 2;
}

int64_t mimo_sample_frames(int64_t total, int64_t n, double fps_src, int64_t *idx, float *ts) {
    clear_error();
    if (total < 1 || n < 1 || !(fps_src > 0.0) || !idx || !ts)
        return set_error(MIMO_E_INVALID, "sample_frames: bad arguments");
    // linspace(0, total - 1, n) as numpy evaluates it: i * step + 0, last = stop
    const double stop = double(total - 1);
    const double step = n > 1 ? stop / double(n - 1) : 0.0;
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i) {
        const double v = (n > 1 && i == n - 1) ? stop : double(i) * step;
        const int64_t j = int64_t(v);
        if (k == 0 || idx[k - 1] != j) idx[k++] = j;
    }
    const float rate = float(fps_src);
    for (int64_t i = 0; i < k; ++i) ts[i] = float(idx[i]) / rate;
    return k;
}

size_t mimo_workspace_bytes(int32_t n) { return n < 0 ? 0 : ws_total_bytes(n); }

int mimo_stats255(const double *mean01, const double *std01, float *mean255, float *std255) {
    clear_error();
    if (!mean01 || !std01 || !mean255 || !std255)
        return set_error(MIMO_E_INVALID, "stats255: null pointer");
    for (int c = 0; c < 3; ++c)
        if (!std::isfinite(mean01[c]) || !std::isfinite(std01[c]) || !(std01[c] > 0.0))
            return set_error(MIMO_E_INVALID, "stats255: statistics must be finite with std > 0");
    // the processor's statistics scaled to 0-255 units: the product formed in
    // float64, then rounded once to float32
    for (int c = 0; c < 3; ++c) {
        mean255[c] = float(255.0 * mean01[c]);
        std255[c] = float(255.0 * std01[c]);
    }
    return MIMO_OK;
}

int mimo_column_permutation(int64_t grid_t, int64_t grid_h, int64_t grid_w, int64_t merge,
                            int64_t *perm) {
    clear_error();
    if (grid_t < 1 || grid_h < 1 || grid_w < 1 || merge < 1 || !perm || grid_h % merge ||
        grid_w % merge)
        return set_error(MIMO_E_INVALID, "column_permutation: bad grid or null output");
    const int64_t bh = grid_h / merge, bw = grid_w / merge, unit = merge * merge;
    // destination unit j of frame t is (block col, block row) = divmod(j, bh);
    // its source unit is block row * bw + block col of the same frame.
    for (int64_t t = 0; t < grid_t; ++t) {
        const int64_t frame = t * bh * bw;
        for (int64_t j = 0; j < bh * bw; ++j) {
            const int64_t bc = j / bh, br = j % bh;
            const int64_t src_unit = frame + br * bw + bc;
            int64_t *dst = perm + (frame + j) * unit;
            for (int64_t k = 0; k < unit; ++k) dst[k] = src_unit * unit + k;
        }
    }
    return MIMO_OK;
}

int mimo_rope_inv_freq(int32_t rope_dim, double theta, float *inv) {
    clear_error();
    if (rope_dim < 2 || rope_dim > MIMO_ROPE_DIM_MAX || rope_dim % 2 || !(theta > 1.0) || !inv)
        return set_error(MIMO_E_INVALID, "rope_inv_freq: rope_dim must be even in [2, 256], theta > 1");
    // theta ** (arange(0, dim, 2) / dim) and its reciprocal, each rounded to
    // float32; the float64 power is within a tiny fraction of a float32 ulp.
    for (int32_t i = 0; i < rope_dim / 2; ++i) {
        const float exponent = float(2 * i) / float(rope_dim);
        const float power = float(std::pow(theta, double(exponent)));
        inv[i] = 1.0f / power;
    }
    return MIMO_OK;
}

int64_t mimo_chunk_seqlens(int32_t n, const mimo_image_desc *desc, int32_t *cu, int64_t capacity) {
    clear_error();
    if (n < 0 || (n > 0 && !desc) || !cu || capacity < 1)
        return set_error(MIMO_E_INVALID, "chunk_seqlens: bad n or null pointer");
    int64_t k = 0, acc = 0;
    cu[0] = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mimo_image_desc &d = desc[i];
        if (d.status != MIMO_OK || d.rows == 0) continue;
        if (d.grid_t < 1 || d.grid_h < 1 || d.grid_w < 1)
            return set_error(MIMO_E_INVALID, "chunk_seqlens: item " + std::to_string(i) + " has a bad grid");
        for (int32_t t = 0; t < d.grid_t; ++t) {
            if (k + 2 > capacity)
                return set_error(MIMO_E_CAPACITY, "chunk_seqlens: cu holds fewer than sum(grid_t) + 1 entries");
            acc += int64_t(d.grid_h) * d.grid_w;
            if (acc > 0x7FFFFFFFll)
                return set_error(MIMO_E_TOO_LARGE, "chunk_seqlens: a boundary exceeds 2^31 - 1");
            cu[++k] = int32_t(acc);
        }
    }
    return k;
}

const char *mimo_status_string(int status) {
    switch (status) {
        case MIMO_OK: return "ok";
        case MIMO_E_INVALID: return "invalid argument";
        case MIMO_E_ASPECT: return "aspect ratio above max_aspect";
        case MIMO_E_DEGENERATE: return "degenerate shrink (a side floors to zero)";
        case MIMO_E_UNSUPPORTED: return "unsupported parameters";
        case MIMO_E_CAPACITY: return "buffer too small";
        case MIMO_E_HIP: return "HIP runtime error";
        case MIMO_E_TOO_LARGE: return "size above the library's index limits";
        default: return "unknown status";
    }
}

const char *mimo_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
