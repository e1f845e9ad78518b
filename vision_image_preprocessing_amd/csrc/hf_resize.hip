// hf_resize.hip -- the stock-HF contrast path for AMD Instinct MI355X
// (gfx950): the pixels the stock Qwen2-VL processor would give, so a caller
// can measure or reproduce the shift the MiMo path avoids.
//
// What is computed (NeMo Automodel "mimo_v2_flash.processing", module
// docstring, on the stock processor): alpha dropped (RGB bytes kept), a PIL
// antialiased bicubic resize that returns bytes, a 0-1 rescale and a
// float32 normalisation, then the same rows as the MiMo path (two identical
// frames, (c, tt, py, px), merge-block or column order).
//
// Resize arithmetic, as PIL's 8-bit resampler does it: for each resampled
// axis, output i takes inputs [first, first + count) weighted by Keys' cubic
// (a = -0.5) widened by max(n_in / n_out, 1) and normalised; weights are
// rounded to 22 fractional bits; a pass sums bytes x weights in int32 and
// rounds back to a byte, (acc + 2^21) >> 22 clamped to [0, 255].  The
// horizontal pass runs first (only if the width changes), then the vertical
// one (only if the height changes).  The host computes the taps (float64,
// like PIL) and a 256-entry table per channel of the rescale and
// normalisation (float32(float64(v) / 255) then (x - mean) / std in
// float32); so the kernel is integer up to that lookup and its results are
// bit-exact.
//
// Kernel: one workgroup per merge unit (32 x 32 output pixels), in groups
// of output rows sized so that the band of source rows their vertical taps
// need fits LDS.  Per group: the source block the tile's taps touch is
// staged into LDS (one dword per pixel, RGB bytes; aligned dword buffer
// loads realigned with v_alignbyte, in row chunks that fit), the horizontal
// pass reads it from there into the band, the vertical pass turns the band
// into a 32 x 32 byte block; then the unit's 4 rows (both temporal slots)
// go out with 16-byte stores, to merge-block and/or column order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "device_util.h"
#include "internal.h"
#include "runtime.h"

namespace mimo {
namespace {

constexpr int kHfThreads = 512;
constexpr int kWeightBits = 22;           // fractional bits of the resampler's weights
constexpr int kMidRows = 256;             // LDS band rows (32 pixels each)
constexpr int kStageDwords = 4096;        // LDS source staging (one dword per pixel)
constexpr int kTapBudget = 2048;          // LDS weights per axis (else they are read from memory)
constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource word 3 (gfx9 family)

// Per-item record of the contrast kernel (64 bytes).
struct HfItem {
    int64_t src_offset;   // bytes into the packed sources
    int64_t row_offset;   // first output row
    int64_t x_tab;        // int32 offset of the column taps (first, count, weights), or -1
    int64_t y_tab;        // int32 offset of the row taps, or -1
    int32_t src_h, src_w;
    int32_t channels;     // 3 or 4 (alpha ignored)
    int32_t blocks_h, blocks_w;
    int32_t kx, ky;       // weights per output column / row
    int32_t group;        // output rows per vertical group (divides 32)
};
static_assert(sizeof(HfItem) == 64, "HfItem must stay 64 bytes");

struct HfArgs {
    const uint8_t *src;
    int64_t src_end;            // bytes readable from src
    const HfItem *items;
    const int64_t *tile_begin;  // [n + 1]
    const float *lut;           // [3][256]
    const int32_t *taps;
    void *rows;                 // merge-block order, nullable
    void *rows_col;             // column order, nullable
    int32_t n;
};

// workspace: [HfItem x n][int64 tile_begin x (n+1)][float lut x 768][int32 taps]
size_t hf_items_bytes(int32_t n) { return align256(sizeof(HfItem) * size_t(n)); }
size_t hf_prefix_bytes(int32_t n) { return align256(sizeof(int64_t) * (size_t(n) + 1)); }
constexpr size_t kLutBytes = 3 * 256 * sizeof(float);

__device__ __forceinline__ uint32_t round_clip_byte(int32_t acc) {
    const int32_t v = (acc + (1 << (kWeightBits - 1))) >> kWeightBits;
    return uint32_t(v < 0 ? 0 : (v > 255 ? 255 : v));
}

// A raw buffer resource over [base & ~3, src_end): reads past the end
// return zero.  `lead` is base's offset inside it.
struct SrcWindow {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t lead;
};

__device__ __forceinline__ SrcWindow src_window(const HfArgs &a, uint64_t base) {
    const uint64_t start = base & ~uint64_t(3);
    const uint64_t end = reinterpret_cast<uint64_t>(a.src) + uint64_t(a.src_end);
    const uint64_t avail = end > start ? end - start : 0;
    SrcWindow w;
    w.rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(start), 0,
                                               avail > 0x7FFFFFF0ull ? 0x7FFFFFF0 : int(avail),
                                               kBufferWord3);
    w.lead = uint32_t(base - start);
    return w;
}

// RGB bytes of the pixel at byte offset `off` of the window (any alignment).
__device__ __forceinline__ uint32_t load_rgb(const SrcWindow &w, uint32_t off) {
    const uint32_t al = off & ~3u, sh = off & 3u;
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(w.rsrc, int(al), 0, 0);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(w.rsrc, int(al) + 4, 0, 0);
    return __builtin_amdgcn_alignbyte(hi, lo, sh) & 0x00FFFFFFu;
}

// One output value of the tile in the final layout: 4 floats (4 pixels of
// one patch row, one channel) into both temporal slots.
template <typename OutT>
__device__ __forceinline__ void store_pair(OutT *row_ptr, const float (&v)[4]);

template <>
__device__ __forceinline__ void store_pair<float>(float *p, const float (&v)[4]) {
    const f32x4 q = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(q, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store(q, reinterpret_cast<f32x4 *>(p + kPlane));
}

template <>
__device__ __forceinline__ void store_pair<uint16_t>(uint16_t *p, const float (&v)[4]) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = {__bf16(v[0]), __bf16(v[1])}, b = {__bf16(v[2]), __bf16(v[3])};
    const u32x2 q = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
    __builtin_nontemporal_store(q, reinterpret_cast<u32x2 *>(p));
    __builtin_nontemporal_store(q, reinterpret_cast<u32x2 *>(p + kPlane));
}

template <typename OutT>
__global__ __launch_bounds__(kHfThreads) void hf_preprocess_kernel(HfArgs a) {
    __shared__ float lut[3 * 256];
    __shared__ uint32_t block[kUnitPx * kUnitPx];  // the unit's output bytes (RGB per dword)
    __shared__ uint32_t mid[kMidRows * kUnitPx];   // horizontal-pass band
    __shared__ uint32_t stage[kStageDwords];       // source pixels of the current row chunk
    // the tile's taps: first (relative to the staged block / band), count, weights
    __shared__ int32_t xfirst_s[kUnitPx], xcount_s[kUnitPx], xw_s[kTapBudget];
    __shared__ int32_t yfirst_s[kUnitPx], ycount_s[kUnitPx], yw_s[kTapBudget];
    const int64_t tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    const int img = find_segment(a.tile_begin, a.n, tile);
    const HfItem d = a.items[img];
    const int local = int(tile - a.tile_begin[img]);
    const int br = div_small(local, d.blocks_w, 1.0f / float(d.blocks_w));
    const int bc = local - br * d.blocks_w;
    const int oy0 = br * kUnitPx, ox0 = bc * kUnitPx;
    const int tid = threadIdx.x;
    for (int i = tid; i < 3 * 256; i += kHfThreads) lut[i] = a.lut[i];

    const uint8_t *img_src = a.src + d.src_offset;
    const int64_t row_bytes = int64_t(d.src_w) * d.channels;
    const int dst_w = d.blocks_w * kUnitPx, dst_h = d.blocks_h * kUnitPx;
    const int32_t *xf = d.kx ? a.taps + d.x_tab : nullptr;  // first[dst_w], count[dst_w], w[dst_w][kx]
    const int32_t *yf = d.ky ? a.taps + d.y_tab : nullptr;
    const int G = d.group;
    // source columns the tile's 32 output columns read, and their taps in LDS
    // (the weights too, when they fit; else they are read from memory)
    const int xlo = xf ? xf[ox0] : ox0;
    const int xhi = xf ? xf[ox0 + kUnitPx - 1] + xf[dst_w + ox0 + kUnitPx - 1] : ox0 + kUnitPx;
    const int ncols = xhi - xlo;  // <= kStageDwords (the host checked)
    const bool xw_in_lds = xf && kUnitPx * d.kx <= kTapBudget;
    if (xf) {
        for (int i = tid; i < kUnitPx; i += kHfThreads) {
            xfirst_s[i] = xf[ox0 + i] - xlo;
            xcount_s[i] = xf[dst_w + ox0 + i];
        }
        if (xw_in_lds)
            for (int i = tid; i < kUnitPx * d.kx; i += kHfThreads)
                xw_s[i] = xf[2 * dst_w + int64_t(ox0) * d.kx + i];
    }
    const bool yw_in_lds = yf && G * d.ky <= kTapBudget;
    for (int g0 = 0; g0 < kUnitPx; g0 += G) {
        const int oy_a = oy0 + g0, oy_b = oy_a + G - 1;
        const int ylo = yf ? yf[oy_a] : oy_a;
        const int yhi = yf ? yf[oy_b] + yf[dst_h + oy_b] : oy_b + 1;
        const int nrows = yhi - ylo;  // <= kMidRows (the host sized G)
        if (yf) {
            for (int i = tid; i < G; i += kHfThreads) {
                yfirst_s[i] = yf[oy_a + i] - ylo;
                ycount_s[i] = yf[dst_h + oy_a + i];
            }
            if (yw_in_lds)
                for (int i = tid; i < G * d.ky; i += kHfThreads)
                    yw_s[i] = yf[2 * dst_h + int64_t(oy_a) * d.ky + i];
        }
        const int chunk = min(nrows, kStageDwords / ncols);
        const float inv_ncols = 1.0f / float(ncols);
        for (int r0 = 0; r0 < nrows; r0 += chunk) {
            const int nr = min(chunk, nrows - r0);
            // stage source rows [ylo + r0, ylo + r0 + nr) x [xlo, xhi)
            const SrcWindow win = src_window(a, reinterpret_cast<uint64_t>(img_src) +
                                                    uint64_t(int64_t(ylo + r0) * row_bytes +
                                                             int64_t(xlo) * d.channels));
            for (int idx = tid; idx < nr * ncols; idx += kHfThreads) {
                const int r = div_small(idx, ncols, inv_ncols);
                const int c = idx - r * ncols;
                stage[idx] = load_rgb(win, win.lead + uint32_t(int64_t(r) * row_bytes + c * d.channels));
            }
            __syncthreads();
            // horizontal pass (or a copy) into band rows [r0, r0 + nr)
            for (int idx = tid; idx < nr * kUnitPx; idx += kHfThreads) {
                const int r = idx >> 5, x = idx & 31;
                const uint32_t *line = &stage[r * ncols];
                uint32_t px;
                if (xf) {
                    const int first = xfirst_s[x], count = xcount_s[x];
                    const int32_t *w = xw_in_lds ? &xw_s[x * d.kx]
                                                 : xf + 2 * dst_w + int64_t(ox0 + x) * d.kx;
                    int32_t acc0 = 0, acc1 = 0, acc2 = 0;
                    for (int j = 0; j < count; ++j) {
                        const uint32_t p = line[first + j];
                        acc0 += int32_t(p & 255u) * w[j];
                        acc1 += int32_t((p >> 8) & 255u) * w[j];
                        acc2 += int32_t((p >> 16) & 255u) * w[j];
                    }
                    px = round_clip_byte(acc0) | (round_clip_byte(acc1) << 8) | (round_clip_byte(acc2) << 16);
                } else {
                    px = line[x];
                }
                mid[(r0 + r) * kUnitPx + x] = px;
            }
            __syncthreads();
        }
        // vertical pass (or a copy) for output rows [oy_a, oy_b]
        for (int idx = tid; idx < G * kUnitPx; idx += kHfThreads) {
            const int r = idx >> 5, x = idx & 31;
            const int oy = oy_a + r;
            uint32_t px;
            if (yf) {
                const int first = yfirst_s[r], count = ycount_s[r];
                const int32_t *w = yw_in_lds ? &yw_s[r * d.ky] : yf + 2 * dst_h + int64_t(oy) * d.ky;
                int32_t acc0 = 0, acc1 = 0, acc2 = 0;
                for (int j = 0; j < count; ++j) {
                    const uint32_t p = mid[(first + j) * kUnitPx + x];
                    acc0 += int32_t(p & 255u) * w[j];
                    acc1 += int32_t((p >> 8) & 255u) * w[j];
                    acc2 += int32_t((p >> 16) & 255u) * w[j];
                }
                px = round_clip_byte(acc0) | (round_clip_byte(acc1) << 8) | (round_clip_byte(acc2) << 16);
            } else {
                px = mid[idx];
            }
            block[(g0 + r) * kUnitPx + x] = px;
        }
        __syncthreads();
    }

    // 4 rows x 3 channels x 16 patch rows x 4 quads of 4 pixels; each thread
    // stores one quad into both temporal slots
    for (int idx = tid; idx < kRowsPerUnit * 3 * kPatch * 4; idx += kHfThreads) {
        const int q = idx / (3 * kPatch * 4);
        const int rem = idx - q * (3 * kPatch * 4);
        const int c = rem / (kPatch * 4);
        const int py = (rem >> 2) & (kPatch - 1);
        const int qd = rem & 3;
        const int mh = q >> 1, mw = q & 1;
        const uint32_t *src_px = &block[(mh * kPatch + py) * kUnitPx + mw * kPatch + qd * 4];
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = lut[c * 256 + ((src_px[j] >> (8 * c)) & 255u)];
        const int64_t elem = int64_t(c) * (kTemporal * kPlane) + py * kPatch + qd * 4;
        if (a.rows) {
            const int64_t row = d.row_offset + int64_t(br * d.blocks_w + bc) * kRowsPerUnit + q;
            store_pair<OutT>(static_cast<OutT *>(a.rows) + row * kRowLen + elem, v);
        }
        if (a.rows_col) {
            const int64_t row = d.row_offset + int64_t(bc * d.blocks_h + br) * kRowsPerUnit + q;
            store_pair<OutT>(static_cast<OutT *>(a.rows_col) + row * kRowLen + elem, v);
        }
    }
}

// ----------------------------------------------------------------- host side

// Keys' cubic convolution kernel, a = -0.5.
double keys_bicubic(double x) {
    const double a = -0.5;
    x = std::fabs(x);
    if (x < 1.0) return ((a + 2.0) * x - (a + 3.0)) * x * x + 1.0;
    if (x < 2.0) return (((x - 5.0) * x + 8.0) * x - 4.0) * a;
    return 0.0;
}

int axis_taps_per_output(int64_t n_in, int64_t n_out) {
    const double scale = double(n_in) / double(n_out);
    const double support = 2.0 * (scale < 1.0 ? 1.0 : scale);
    return int(std::ceil(support)) * 2 + 1;
}

// Appends first[n_out], count[n_out], weights[n_out][k] of one axis.
void append_axis_taps(int64_t n_in, int64_t n_out, std::vector<int32_t> &tab) {
    const double scale = double(n_in) / double(n_out);
    const double widen = scale < 1.0 ? 1.0 : scale;
    const double support = 2.0 * widen;
    const int k = axis_taps_per_output(n_in, n_out);
    const size_t base = tab.size();
    tab.resize(base + size_t(n_out) * (2 + k), 0);
    int32_t *first = tab.data() + base;
    int32_t *count = first + n_out;
    int32_t *weight = count + n_out;
    std::vector<double> w(size_t(k) + 1);
    for (int64_t i = 0; i < n_out; ++i) {
        const double centre = (double(i) + 0.5) * scale;
        int64_t lo = int64_t(centre - support + 0.5);
        if (lo < 0) lo = 0;
        int64_t hi = int64_t(centre + support + 0.5);
        if (hi > n_in) hi = n_in;
        const int64_t cnt = hi - lo;
        double sum = 0.0;
        for (int64_t j = 0; j < cnt; ++j) {
            w[j] = keys_bicubic((double(j + lo) - centre + 0.5) / widen);
            sum += w[j];
        }
        for (int64_t j = 0; j < cnt; ++j) {
            const double v = sum != 0.0 ? w[j] / sum : w[j];
            const double fixed = v * double(1 << kWeightBits);
            weight[i * k + j] = int32_t(v < 0.0 ? fixed - 0.5 : fixed + 0.5);
        }
        first[i] = int32_t(lo);
        count[i] = int32_t(cnt);
    }
}

struct HfTables {
    std::vector<uint8_t> head;    // items, tile prefix, lut
    std::vector<int32_t> taps;
    int64_t tiles = 0;
    int64_t rows = 0;
};

// Output rows per vertical group so that the band of source rows one group
// needs fits kMidRows: the largest of 32, 16, ..., 1 that fits everywhere.
int choose_group(const int32_t *yfirst, const int32_t *ycount, int dst_h) {
    for (int g = kUnitPx; g >= 1; g >>= 1) {
        bool fits = true;
        for (int y0 = 0; y0 < dst_h && fits; y0 += g) {
            const int y1 = y0 + g - 1;
            fits = yfirst[y1] + ycount[y1] - yfirst[y0] <= kMidRows;
        }
        if (fits) return g;
    }
    return 0;
}

int build_hf_tables(int32_t n, const mimo_image_desc *desc, const float *mean01,
                    const float *std01, HfTables &out) {
    out.head.assign(hf_items_bytes(n) + hf_prefix_bytes(n) + align256(kLutBytes), 0);
    HfItem *items = reinterpret_cast<HfItem *>(out.head.data());
    int64_t *tile_begin = reinterpret_cast<int64_t *>(out.head.data() + hf_items_bytes(n));
    float *lut = reinterpret_cast<float *>(out.head.data() + hf_items_bytes(n) + hf_prefix_bytes(n));
    // rescale as float32(float64(v) * (1 / 255)), then (x - mean) / std in float32
    const double rescale = 1.0 / 255.0;
    for (int c = 0; c < 3; ++c)
        for (int v = 0; v < 256; ++v) {
            const float x = float(double(v) * rescale);
            lut[c * 256 + v] = (x - mean01[c]) / std01[c];
        }
    int64_t tiles = 0, rows = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mimo_image_desc &s = desc[i];
        HfItem d;
        std::memset(&d, 0, sizeof(d));
        d.x_tab = d.y_tab = -1;
        tile_begin[i] = tiles;
        d.src_offset = s.src_offset;
        d.row_offset = rows;
        d.blocks_w = 1;
        if (s.status != MIMO_OK || s.rows == 0) {
            items[i] = d;
            continue;
        }
        if (s.src_h < 1 || s.src_w < 1 || (s.channels != 3 && s.channels != 4) || s.frames != 1 ||
            s.dst_h < kUnitPx || s.dst_w < kUnitPx || s.dst_h % kUnitPx || s.dst_w % kUnitPx ||
            s.grid_t != 1 || s.grid_h * kPatch != s.dst_h || s.grid_w * kPatch != s.dst_w ||
            s.rows != int64_t(s.grid_h) * s.grid_w || s.row_offset != rows || s.src_offset < 0)
            return set_error(MIMO_E_INVALID, "preprocess_hf: descriptor " + std::to_string(i) +
                                                 " is not a still-image plan of the 16/2/2 kernels");
        // the staging window addresses up to kMidRows source rows with 32-bit offsets
        if (s.src_h > kMaxSide || s.src_w > kMaxSide || s.dst_h > kMaxSide || s.dst_w > kMaxSide ||
            int64_t(s.src_w) * s.channels * (kMidRows + 1) >= 0x7FFFFFF0ll)
            return set_error(MIMO_E_TOO_LARGE, "preprocess_hf: descriptor " + std::to_string(i) + ": side too large");
        d.src_h = s.src_h;
        d.src_w = s.src_w;
        d.channels = s.channels;
        d.blocks_h = s.dst_h / kUnitPx;
        d.blocks_w = s.dst_w / kUnitPx;
        d.group = kUnitPx;
        if (s.dst_w != s.src_w) {
            d.kx = axis_taps_per_output(s.src_w, s.dst_w);
            d.x_tab = int64_t(out.taps.size());
            append_axis_taps(s.src_w, s.dst_w, out.taps);
        }
        if (s.dst_h != s.src_h) {
            d.ky = axis_taps_per_output(s.src_h, s.dst_h);
            d.y_tab = int64_t(out.taps.size());
            append_axis_taps(s.src_h, s.dst_h, out.taps);
            const int32_t *yfirst = out.taps.data() + d.y_tab;
            d.group = choose_group(yfirst, yfirst + s.dst_h, s.dst_h);
            if (d.group == 0)
                return set_error(MIMO_E_UNSUPPORTED, "preprocess_hf: descriptor " + std::to_string(i) +
                                                         ": vertical downscale beyond the kernel's band");
        }
        if (d.kx) {
            // the widest source block one tile's 32 output columns read
            const int32_t *xfirst = out.taps.data() + d.x_tab;
            const int32_t *xcount = xfirst + s.dst_w;
            for (int32_t x0 = 0; x0 < s.dst_w; x0 += kUnitPx) {
                const int32_t x1 = x0 + kUnitPx - 1;
                if (xfirst[x1] + xcount[x1] - xfirst[x0] > kStageDwords)
                    return set_error(MIMO_E_UNSUPPORTED, "preprocess_hf: descriptor " + std::to_string(i) +
                                                             ": horizontal downscale beyond the kernel's staging");
            }
        }
        items[i] = d;
        tiles += int64_t(d.blocks_h) * d.blocks_w;
        rows += s.rows;
    }
    tile_begin[n] = tiles;
    out.tiles = tiles;
    out.rows = rows;
    if (out.taps.size() > size_t(0x7FFFFFFF))
        return set_error(MIMO_E_TOO_LARGE, "preprocess_hf: tap tables above 2^31 entries");
    return MIMO_OK;
}

}  // namespace
}  // namespace mimo

using namespace mimo;

extern "C" {

size_t mimo_hf_workspace_bytes(int32_t n, const mimo_image_desc *desc) {
    if (n < 0 || (n > 0 && !desc)) return 0;
    size_t entries = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mimo_image_desc &s = desc[i];
        if (s.status != MIMO_OK || s.rows == 0 || s.dst_w < 1 || s.dst_h < 1) continue;
        if (s.dst_w != s.src_w)
            entries += size_t(s.dst_w) * (2 + axis_taps_per_output(s.src_w, s.dst_w));
        if (s.dst_h != s.src_h)
            entries += size_t(s.dst_h) * (2 + axis_taps_per_output(s.src_h, s.dst_h));
    }
    return hf_items_bytes(n) + hf_prefix_bytes(n) + align256(kLutBytes) +
           align256(std::max<size_t>(entries, 1) * sizeof(int32_t));
}

int mimo_preprocess_hf_batch(int32_t n, const mimo_image_desc *desc, const uint8_t *src,
                             int64_t src_capacity, const float *mean01, const float *std01,
                             int32_t out_dtype, void *rows, void *rows_col, int64_t capacity_rows,
                             void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    if (n < 0 || (n > 0 && !desc) || !mean01 || !std01)
        return set_error(MIMO_E_INVALID, "preprocess_hf: bad n or null pointer");
    if (out_dtype != MIMO_F32 && out_dtype != MIMO_BF16)
        return set_error(MIMO_E_INVALID, "preprocess_hf: out_dtype must be MIMO_F32 or MIMO_BF16");
    if (!rows && !rows_col)
        return set_error(MIMO_E_INVALID, "preprocess_hf: both outputs are null");
    if ((rows && !check_ptr_align(rows, 16)) || (rows_col && !check_ptr_align(rows_col, 16)))
        return set_error(MIMO_E_INVALID, "preprocess_hf: outputs must be 16-byte aligned");
    for (int c = 0; c < 3; ++c)
        if (!(std01[c] > 0.0f) || !std::isfinite(std01[c]) || !std::isfinite(mean01[c]))
            return set_error(MIMO_E_INVALID, "preprocess_hf: std01 must be > 0 and finite");
    if (n == 0) return MIMO_OK;
    if (!src) return set_error(MIMO_E_INVALID, "preprocess_hf: null src");
    if (!workspace || !check_ptr_align(workspace, 16))
        return set_error(MIMO_E_INVALID, "preprocess_hf: workspace must be non-null and 16-byte aligned");
    HfTables t;
    int st = build_hf_tables(n, desc, mean01, std01, t);
    if (st != MIMO_OK) return st;
    const size_t need = t.head.size() + align256(std::max<size_t>(t.taps.size(), 1) * sizeof(int32_t));
    if (workspace_bytes < need)
        return set_error(MIMO_E_CAPACITY, "preprocess_hf: workspace smaller than mimo_hf_workspace_bytes(n, desc)");
    int64_t src_needed = 0;
    for (int32_t i = 0; i < n; ++i)
        if (desc[i].status == MIMO_OK && desc[i].rows > 0)
            src_needed = std::max<int64_t>(src_needed, desc[i].src_offset + int64_t(desc[i].src_h) *
                                                                                 desc[i].src_w * desc[i].channels);
    if (src_capacity < src_needed)
        return set_error(MIMO_E_CAPACITY, "preprocess_hf: src_capacity below the packed size");
    if (t.rows > capacity_rows)
        return set_error(MIMO_E_CAPACITY, "preprocess_hf: capacity_rows below the plan's total rows");
    if (t.tiles == 0) return MIMO_OK;
    if (t.tiles > 0x7FFFFFFFll)
        return set_error(MIMO_E_TOO_LARGE, "preprocess_hf: more than 2^31 - 1 tiles");

    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    hipError_t e = upload_table(t.head.data(), t.head.size(), ws, s);
    if (e == hipSuccess && !t.taps.empty())
        e = upload_table(t.taps.data(), t.taps.size() * sizeof(int32_t), ws + t.head.size(), s);
    if (e != hipSuccess) return hip_error(e, "preprocess_hf: table upload");
    HfArgs a;
    a.src = src;
    a.src_end = src_capacity;
    a.items = reinterpret_cast<const HfItem *>(ws);
    a.tile_begin = reinterpret_cast<const int64_t *>(ws + hf_items_bytes(n));
    a.lut = reinterpret_cast<const float *>(ws + hf_items_bytes(n) + hf_prefix_bytes(n));
    a.taps = reinterpret_cast<const int32_t *>(ws + t.head.size());
    a.rows = rows;
    a.rows_col = rows_col;
    a.n = n;
    const dim3 grid{unsigned(t.tiles), 1, 1}, block{unsigned(kHfThreads), 1, 1};
    e = timed_launch(s, [&] {
        if (out_dtype == MIMO_F32)
            hipLaunchKernelGGL(hf_preprocess_kernel<float>, grid, block, 0, s, a);
        else
            hipLaunchKernelGGL(hf_preprocess_kernel<uint16_t>, grid, block, 0, s, a);
    });
    if (e != hipSuccess) return hip_error(e, "preprocess_hf: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

}  // extern "C"
