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
// Kernel: one workgroup per merge unit (32 x 32 output pixels).  A unit
// that neither axis resizes reads its source pixels straight into the
// output block.  Otherwise it works in groups of output rows sized so that
// the band of source rows their vertical taps need fits LDS.  Per group:
// the source block the tile's taps touch is staged into LDS (one dword per
// pixel, RGB bytes; 4 pixels per load, realigned with v_alignbyte, in row
// chunks that fit), the horizontal pass reads it from there into the band,
// the vertical pass turns the band into a 32 x 32 byte block; then the
// unit's 4 rows (both temporal slots) go out with 16-byte stores, to
// merge-block and/or column order.  The LDS is dynamic, sized by the host
// for the batch's widest band, staging and tap tables, so that batches of
// mild resizes keep several workgroups on each CU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <string>
#include <thread>
#include <utility>
#include <vector>

#include "device_util.h"
#include "internal.h"
#include "runtime.h"

namespace mimo {
namespace {

// Threads per workgroup: 512, or 256 for a batch of at least
// kNarrowMinTiles tiles whose resized axes have at most kNarrowMaxTaps taps
// per output (mild resizes), where smaller workgroups keep more units in
// flight (RGBA 640x480..1920x1080 under the stock geometry: 0.53 against
// 0.62 ms; a 1.7x downscale would take 1.81 against 1.49 ms).  A small grid
// keeps the wide workgroups, which finish each tile sooner.
constexpr int kHfThreadsWide = 512, kHfThreadsNarrow = 256;
constexpr int kNarrowMaxTaps = 5;
constexpr int64_t kNarrowMinTiles = 1024;
constexpr int kWeightBits = 22;           // fractional bits of the resampler's weights
constexpr int kMidRows = 256;             // most LDS band rows (32 pixels each)
constexpr int kStageDwords = 4096;        // most LDS source staging (one dword per pixel)
constexpr int kTapBudget = 2048;          // most LDS weights per axis (else they are read from memory)
constexpr int64_t kParallelTapWork = 1 << 18;  // weights (outputs x taps) worth several host threads
constexpr int kFixedDwords = 3 * 256 + kUnitPx * kUnitPx + 2 * kUnitPx;  // lut, block, first x/y
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
    // dynamic LDS, sized for the batch (dwords, each a multiple of 4):
    // [fixed][x weights][y weights][band mid_rows x 32][stage]
    int32_t xw_budget, yw_budget, mid_rows, stage_dwords;
};

// workspace: [HfItem x n][int64 tile_begin x (n+1)][float lut x 768][int32 taps]
size_t hf_items_bytes(int32_t n) { return align256(sizeof(HfItem) * size_t(n)); }
size_t hf_prefix_bytes(int32_t n) { return align256(sizeof(int64_t) * (size_t(n) + 1)); }
constexpr size_t kLutBytes = 3 * 256 * sizeof(float);

__device__ __forceinline__ uint32_t round_clip_byte(int32_t acc) {
    const int32_t v = (acc + (1 << (kWeightBits - 1))) >> kWeightBits;
    return uint32_t(v < 0 ? 0 : (v > 255 ? 255 : v));
}

typedef const __attribute__((address_space(3))) int32_t *lds_weights;

// One resampled pixel: `taps` taps of px[j * stride] (RGB bytes in a dword,
// in LDS) weighted by w[j], summed per channel in int32 and rounded back to
// a byte.  `taps` is the same for every output of an axis (unused taps have
// zero weight), so the loop is uniform across the wavefront.  The weights
// have kWeightBits fraction bits and magnitude below 2, so they are 24-bit
// signed values: said so explicitly, the products run on the full-rate
// 24-bit multiplier instead of a 64-bit multiply-add.  The weights come from
// LDS or from memory; the two are separate overloads so that neither goes
// through flat (generic) addressing.
template <typename Weights>
__device__ __forceinline__ uint32_t resample_px(const uint32_t *px, int stride, Weights w, int taps) {
    int32_t acc0 = 0, acc1 = 0, acc2 = 0;
    for (int j = 0; j < taps; ++j) {
        const uint32_t p = px[j * stride];
        const int32_t wj = __builtin_amdgcn_sbfe(w[j], 0, 24);
        acc0 += int32_t(p & 255u) * wj;
        acc1 += int32_t((p >> 8) & 255u) * wj;
        acc2 += int32_t((p >> 16) & 255u) * wj;
    }
    return round_clip_byte(acc0) | (round_clip_byte(acc1) << 8) | (round_clip_byte(acc2) << 16);
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

// RGB bytes of the four consecutive pixels at byte offset `off` of the
// window (any alignment), one pixel per dword; alpha is dropped.  One
// 12-byte (RGB) or 16-byte (RGBA) load when `off` is dword aligned, else a
// 16-byte load (plus a dword for RGBA) realigned with v_alignbyte.
__device__ __forceinline__ void load_quad(const SrcWindow &w, uint32_t off, int channels, u32x4 &p) {
    const uint32_t al = off & ~3u, sh = off & 3u;
    if (channels == 3) {
        uint32_t u0, u1, u2;
        if (sh == 0) {
            const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(w.rsrc, int(al), 0, 0));
            u0 = v.x; u1 = v.y; u2 = v.z;
        } else {
            const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w.rsrc, int(al), 0, 0));
            u0 = __builtin_amdgcn_alignbyte(v.y, v.x, sh);
            u1 = __builtin_amdgcn_alignbyte(v.z, v.y, sh);
            u2 = __builtin_amdgcn_alignbyte(v.w, v.z, sh);
        }
        // bytes R0 G0 B0 R1 | G1 B1 R2 G2 | B2 R3 G3 B3 -> one pixel per dword
        p.x = u0 & 0x00FFFFFFu;
        p.y = __builtin_amdgcn_perm(u1, u0, 0x0C050403u);
        p.z = __builtin_amdgcn_perm(u2, u1, 0x0C040302u);
        p.w = u2 >> 8;
    } else {
        u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w.rsrc, int(al), 0, 0));
        if (sh != 0) {
            const uint32_t v4 = __builtin_amdgcn_raw_buffer_load_b32(w.rsrc, int(al) + 16, 0, 0);
            v = {__builtin_amdgcn_alignbyte(v.y, v.x, sh), __builtin_amdgcn_alignbyte(v.z, v.y, sh),
                 __builtin_amdgcn_alignbyte(v.w, v.z, sh), __builtin_amdgcn_alignbyte(v4, v.w, sh)};
        }
        p = v & 0x00FFFFFFu;
    }
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

template <typename OutT, int kHfThreads>
__global__ __launch_bounds__(kHfThreads) void hf_preprocess_kernel(HfArgs a) {
    // LDS, sized by the host for the batch (see HfArgs)
    extern __shared__ uint32_t lds[];
    float *lut = reinterpret_cast<float *>(lds);                     // [3][256]
    uint32_t *block = lds + 3 * 256;                                  // the unit's output bytes (RGB per dword)
    int32_t *xfirst_s = reinterpret_cast<int32_t *>(block + kUnitPx * kUnitPx);  // the tile's taps: first
    int32_t *yfirst_s = xfirst_s + kUnitPx;                           // (relative to the staged block /
                                                                      // band) and weights
    int32_t *xw_s = reinterpret_cast<int32_t *>(lds + kFixedDwords);
    int32_t *yw_s = xw_s + a.xw_budget;
    uint32_t *mid = reinterpret_cast<uint32_t *>(yw_s + a.yw_budget);  // horizontal-pass band
    uint32_t *stage = mid + a.mid_rows * kUnitPx;                     // source pixels of a row chunk
    const int64_t tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    const int img = find_segment(a.tile_begin, a.n, tile);
    const HfItem d = a.items[img];
    // An item lists one tile per (merge unit, group of G output rows); G is
    // a power of two, 32 (one tile per unit) unless the vertical taps of 32
    // rows do not fit the band.
    const int G = d.group;
    const int gsh = __builtin_ctz(unsigned(G));
    const int local = int(tile - a.tile_begin[img]);
    const int unit = local >> (5 - gsh);
    const int g0 = (local & ((kUnitPx >> gsh) - 1)) << gsh;  // the group's first row in the unit
    const int br = div_small(unit, d.blocks_w, 1.0f / float(d.blocks_w));
    const int bc = unit - br * d.blocks_w;
    const int oy0 = br * kUnitPx, ox0 = bc * kUnitPx;
    const int tid = threadIdx.x;
    for (int i = tid; i < 3 * 256; i += kHfThreads) lut[i] = a.lut[i];

    const uint8_t *img_src = a.src + d.src_offset;
    const int64_t row_bytes = int64_t(d.src_w) * d.channels;
    if (!d.kx && !d.ky) {
        // no resize: the unit's 32 x 32 source pixels go straight to the block
        const SrcWindow win = src_window(a, reinterpret_cast<uint64_t>(img_src) +
                                                uint64_t(int64_t(oy0) * row_bytes + int64_t(ox0) * d.channels));
        for (int idx = tid; idx < kUnitPx * kUnitPx / 4; idx += kHfThreads) {
            const int r = idx >> 3, q = idx & 7;
            u32x4 px;
            load_quad(win, win.lead + uint32_t(int64_t(r) * row_bytes + 4 * q * d.channels), d.channels, px);
            *reinterpret_cast<u32x4 *>(&block[r * kUnitPx + 4 * q]) = px;
        }
        __syncthreads();
    } else {
        const int dst_w = d.blocks_w * kUnitPx, dst_h = d.blocks_h * kUnitPx;
        const int32_t *xf = d.kx ? a.taps + d.x_tab : nullptr;  // first[dst_w], count[dst_w], w[dst_w][kx]
        const int32_t *yf = d.ky ? a.taps + d.y_tab : nullptr;
        // source columns the tile's 32 output columns read, and their taps in LDS
        // (the weights too, when they fit; else they are read from memory)
        const int xlo = xf ? xf[ox0] : ox0;
        const int xhi = xf ? xf[ox0 + kUnitPx - 1] + xf[dst_w + ox0 + kUnitPx - 1] : ox0 + kUnitPx;
        const int quads = (xhi - xlo + 3) >> 2;  // staged 4 pixels at a time
        const int spitch = 4 * quads;             // <= a.stage_dwords (the host checked)
        const bool xw_in_lds = xf && kUnitPx * d.kx <= a.xw_budget;
        if (xf) {
            for (int i = tid; i < kUnitPx; i += kHfThreads) xfirst_s[i] = xf[ox0 + i] - xlo;
            if (xw_in_lds)
                for (int i = tid; i < kUnitPx * d.kx; i += kHfThreads)
                    xw_s[i] = xf[2 * dst_w + int64_t(ox0) * d.kx + i];
        }
        const bool yw_in_lds = yf && G * d.ky <= a.yw_budget;
        const int oy_a = oy0 + g0, oy_b = oy_a + G - 1;
        const int ylo = yf ? yf[oy_a] : oy_a;
        const int yhi = yf ? yf[oy_b] + yf[dst_h + oy_b] : oy_b + 1;
        const int nrows = yhi - ylo;  // <= a.mid_rows (the host sized G)
        if (yf) {
            for (int i = tid; i < G; i += kHfThreads) yfirst_s[i] = yf[oy_a + i] - ylo;
            if (yw_in_lds)
                for (int i = tid; i < G * d.ky; i += kHfThreads)
                    yw_s[i] = yf[2 * dst_h + int64_t(oy_a) * d.ky + i];
        }
        const int chunk = min(nrows, a.stage_dwords / spitch);
        const float inv_quads = 1.0f / float(quads);
        for (int r0 = 0; r0 < nrows; r0 += chunk) {
            const int nr = min(chunk, nrows - r0);
            // stage source rows [ylo + r0, ylo + r0 + nr) x [xlo, xlo + spitch);
            // the up to 3 pixels past xhi are never read
            const SrcWindow win = src_window(a, reinterpret_cast<uint64_t>(img_src) +
                                                    uint64_t(int64_t(ylo + r0) * row_bytes +
                                                             int64_t(xlo) * d.channels));
            for (int idx = tid; idx < nr * quads; idx += kHfThreads) {
                const int r = div_small(idx, quads, inv_quads);
                const int q = idx - r * quads;
                u32x4 px;
                load_quad(win, win.lead + uint32_t(int64_t(r) * row_bytes + 4 * q * d.channels), d.channels, px);
                *reinterpret_cast<u32x4 *>(&stage[r * spitch + 4 * q]) = px;
            }
            __syncthreads();
            // horizontal pass (or a copy) into band rows [r0, r0 + nr)
            for (int idx = tid; idx < nr * kUnitPx; idx += kHfThreads) {
                const int r = idx >> 5, x = idx & 31;
                const uint32_t *line = &stage[r * spitch];
                uint32_t px;
                if (xf) {
                    const int first = xfirst_s[x];
                    if (xw_in_lds)
                        px = resample_px(line + first, 1, (lds_weights)(&xw_s[x * d.kx]), d.kx);
                    else
                        px = resample_px(line + first, 1, xf + 2 * dst_w + int64_t(ox0 + x) * d.kx, d.kx);
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
                const uint32_t *col = &mid[yfirst_s[r] * kUnitPx + x];
                if (yw_in_lds)
                    px = resample_px(col, kUnitPx, (lds_weights)(&yw_s[r * d.ky]), d.ky);
                else
                    px = resample_px(col, kUnitPx, yf + 2 * dst_h + int64_t(oy) * d.ky, d.ky);
            } else {
                px = mid[idx];
            }
            block[(g0 + r) * kUnitPx + x] = px;
        }
        __syncthreads();
    }

    // The group's G pixel rows x 2 patch columns x 3 channels x 4 quads of 4
    // pixels; each thread stores one quad into both temporal slots, a wave
    // one contiguous run of a (c, tt) plane.
    for (int idx = tid; idx < G * 2 * 3 * 4; idx += kHfThreads) {
        const int qd = idx & 3;
        const int yl = (idx >> 2) & (G - 1);
        const int mc = idx >> (2 + gsh);  // (mw, c): 0 .. 5
        const int mw = mc >= 3 ? 1 : 0;
        const int c = mc - 3 * mw;
        const int y = g0 + yl;            // pixel row in the unit
        const int mh = y >> 4, py = y & (kPatch - 1);
        const int q = mh * kMerge + mw;   // row of the unit
        const uint32_t *src_px = &block[y * kUnitPx + mw * kPatch + qd * 4];
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

// PIL's window of output i on an axis of n_in inputs: [lo, hi).
struct AxisMap {
    int64_t n_in, n_out;
    double scale, widen, support;
    AxisMap(int64_t in, int64_t out) : n_in(in), n_out(out) {
        scale = double(n_in) / double(n_out);
        widen = scale < 1.0 ? 1.0 : scale;
        support = 2.0 * widen;
    }
    void window(int64_t i, int64_t &lo, int64_t &hi, double &centre) const {
        centre = (double(i) + 0.5) * scale;
        lo = int64_t(centre - support + 0.5);
        if (lo < 0) lo = 0;
        hi = int64_t(centre + support + 0.5);
        if (hi > n_in) hi = n_in;
    }
};

// An axis table is first[n_out], count[n_out], weights[n_out][k].  Every
// output gets the same k taps, the most any output of the axis has: its
// window [first, first + k) is moved left where it would run past the last
// input (its own taps then sit further right in the row), and the weights
// it does not use are zero.  The kernel then runs one tap count for every
// output and never reads outside the image; the sums are those of the
// outputs' own taps, since the extra terms are zero.

// k of an axis (at least 1, at most n_in).
int axis_tap_count(int64_t n_in, int64_t n_out) {
    const AxisMap m(n_in, n_out);
    int64_t k = 1;
    for (int64_t i = 0; i < n_out; ++i) {
        int64_t lo, hi;
        double centre;
        m.window(i, lo, hi, centre);
        k = std::max(k, hi - lo);
    }
    return int(k);
}

// first and count of an axis table at tab (the cheap part: what the host's
// band and staging sizes need).
void fill_axis_heads(int64_t n_in, int64_t n_out, int k, int32_t *tab) {
    const AxisMap m(n_in, n_out);
    for (int64_t i = 0; i < n_out; ++i) {
        int64_t lo, hi;
        double centre;
        m.window(i, lo, hi, centre);
        tab[i] = int32_t(std::min<int64_t>(lo, n_in - k));
        tab[n_out + i] = k;
    }
}

// The weights of an axis table at tab (zeroed by the caller), in float64
// as PIL computes them, rounded half away from zero to kWeightBits.
void fill_axis_weights(int64_t n_in, int64_t n_out, int k, int32_t *tab) {
    const AxisMap m(n_in, n_out);
    int32_t *weight = tab + 2 * n_out;
    std::vector<double> w(size_t(k) + 1);
    for (int64_t i = 0; i < n_out; ++i) {
        int64_t lo, hi;
        double centre;
        m.window(i, lo, hi, centre);
        const int64_t cnt = hi - lo;
        double sum = 0.0;
        for (int64_t j = 0; j < cnt; ++j) {
            w[j] = keys_bicubic((double(j + lo) - centre + 0.5) / m.widen);
            sum += w[j];
        }
        const int64_t shift = lo - tab[i];
        for (int64_t j = 0; j < cnt; ++j) {
            const double v = sum != 0.0 ? w[j] / sum : w[j];
            const double fixed = v * double(1 << kWeightBits);
            weight[i * k + shift + j] = int32_t(v < 0.0 ? fixed - 0.5 : fixed + 0.5);
        }
    }
}

struct HfTables {
    std::vector<uint8_t> head;    // items, tile prefix, lut
    std::vector<int32_t> taps;
    int64_t tiles = 0;
    int64_t rows = 0;
    // dynamic LDS the batch needs (dwords, multiples of 4; see HfArgs)
    int32_t xw_budget = 0, yw_budget = 0, mid_rows = 0, stage_dwords = 0;
    int32_t max_taps = 0;  // the most taps per output over the batch's resized axes
    size_t lds_bytes() const {
        return 4 * (size_t(kFixedDwords) + xw_budget + yw_budget + size_t(mid_rows) * kUnitPx + stage_dwords);
    }
};

int32_t round4(int64_t v) { return int32_t((v + 3) & ~int64_t(3)); }

// The most source rows one group of g output rows reads.
int band_rows(const int32_t *yfirst, const int32_t *ycount, int dst_h, int g) {
    int most = 0;
    for (int y0 = 0; y0 < dst_h; y0 += g) {
        const int y1 = y0 + g - 1;
        most = std::max(most, yfirst[y1] + ycount[y1] - yfirst[y0]);
    }
    return most;
}

// Output rows per vertical group so that the band of source rows one group
// needs fits kMidRows: the largest of 32, 16, ..., 1 that fits everywhere.
int choose_group(const int32_t *yfirst, const int32_t *ycount, int dst_h) {
    for (int g = kUnitPx; g >= 1; g >>= 1)
        if (band_rows(yfirst, ycount, dst_h, g) <= kMidRows) return g;
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
    // One tap table per (input length, output length) pair in the batch:
    // items of the same size share it (built and uploaded once).  Its first
    // and count entries are filled here; the weights, the costly part, after
    // the loop, several tables at a time.
    std::map<std::pair<int32_t, int32_t>, std::pair<int64_t, int32_t>> tables;
    auto axis_table = [&](int32_t n_in, int32_t n_out, int64_t &tab, int32_t &k) {
        const auto key = std::make_pair(n_in, n_out);
        const auto it = tables.find(key);
        if (it != tables.end()) {
            tab = it->second.first;
            k = it->second.second;
            return;
        }
        k = axis_tap_count(n_in, n_out);
        tab = int64_t(out.taps.size());
        out.taps.resize(out.taps.size() + size_t(n_out) * (2 + k), 0);
        fill_axis_heads(n_in, n_out, k, out.taps.data() + tab);
        tables.emplace(key, std::make_pair(tab, k));
    };
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
        if (s.dst_w != s.src_w) axis_table(s.src_w, s.dst_w, d.x_tab, d.kx);
        if (s.dst_h != s.src_h) {
            axis_table(s.src_h, s.dst_h, d.y_tab, d.ky);
            const int32_t *yfirst = out.taps.data() + d.y_tab;
            d.group = choose_group(yfirst, yfirst + s.dst_h, s.dst_h);
            if (d.group == 0)
                return set_error(MIMO_E_UNSUPPORTED, "preprocess_hf: descriptor " + std::to_string(i) +
                                                         ": vertical downscale beyond the kernel's band");
        }
        int spitch = kUnitPx;  // staged pixels per source row (whole quads)
        if (d.kx) {
            // the widest source block one tile's 32 output columns read
            const int32_t *xfirst = out.taps.data() + d.x_tab;
            const int32_t *xcount = xfirst + s.dst_w;
            for (int32_t x0 = 0; x0 < s.dst_w; x0 += kUnitPx) {
                const int32_t x1 = x0 + kUnitPx - 1;
                spitch = std::max(spitch, round4(xfirst[x1] + xcount[x1] - xfirst[x0]));
            }
            if (spitch > kStageDwords)
                return set_error(MIMO_E_UNSUPPORTED, "preprocess_hf: descriptor " + std::to_string(i) +
                                                         ": horizontal downscale beyond the kernel's staging");
            if (kUnitPx * d.kx <= kTapBudget) out.xw_budget = std::max(out.xw_budget, round4(kUnitPx * d.kx));
        }
        if (d.kx || d.ky) {
            // band rows of one group, and staging for all of them at once when that fits
            const int nrows = d.ky ? band_rows(out.taps.data() + d.y_tab, out.taps.data() + d.y_tab + s.dst_h,
                                               s.dst_h, d.group)
                                   : d.group;
            out.mid_rows = std::max(out.mid_rows, round4(nrows));
            out.stage_dwords = std::max<int32_t>(
                out.stage_dwords, int32_t(std::min<int64_t>(kStageDwords, int64_t(nrows) * spitch)));
            if (d.ky && d.group * d.ky <= kTapBudget)
                out.yw_budget = std::max(out.yw_budget, round4(d.group * d.ky));
        }
        items[i] = d;
        out.max_taps = std::max(out.max_taps, std::max(d.kx, d.ky));
        tiles += int64_t(d.blocks_h) * d.blocks_w * (kUnitPx / d.group);
        rows += s.rows;
    }
    tile_begin[n] = tiles;
    out.tiles = tiles;
    out.rows = rows;
    if (out.taps.size() > size_t(0x7FFFFFFF))
        return set_error(MIMO_E_TOO_LARGE, "preprocess_hf: tap tables above 2^31 entries");
    // the weights: tables are independent, so large batches of them are
    // shared out over up to 16 host threads
    struct Job {
        int32_t n_in, n_out, k;
        int64_t tab;
    };
    std::vector<Job> jobs;
    int64_t work = 0;
    for (const auto &t : tables) {
        jobs.push_back({t.first.first, t.first.second, t.second.second, t.second.first});
        work += int64_t(t.first.second) * t.second.second;
    }
    auto run = [&](size_t from, size_t step) {
        for (size_t j = from; j < jobs.size(); j += step)
            fill_axis_weights(jobs[j].n_in, jobs[j].n_out, jobs[j].k, out.taps.data() + jobs[j].tab);
    };
    const size_t threads =
        std::min<size_t>({size_t(16), jobs.size(), size_t(std::max(1u, std::thread::hardware_concurrency()))});
    if (threads < 2 || work < kParallelTapWork) {
        run(0, 1);
    } else {
        std::vector<std::thread> pool;
        for (size_t t = 1; t < threads; ++t) pool.emplace_back(run, t, threads);
        run(0, threads);
        for (auto &th : pool) th.join();
    }
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
    a.xw_budget = t.xw_budget;
    a.yw_budget = t.yw_budget;
    a.mid_rows = t.mid_rows;
    a.stage_dwords = t.stage_dwords;
    const size_t lds = t.lds_bytes();
    const bool narrow = t.max_taps >= 1 && t.max_taps <= kNarrowMaxTaps && t.tiles >= kNarrowMinTiles;
    const bool f32 = out_dtype == MIMO_F32;
    const void *kernel =
        narrow ? (f32 ? reinterpret_cast<const void *>(hf_preprocess_kernel<float, kHfThreadsNarrow>)
                      : reinterpret_cast<const void *>(hf_preprocess_kernel<uint16_t, kHfThreadsNarrow>))
               : (f32 ? reinterpret_cast<const void *>(hf_preprocess_kernel<float, kHfThreadsWide>)
                      : reinterpret_cast<const void *>(hf_preprocess_kernel<uint16_t, kHfThreadsWide>));
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return hip_error(e, "preprocess_hf: LDS size");
    const dim3 grid{unsigned(t.tiles), 1, 1};
    const dim3 block{unsigned(narrow ? kHfThreadsNarrow : kHfThreadsWide), 1, 1};
    e = timed_launch(s, [&] {
        if (narrow && f32)
            hipLaunchKernelGGL((hf_preprocess_kernel<float, kHfThreadsNarrow>), grid, block, lds, s, a);
        else if (narrow)
            hipLaunchKernelGGL((hf_preprocess_kernel<uint16_t, kHfThreadsNarrow>), grid, block, lds, s, a);
        else if (f32)
            hipLaunchKernelGGL((hf_preprocess_kernel<float, kHfThreadsWide>), grid, block, lds, s, a);
        else
            hipLaunchKernelGGL((hf_preprocess_kernel<uint16_t, kHfThreadsWide>), grid, block, lds, s, a);
    });
    if (e != hipSuccess) return hip_error(e, "preprocess_hf: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

}  // extern "C"
