// preprocess.hip -- fused MiMo-V2 pixel-path kernel and column-order gather
// kernel for AMD Instinct MI355X (gfx950, CDNA4).
//
// What is computed (NeMo Automodel "mimo_v2_flash.processing", class
// docstring of MimoV2ImageProcessor and _to_rgb; docs.rs
// "cortiq_engine::mimo_vision", module conventions, resize_bilinear and
// column_permutation): RGBA flattened onto white, cast to float 0-255,
// bilinear resize with align_corners=False and no antialias (W taps on the
// two source rows, then the H tap), standardisation in 0-255 units, two
// identical frames, rows of 1536 values flattened as (c, tt, py, px) in
// merge-block order (t, block row, block col, mh, mw), and optionally the
// same rows in column order (t, block col, block row).
//
// Work decomposition.  A tile is a run of up to K merge units (32x32 output
// pixels each) along one block row of one image; one 256-thread workgroup
// (four 64-wide wavefronts) owns a tile, so every output byte has exactly
// one writer.  Ragged batches are one flat tile list: a workgroup finds its
// image with a 64-ary wavefront search over the per-image tile prefix sums.
//
// Per tile: (1) the source band the tile's taps touch is copied from HBM
// into LDS with 16-byte buffer loads, realigned and converted to one dword
// per pixel (R, G, B bytes; RGBA flattened onto white here, in integer
// arithmetic); (2) each wavefront produces one output row (one 16x16 patch,
// 3 channels) at a time: lane (py, q) computes 4 consecutive pixels, and the
// wavefront stores each (c, tt) plane as one contiguous 1 KB run of
// non-temporal 16-byte stores (fp32) or 512 B (bf16), writing every value
// twice (tt = 0, 1).  Tiles whose band would not fit the LDS budget read
// their taps straight from global memory instead (same arithmetic).
//
// Arithmetic (matches torch's float32 CPU/GPU bilinear): scale =
// float(n_in)/float(n_out) (host), src = fma(scale, d + 0.5, -0.5) clamped
// at 0, i0 = floor(src), l1 = src - i0, l0 = 1 - l1, i1 = min(i0+1, n_in-1);
// t = fma(l0x, v00, l1x*v01) per source row, out = fma(l0y, t0, l1y*t1).
// Standardisation is (out - mean255) * (1/std255): the subtraction is the
// same as in (out - mean255) / std255 (exact near the mean), and the product
// with the rounded reciprocal stays within two float32 ulps of the quotient
// (relative), so a bf16 rounding of it is within one bf16 ulp even for
// outputs near zero.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "device_util.h"
#include "internal.h"
#include "runtime.h"
#include "tables.h"

namespace mimo {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// LDS budget for one tile's source band, in dwords (one dword per pixel).
constexpr int kBandBudgetDwords = 12288;  // 48 KB
// Most output columns of one tile (three merge units side by side): the size
// of each of the three x-tap arrays that follow the band in LDS.
constexpr int kMaxTileCols = 3 * kUnitPx;
constexpr int kMaxTileRows = kUnitPx;  // output rows one tile covers
static_assert(MIMO_ROWS_PER_TILE <= 3 * kRowsPerUnit && MIMO_ROWS_PER_TILE_CLIPS <= 3 * kRowsPerUnit &&
                  MIMO_ROWS_PER_TILE_DUAL <= kRowsPerUnit,
              "a tile spans at most three merge units of output columns");
// Buffer resource word 3 for raw (untyped) buffer loads on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;

// Batches of at most this many images carry their descriptor tables in the
// kernel arguments (296 bytes), so a call makes no table upload.
constexpr int kInlineImages = 4;

struct PreArgs {
    const uint8_t *src;
    const DevImage *images;     // null: the tables are inline (below)
    const int64_t *tile_begin;  // [n + 1]
    void *rows;                 // merge-block order, nullable
    void *rows_col;             // column order, nullable
    int64_t src_end;            // bytes readable from src
    int64_t tiles_per_pass;     // tiles of one output; a second pass follows for rows_col
    int32_t n;
    int32_t band_capacity;      // dwords of dynamic LDS
    int32_t rows_per_tile;      // 1, 2 or a multiple of 4 (at most 4 with two outputs)
    int32_t xcd_order;          // map workgroups to XCD-contiguous tile runs
    float inv_std[3];           // 1 / std255, rounded once
    float mean[3];              // mean255
    DevImage inl_images[kInlineImages];
    int64_t inl_tile_begin[kInlineImages + 1];
};

// The image that holds `tile` (largest i with tile_begin[i] <= tile), from
// the inline tables (kInline) or the workspace; wave-uniform.
template <bool kInline>
__device__ __forceinline__ int tile_image(const PreArgs &a, int64_t tile) {
    if (!kInline) return find_segment(a.tile_begin, a.n, tile);
    int img = 0;
#pragma unroll
    for (int i = 1; i < kInlineImages; ++i)
        if (i < a.n && a.inl_tile_begin[i] <= tile) img = i;
    return img;
}

// Entry `img` of the tables.  The inline arrays are read with constant
// indices only (scalar loads from the kernel arguments).
template <bool kInline>
__device__ __forceinline__ DevImage image_at(const PreArgs &a, int img) {
    if (!kInline) return a.images[img];
    DevImage d = a.inl_images[0];
#pragma unroll
    for (int i = 1; i < kInlineImages; ++i)
        if (img == i) d = a.inl_images[i];
    return d;
}

template <bool kInline>
__device__ __forceinline__ int64_t tile_begin_at(const PreArgs &a, int img) {
    if (!kInline) return a.tile_begin[img];
    int64_t b = a.inl_tile_begin[0];
#pragma unroll
    for (int i = 1; i <= kInlineImages; ++i)
        if (img == i) b = a.inl_tile_begin[i];
    return b;
}

struct PermArgs {
    const DevImage *images;
    const int64_t *row_begin;  // [n + 1]
    const void *in;
    void *out;
    int64_t total_units;
    int32_t n;
};

// ---------------------------------------------------------------- helpers

struct Tap {
    int i0;
    float l0, l1;
};

// Half-pixel source coordinate for destination index d on an axis of n_in
// source samples (align_corners=False, clamped below at 0): the first tap
// and the two weights.  The second tap is i0 + 1, or i0 at the last sample.
__device__ __forceinline__ Tap make_tap(float scale, int d, int n_in) {
    float s = __builtin_fmaf(scale, float(d) + 0.5f, -0.5f);
    s = s < 0.0f ? 0.0f : s;
    int i0 = int(s);  // s >= 0: truncation is floor
    i0 = i0 < n_in - 1 ? i0 : n_in - 1;
    Tap t;
    t.i0 = i0;
    t.l1 = s - float(i0);
    t.l0 = 1.0f - t.l1;
    return t;
}

// One channel of an RGBA pixel composited over white with coverage a/255,
// rounded to nearest: 255 - a + round(v*a/255).  v*a/255 never lies exactly
// halfway between integers, so round(x) = floor((v*a + 127) / 255).
__device__ __forceinline__ uint32_t flatten_channel(uint32_t v, uint32_t a) {
    return 255u - a + (v * a + 127u) / 255u;
}

__device__ __forceinline__ uint32_t flatten_rgba(uint32_t px) {
    const uint32_t a = px >> 24;
    const uint32_t r = flatten_channel(px & 255u, a);
    const uint32_t g = flatten_channel((px >> 8) & 255u, a);
    const uint32_t b = flatten_channel((px >> 16) & 255u, a);
    return r | (g << 8) | (b << 16);
}

__device__ __forceinline__ float chan(uint32_t px, int c) {
    return float((px >> (8 * c)) & 255u);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {__bf16(lo), __bf16(hi)};  // hardware round-to-nearest-even
    return __builtin_bit_cast(uint32_t, v);
}

// Stores one lane's 4 consecutive values of channel c into temporal slot TT
// of a row, or into both slots when TT < 0 (two identical frames).  row_ptr
// points at the row's element (py*16 + 4q).
template <int TT>
__device__ __forceinline__ void store_frames(float *row_ptr, int c, const float (&v)[4]) {
    const f32x4 q = {v[0], v[1], v[2], v[3]};
    float *p = row_ptr + c * (kTemporal * kPlane);
    if (TT <= 0) __builtin_nontemporal_store(q, reinterpret_cast<f32x4 *>(p));
    if (TT != 0) __builtin_nontemporal_store(q, reinterpret_cast<f32x4 *>(p + kPlane));
}

template <int TT>
__device__ __forceinline__ void store_frames(uint16_t *row_ptr, int c, const float (&v)[4]) {
    const u32x2 q = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    uint16_t *p = row_ptr + c * (kTemporal * kPlane);
    if (TT <= 0) __builtin_nontemporal_store(q, reinterpret_cast<u32x2 *>(p));
    if (TT != 0) __builtin_nontemporal_store(q, reinterpret_cast<u32x2 *>(p + kPlane));
}

// A raw buffer resource over [first & ~3, src_end): `lead` is first's offset
// in it.  Reads past the end return zero.
struct SourceWindow {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t lead;
};

__device__ __forceinline__ SourceWindow source_window(const PreArgs &a, uint64_t first) {
    const uint64_t base = first & ~uint64_t(3);
    const uint64_t end = reinterpret_cast<uint64_t>(a.src) + uint64_t(a.src_end);
    const uint64_t avail = end - base;
    const int num = avail > 0x7FFFFFF0ull ? 0x7FFFFFF0 : int(avail);
    SourceWindow w;
    w.rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(base), 0, num, kBufferWord3);
    w.lead = uint32_t(first - base);
    return w;
}

// Four consecutive pixels starting `off` bytes into the window, as dwords
// R | G<<8 | B<<16 (RGBA flattened onto white).  One buffer load of exactly
// 12 (RGB) or 16 (RGBA) bytes when `off` is dword aligned, else a 16-byte
// load (plus a dword for RGBA) realigned with v_alignbyte.
__device__ __forceinline__ void load_4px(const SourceWindow &w, uint32_t off, int channels,
                                         uint32_t (&p)[4]) {
    const uint32_t al = off & ~3u;
    const uint32_t sh = off & 3u;
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
        p[0] = u0 & 0x00FFFFFFu;
        p[1] = __builtin_amdgcn_perm(u1, u0, 0x0C050403u);
        p[2] = __builtin_amdgcn_perm(u2, u1, 0x0C040302u);
        p[3] = u2 >> 8;
    } else {
        const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w.rsrc, int(al), 0, 0));
        if (sh == 0) {
            p[0] = flatten_rgba(v.x); p[1] = flatten_rgba(v.y);
            p[2] = flatten_rgba(v.z); p[3] = flatten_rgba(v.w);
        } else {
            const uint32_t v4 = __builtin_amdgcn_raw_buffer_load_b32(w.rsrc, int(al) + 16, 0, 0);
            p[0] = flatten_rgba(__builtin_amdgcn_alignbyte(v.y, v.x, sh));
            p[1] = flatten_rgba(__builtin_amdgcn_alignbyte(v.z, v.y, sh));
            p[2] = flatten_rgba(__builtin_amdgcn_alignbyte(v.w, v.z, sh));
            p[3] = flatten_rgba(__builtin_amdgcn_alignbyte(v4, v.w, sh));
        }
    }
}

// Destination of output row (t, br, bc, mh, mw): its merge-block position,
// or its column-order position when `column` (units of temporal patch t
// listed by (block col, block row)).
template <typename OutT>
__device__ __forceinline__ OutT *row_dest(OutT *out, const DevImage &d, int t, int br, int bc,
                                          int mh, int mw, bool column) {
    const int64_t units = int64_t(d.blocks_h) * d.blocks_w;
    const int64_t unit = t * units +
                         (column ? int64_t(bc) * d.blocks_h + br : int64_t(br) * d.blocks_w + bc);
    const int64_t row = d.row_offset + unit * kRowsPerUnit + mh * kMerge + mw;
    const int lane = threadIdx.x & 63;
    // the row's start (uniform across the wave) plus the lane's 32-bit offset
    OutT *const start = out + row * kRowLen;
    return start + ((lane >> 2) * kPatch + 4 * (lane & 3));
}

// Identity resize (dst == src): output pixel (y, x) is source pixel (y, x).
// Each lane reads its 4 pixels straight from HBM; no LDS.  The values go to
// temporal slot TT of row (t, br, bc, mh, mw), or to both slots if TT < 0.
template <typename OutT, int TT>
__device__ __forceinline__ void identity_patch(const PreArgs &a, const DevImage &d,
                                               const SourceWindow &w, int64_t row_bytes, int oy0,
                                               int ox0, int t, int br, int bc, int mh, int mw,
                                               OutT *out, bool column) {
    const int lane = threadIdx.x & 63;
    const int py = lane >> 2, q = lane & 3;
    const int oy = (br * kMerge + mh) * kPatch + py;
    const int ox = (bc * kMerge + mw) * kPatch + 4 * q;
    const uint32_t off = w.lead + uint32_t(int64_t(oy - oy0) * row_bytes) + uint32_t((ox - ox0) * d.channels);
    uint32_t p[4];
    load_4px(w, off, d.channels, p);
    float v[3][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 3; ++c) v[c][j] = (chan(p[j], c) - a.mean[c]) * a.inv_std[c];
    OutT *dst = row_dest(out, d, t, br, bc, mh, mw, column);
#pragma unroll
    for (int c = 0; c < 3; ++c) store_frames<TT>(dst, c, v[c]);
}

// Source pixels for the bilinear taps.  Both give the pixel at (y, x) for
// y <= n_rows and x <= n_cols, where row n_rows / column n_cols stand for
// the last row / column (the second tap at the image edge).
struct BandPixels {  // staged in LDS, edge already replicated
    const uint32_t *band;
    int pitch, r_lo, c_lo;
    // the x taps of the tile's output columns (from column ox_first), made
    // once per tile: first tap relative to c_lo, and its two weights
    const int32_t *xi;
    const float *xl0, *xl1;
    int ox_first;
    // (clip instance) the y taps of its output rows (from row oy_first),
    // likewise: per row the band offsets (dwords) of its two rows, then its
    // two weights
    const i32x4 *yt;
    int oy_first;
};

struct GlobalPixels {  // straight from memory, clamped
    const uint8_t *img;
    int64_t row_bytes;
    int channels, h, w;
    __device__ __forceinline__ uint32_t at(int y, int x) const {
        y = min(y, h - 1);
        x = min(x, w - 1);
        const uint8_t *p = img + int64_t(y) * row_bytes + int64_t(x) * channels;
        const uint32_t px = uint32_t(p[0]) | (uint32_t(p[1]) << 8) | (uint32_t(p[2]) << 16);
        return channels == 4 ? flatten_rgba(px | (uint32_t(p[3]) << 24)) : px;
    }
};

// Bilinear output row (t, br, bc, mh, mw): a 16x16 patch, 3 channels, into
// temporal slot TT (both slots if TT < 0).  W taps on the two source rows,
// then the H tap.
template <typename OutT, int TT, typename Pixels>
__device__ __forceinline__ void bilinear_patch(const Pixels &px, const DevImage &d, const PreArgs &a,
                                               int t, int br, int bc, int mh, int mw, OutT *out,
                                               bool column) {
    const int lane = threadIdx.x & 63;
    const int py = lane >> 2, q = lane & 3;
    const int oy = (br * kMerge + mh) * kPatch + py;
    const int ox0 = (bc * kMerge + mw) * kPatch + 4 * q;
    const Tap ty = make_tap(d.scale_y, oy, d.src_h);
    float v[3][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const Tap tx = make_tap(d.scale_x, ox0 + j, d.src_w);
        const uint32_t p00 = px.at(ty.i0, tx.i0);
        const uint32_t p01 = px.at(ty.i0, tx.i0 + 1);
        const uint32_t p10 = px.at(ty.i0 + 1, tx.i0);
        const uint32_t p11 = px.at(ty.i0 + 1, tx.i0 + 1);
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            const float top = __builtin_fmaf(tx.l0, chan(p00, c), tx.l1 * chan(p01, c));
            const float bot = __builtin_fmaf(tx.l0, chan(p10, c), tx.l1 * chan(p11, c));
            const float val = __builtin_fmaf(ty.l0, top, ty.l1 * bot);
            v[c][j] = (val - a.mean[c]) * a.inv_std[c];
        }
    }
    OutT *dst = row_dest(out, d, t, br, bc, mh, mw, column);
#pragma unroll
    for (int c = 0; c < 3; ++c) store_frames<TT>(dst, c, v[c]);
}

// The same for a tile staged in LDS: the row tap per lane, the column taps
// from the tile's table (three 16-byte LDS reads for the lane's 4 pixels),
// the second taps always one row / column on (the band repeats the image's
// last row and column).  Bitwise the same values as bilinear_patch.
template <typename OutT, int TT, bool kYTab>
__device__ __forceinline__ void bilinear_patch_band(const BandPixels &px, const DevImage &d, const PreArgs &a,
                                                    int t, int br, int bc, int mh, int mw, OutT *out,
                                                    bool column) {
    const int lane = threadIdx.x & 63;
    const int py = lane >> 2, q = lane & 3;
    const int oy = (br * kMerge + mh) * kPatch + py;
    const int xc = (bc * kMerge + mw) * kPatch + 4 * q - px.ox_first;
    Tap ty{0, 0.0f, 0.0f};
    const uint32_t *r0, *r1;
    if (kYTab) {
        // the row offsets now, the weights (a load of their own) where the
        // vertical step needs them
        const int32_t *ye = reinterpret_cast<const int32_t *>(px.yt + (oy - px.oy_first));
        r0 = px.band + ye[0];
        r1 = px.band + ye[1];
        const float *yw = reinterpret_cast<const float *>(ye + 2);
        ty.l0 = yw[0];
        ty.l1 = yw[1];
    } else {
        ty = make_tap(d.scale_y, oy, d.src_h);
        // (both factors below 2^23: the 24-bit multiplier)
        r0 = px.band + __mul24(ty.i0 - px.r_lo, px.pitch);
        r1 = r0 + px.pitch;
    }
    const i32x4 xi = *reinterpret_cast<const i32x4 *>(px.xi + xc);
    const f32x4 l0 = *reinterpret_cast<const f32x4 *>(px.xl0 + xc);
    const f32x4 l1 = *reinterpret_cast<const f32x4 *>(px.xl1 + xc);
    float v[3][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t p00 = r0[xi[j]], p01 = r0[xi[j] + 1];
        const uint32_t p10 = r1[xi[j]], p11 = r1[xi[j] + 1];
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            const float top = __builtin_fmaf(l0[j], chan(p00, c), l1[j] * chan(p01, c));
            const float bot = __builtin_fmaf(l0[j], chan(p10, c), l1[j] * chan(p11, c));
            const float val = __builtin_fmaf(ty.l0, top, ty.l1 * bot);
            v[c][j] = (val - a.mean[c]) * a.inv_std[c];
        }
    }
    OutT *dst = row_dest(out, d, t, br, bc, mh, mw, column);
#pragma unroll
    for (int c = 0; c < 3; ++c) store_frames<TT>(dst, c, v[c]);
}

// Four consecutive pixels as dwords R | G<<8 | B<<16 (RGBA flattened onto
// white) from the 16 bytes `v` at a dword boundary, the dword `v4` after
// them (RGBA only) and the pixels' byte offset `sh` (0..3) past that
// boundary.
template <int C>
__device__ __forceinline__ u32x4 unpack_4px(const u32x4 &v, uint32_t v4, uint32_t sh) {
    if (C == 3) {
        const uint32_t u0 = __builtin_amdgcn_alignbyte(v.y, v.x, sh);
        const uint32_t u1 = __builtin_amdgcn_alignbyte(v.z, v.y, sh);
        const uint32_t u2 = __builtin_amdgcn_alignbyte(v.w, v.z, sh);
        // bytes R0 G0 B0 R1 | G1 B1 R2 G2 | B2 R3 G3 B3 -> one pixel per dword
        return u32x4{u0 & 0x00FFFFFFu, __builtin_amdgcn_perm(u1, u0, 0x0C050403u),
                     __builtin_amdgcn_perm(u2, u1, 0x0C040302u), u2 >> 8};
    } else {
        return u32x4{flatten_rgba(__builtin_amdgcn_alignbyte(v.y, v.x, sh)),
                     flatten_rgba(__builtin_amdgcn_alignbyte(v.z, v.y, sh)),
                     flatten_rgba(__builtin_amdgcn_alignbyte(v.w, v.z, sh)),
                     flatten_rgba(__builtin_amdgcn_alignbyte(v4, v.w, sh))};
    }
}

// Band staging is batched: a thread issues the loads of kStageBatch of its
// band rows before it unpacks any of them, so it waits for one memory round
// trip per kStageBatch rows.  No load is conditional: a row past the band
// gets an offset past the buffer's range, which reads zero without a memory
// access, and is not written.
#ifndef MIMO_STAGE_BATCH
#define MIMO_STAGE_BATCH 4
#endif
constexpr int kStageBatch = MIMO_STAGE_BATCH;
constexpr uint32_t kOutOfRange = 0x80000000u;  // past any window's range
// The loads of one batch of a thread's band rows (rows r, r + step, ...).
struct RowBatch {
    u32x4 v[kStageBatch];
    uint32_t v4[kStageBatch], sh[kStageBatch];
};

template <int C>
__device__ __forceinline__ void issue_rows(RowBatch &b, const SourceWindow &w, int64_t row_bytes,
                                           uint32_t col_bytes, int r, int step, int rows, int last_row) {
#pragma unroll
    for (int i = 0; i < kStageBatch; ++i) {
        const int sr = min(r + i * step, last_row);
        const uint32_t off = col_bytes + uint32_t(int64_t(sr) * row_bytes);
        b.sh[i] = off & 3u;
        const uint32_t at = r + i * step < rows ? off & ~3u : kOutOfRange;
        b.v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w.rsrc, int(at), 0, 0));
        b.v4[i] = C == 4 ? __builtin_amdgcn_raw_buffer_load_b32(w.rsrc, int(at) + 16, 0, 0) : 0u;
    }
}

template <int C>
__device__ __forceinline__ void write_rows(uint32_t *band, RowBatch &b, int r, int step, int rows, int g,
                                           int pitch) {
    // The batch is consumed here, all at once: otherwise the compiler
    // moves each load into the branch that writes its row, behind a wait
    // for the loads before it.
#pragma unroll
    for (int i = 0; i < kStageBatch; ++i) {
        asm volatile("" : "+v"(b.v[i]));
        if (C == 4) asm volatile("" : "+v"(b.v4[i]));
    }
#pragma unroll
    for (int i = 0; i < kStageBatch; ++i)
        if (r + i * step < rows)
            *reinterpret_cast<u32x4 *>(band + (r + i * step) * pitch + 4 * g) = unpack_4px<C>(b.v[i], b.v4[i], b.sh[i]);
}

// This thread's share of a band: pixel group g (4 pixels) of band rows r0,
// r0 + step, ... below `rows`.
template <int C>
__device__ __forceinline__ void stage_rows(uint32_t *band, const SourceWindow &w, int64_t row_bytes,
                                           int r0, int step, int rows, int last_row, int g, int pitch) {
    const uint32_t col_bytes = w.lead + uint32_t(g * 4 * C);
    for (int r = r0; r < rows; r += kStageBatch * step) {
        RowBatch b;
        issue_rows<C>(b, w, row_bytes, col_bytes, r, step, rows, last_row);
        write_rows<C>(band, b, r, step, rows, g, pitch);
    }
}

// Stages source rows [r_lo, r_lo + rows) x columns [c_lo, c_lo + 4*groups)
// into LDS, one dword per pixel.  Rows past the last image row repeat it;
// a column past the last image column is patched afterwards.
__device__ __forceinline__ void stage_band(uint32_t *band, const PreArgs &a, const DevImage &d,
                                           int64_t frame_offset, int r_lo, int c_lo, int rows,
                                           int groups, int pitch) {
    const int C = d.channels;
    const int64_t row_bytes = int64_t(d.src_w) * C;
    const uint64_t first = reinterpret_cast<uint64_t>(a.src) + uint64_t(frame_offset) +
                           uint64_t(int64_t(r_lo) * row_bytes + int64_t(c_lo) * C);
    const SourceWindow w = source_window(a, first);
    const int last_row = d.src_h - 1 - r_lo;  // band row of the image's last row
    const int nthreads = blockDim.x;
    if (groups <= nthreads) {
        // thread -> (row phase, group) once; rows advance by nthreads / groups
        const int step = nthreads / groups;
        const int r0 = div_small(threadIdx.x, groups, 1.0f / float(groups));
        const int g = threadIdx.x - r0 * groups;
        if (r0 < step) {
            if (C == 3)
                stage_rows<3>(band, w, row_bytes, r0, step, rows, last_row, g, pitch);
            else
                stage_rows<4>(band, w, row_bytes, r0, step, rows, last_row, g, pitch);
        }
    } else {
        for (int i = threadIdx.x; i < rows * groups; i += nthreads) {
            const int r = i / groups;
            const int g = i - r * groups;
            const int sr = min(r, last_row);
            uint32_t p[4];
            load_4px(w, w.lead + uint32_t(int64_t(sr) * row_bytes) + uint32_t(g * 4 * C), C, p);
            const u32x4 o = {p[0], p[1], p[2], p[3]};
            *reinterpret_cast<u32x4 *>(band + r * pitch + 4 * g) = o;
        }
    }
}

// What one workgroup's tile covers: temporal patch t, block row br, rows
// [first, first + count) of that block row (merge order) or of its column-
// order unit, and the output pixel rectangle those rows cover.
struct TileGeom {
    int t, br, first, count;
    int oy_first, oy_last, ox_first, ox_last;
};

// Source band touched by a tile: taps are monotone in the output index, so
// the first and last output rows/columns bound it.  The band runs one past
// the last first-tap so that the second tap is always i0 + 1; at the image
// edge that row/column repeats the last one.
struct Band {
    int r_lo, c_lo, c_end, rows, groups, pitch;
    bool fits;  // the band fits the LDS
};

__device__ __forceinline__ Band tile_band(const PreArgs &a, const DevImage &d, const TileGeom &g) {
    Band b;
    b.r_lo = make_tap(d.scale_y, g.oy_first, d.src_h).i0;
    const int r_end = make_tap(d.scale_y, g.oy_last, d.src_h).i0 + 1;
    b.c_lo = make_tap(d.scale_x, g.ox_first, d.src_w).i0;
    b.c_end = make_tap(d.scale_x, g.ox_last, d.src_w).i0 + 1;
    b.rows = r_end - b.r_lo + 1;
    b.groups = (b.c_end - b.c_lo + 4) >> 2;
    b.pitch = 4 * (b.groups | 1);  // an odd number of 16-byte groups spreads rows over the banks
    b.fits = int64_t(b.rows) * b.pitch <= a.band_capacity &&
             int64_t(b.rows) * d.src_w * d.channels < 0x7FFF0000ll;
    return b;
}

// At the right image edge the band's last column is the second tap of the
// last first-tap: repeat the image's last column there.
__device__ __forceinline__ void replicate_right_edge(uint32_t *band, const DevImage &d, const Band &b) {
    const int xl = d.src_w - 1 - b.c_lo;
    for (int r = threadIdx.x; r < b.rows; r += blockDim.x)
        band[r * b.pitch + xl + 1] = band[r * b.pitch + xl];
}

// The x taps of the tile's output columns into the table that follows the
// band in LDS (the band's first column c_lo as origin); made before the
// band's barrier.
template <bool kYTab>
__device__ __forceinline__ BandPixels band_pixels(uint32_t *band, const PreArgs &a, const DevImage &d,
                                                  const TileGeom &g, const Band &b) {
    BandPixels px;
    px.band = band;
    px.pitch = b.pitch;
    px.r_lo = b.r_lo;
    px.c_lo = b.c_lo;
    int32_t *xi = reinterpret_cast<int32_t *>(band + a.band_capacity);
    float *xl0 = reinterpret_cast<float *>(xi + kMaxTileCols);
    float *xl1 = xl0 + kMaxTileCols;
    for (int i = threadIdx.x; i <= g.ox_last - g.ox_first; i += blockDim.x) {
        const Tap tx = make_tap(d.scale_x, g.ox_first + i, d.src_w);
        xi[i] = tx.i0 - b.c_lo;
        xl0[i] = tx.l0;
        xl1[i] = tx.l1;
    }
    px.xi = xi;
    px.xl0 = xl0;
    px.xl1 = xl1;
    px.ox_first = g.ox_first;
    px.yt = nullptr;
    px.oy_first = g.oy_first;
    if (kYTab) {
        i32x4 *yt = reinterpret_cast<i32x4 *>(xl1 + kMaxTileCols);  // 16-byte aligned
        for (int i = threadIdx.x; i <= g.oy_last - g.oy_first; i += blockDim.x) {
            const Tap ty = make_tap(d.scale_y, g.oy_first + i, d.src_h);
            const int r0 = __mul24(ty.i0 - b.r_lo, b.pitch);
            yt[i] = i32x4{r0, r0 + b.pitch, __builtin_bit_cast(int32_t, ty.l0), __builtin_bit_cast(int32_t, ty.l1)};
        }
        px.yt = yt;
    }
    return px;
}

// Resamples one source frame (at frame_offset) of the tile into temporal
// slot TT of its rows (both slots when TT < 0).
template <typename OutT, int TT, bool kYTab>
__device__ __forceinline__ void tile_pass(const PreArgs &a, const DevImage &d, const TileGeom &g,
                                          int64_t frame_offset, OutT *out, bool column,
                                          uint32_t *band) {
    // the wave index as a scalar: a row's tile coordinates and output
    // address are then the same in every lane, formed on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int waves = blockDim.x >> 6;
    if (d.flags & kFlagIdentity) {
        const int64_t row_bytes = int64_t(d.src_w) * d.channels;
        const uint64_t first_byte = reinterpret_cast<uint64_t>(a.src) + uint64_t(frame_offset) +
                                    uint64_t(int64_t(g.oy_first) * row_bytes +
                                             int64_t(g.ox_first) * d.channels);
        const SourceWindow w = source_window(a, first_byte);
        for (int p = wave; p < g.count; p += waves) {
            const int qr = g.first + p;  // row within the block row: (block col, mh, mw)
            identity_patch<OutT, TT>(a, d, w, row_bytes, g.oy_first, g.ox_first, g.t, g.br, qr >> 2,
                                     (qr >> 1) & 1, qr & 1, out, column);
        }
        return;
    }

    const Band b = tile_band(a, d, g);
    if (b.fits) {
        const BandPixels px = band_pixels<kYTab>(band, a, d, g, b);
        stage_band(band, a, d, frame_offset, b.r_lo, b.c_lo, b.rows, b.groups, b.pitch);
        __syncthreads();
        if (b.c_end == d.src_w) {
            replicate_right_edge(band, d, b);
            __syncthreads();
        }
        for (int p = wave; p < g.count; p += waves) {
            const int qr = g.first + p;
            bilinear_patch_band<OutT, TT, kYTab>(px, d, a, g.t, g.br, qr >> 2, (qr >> 1) & 1, qr & 1, out, column);
        }
    } else {
        const GlobalPixels px{a.src + frame_offset, int64_t(d.src_w) * d.channels, d.channels,
                              d.src_h, d.src_w};
        for (int p = wave; p < g.count; p += waves) {
            const int qr = g.first + p;
            bilinear_patch<OutT, TT>(px, d, a, g.t, g.br, qr >> 2, (qr >> 1) & 1, qr & 1, out, column);
        }
    }
}

// Two distinct frames of a clip tile whose band fits the LDS and whose band
// row has no more 4-pixel groups than the workgroup has threads: frame 1's
// first batch of band loads goes out before frame 0 is resampled, so that
// its latency is spent there.
template <typename OutT, int C, bool kYTab>
__device__ __forceinline__ void clip_pair_pass(const PreArgs &a, const DevImage &d, const TileGeom &g,
                                               const Band &b, int64_t off0, int64_t off1, OutT *out,
                                               bool column, uint32_t *band) {
    const int64_t row_bytes = int64_t(d.src_w) * C;
    const uint64_t lead = uint64_t(int64_t(b.r_lo) * row_bytes + int64_t(b.c_lo) * C);
    const uint64_t base = reinterpret_cast<uint64_t>(a.src);
    const SourceWindow w0 = source_window(a, base + uint64_t(off0) + lead);
    const SourceWindow w1 = source_window(a, base + uint64_t(off1) + lead);
    const int last_row = d.src_h - 1 - b.r_lo;
    const int step = blockDim.x / b.groups;
    const int r0 = div_small(threadIdx.x, b.groups, 1.0f / float(b.groups));
    const int gi = threadIdx.x - r0 * b.groups;
    const bool active = r0 < step;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)), waves = blockDim.x >> 6;
    const BandPixels px = band_pixels<kYTab>(band, a, d, g, b);
    RowBatch next;
    if (active) {
        stage_rows<C>(band, w0, row_bytes, r0, step, b.rows, last_row, gi, b.pitch);
        issue_rows<C>(next, w1, row_bytes, w1.lead + uint32_t(gi * 4 * C), r0, step, b.rows, last_row);
    }
    __syncthreads();
    if (b.c_end == d.src_w) {
        replicate_right_edge(band, d, b);
        __syncthreads();
    }
    for (int p = wave; p < g.count; p += waves) {
        const int qr = g.first + p;
        bilinear_patch_band<OutT, 0, kYTab>(px, d, a, g.t, g.br, qr >> 2, (qr >> 1) & 1, qr & 1, out, column);
    }
    __syncthreads();  // the first frame's band is no longer read
    if (active) {
        write_rows<C>(band, next, r0, step, b.rows, gi, b.pitch);
        const uint32_t col_bytes = w1.lead + uint32_t(gi * 4 * C);
        for (int r = r0 + kStageBatch * step; r < b.rows; r += kStageBatch * step) {
            RowBatch rb;
            issue_rows<C>(rb, w1, row_bytes, col_bytes, r, step, b.rows, last_row);
            write_rows<C>(band, rb, r, step, b.rows, gi, b.pitch);
        }
    }
    __syncthreads();
    if (b.c_end == d.src_w) {
        replicate_right_edge(band, d, b);
        __syncthreads();
    }
    for (int p = wave; p < g.count; p += waves) {
        const int qr = g.first + p;
        bilinear_patch_band<OutT, 1, kYTab>(px, d, a, g.t, g.br, qr >> 2, (qr >> 1) & 1, qr & 1, out, column);
    }
}

// kClips: the batch holds at least one clip (an item with two or more
// frames); batches of still images compile without the temporal decode.
// The clip instance is built for at least 6 waves per SIMD: a clip tile's
// band typically holds a CU to 6 workgroups (25 KB for 1280x720 frames at
// 960x512), and its pair path would otherwise take more registers than that
// occupancy leaves.  The stills instance is built for the full 8, which it
// reaches with no spill and no added instruction in its resample loop.
// kInline: the descriptor tables are in the kernel arguments (batches of at
// most kInlineImages images); a separate instance, since code that could
// take either source keeps the record in vector registers and spills.
template <typename OutT, bool kClips, bool kInline>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kClips ? 6 : 8))) void preprocess_kernel(PreArgs a) {
    extern __shared__ uint32_t band[];
    const int64_t u = a.xcd_order ? xcd_contiguous_tile(blockIdx.x, gridDim.x) : int64_t(blockIdx.x);
    // Pass 0 writes merge-block order (if requested), pass 1 column order:
    // each workgroup writes one output, in that output's own order.
    const bool second = u >= a.tiles_per_pass;
    const int64_t tile = second ? u - a.tiles_per_pass : u;
    const int img = tile_image<kInline>(a, tile);
    int local = int(tile - tile_begin_at<kInline>(a, img));  // the tile's index within its image and pass
    const bool column = second || a.rows == nullptr;
    OutT *const out = static_cast<OutT *>(column ? a.rows_col : a.rows);
    const DevImage d = image_at<kInline>(a, img);
    TileGeom g;
    // temporal patch t of a clip: tiles are listed slice by slice
    g.t = 0;
    if (kClips && d.frames > kTemporal) {
        const int per_slice = d.blocks_h * d.tiles_per_brow;
        g.t = div_small(local, per_slice, 1.0f / float(per_slice));
        local -= g.t * per_slice;
    }
    const int R = a.rows_per_tile;
    if (!column) {
        g.br = div_small(local, d.tiles_per_brow, d.inv_tiles_per_brow);
        g.first = (local - g.br * d.tiles_per_brow) * R;  // first row within the block row
        g.count = min(R, d.blocks_w * kRowsPerUnit - g.first);
    } else {
        // column order lists units by (block col, block row); R <= 4 divides
        // a unit, so a tile is part of one unit
        const int rc = local * R;
        const int unit = rc >> 2;
        const int bc = div_small(unit, d.blocks_h, d.inv_blocks_h);
        g.br = unit - bc * d.blocks_h;
        g.first = bc * kRowsPerUnit + (rc & 3);
        g.count = R;
    }

    // Output rectangle of the tile: whole merge units when R >= 4, else one
    // patch row (mh fixed) of one unit, one or both of its patches.
    if (R >= kRowsPerUnit) {
        g.oy_first = g.br * kUnitPx;
        g.oy_last = g.oy_first + kUnitPx - 1;
        g.ox_first = (g.first >> 2) * kUnitPx;
        g.ox_last = ((g.first + g.count - 1) >> 2) * kUnitPx + kUnitPx - 1;
    } else {
        const int mh = (g.first >> 1) & 1;
        g.oy_first = (g.br * kMerge + mh) * kPatch;
        g.oy_last = g.oy_first + kPatch - 1;
        const int bc = g.first >> 2;
        g.ox_first = (bc * kMerge + (g.first & 1)) * kPatch;
        g.ox_last = (bc * kMerge + ((g.first + g.count - 1) & 1)) * kPatch + kPatch - 1;
    }

    // Temporal slot tt of patch t shows frame min(2t + tt, frames - 1): an
    // odd frame count repeats its last frame, a still image is two copies of
    // its one frame.  Identical frames are computed once and stored to both
    // slots; distinct frames take one pass per slot.
    if (!kClips) {
        tile_pass<OutT, -1, false>(a, d, g, d.src_offset, out, column, band);
        return;
    }
    const int64_t frame_bytes = int64_t(d.src_h) * d.src_w * d.channels;
    const int f0 = min(kTemporal * g.t, d.frames - 1);
    const int f1 = min(kTemporal * g.t + 1, d.frames - 1);
    const int64_t off0 = d.src_offset + int64_t(f0) * frame_bytes;
    if (f0 == f1) {
        tile_pass<OutT, -1, true>(a, d, g, off0, out, column, band);
    } else {
        const int64_t off1 = d.src_offset + int64_t(f1) * frame_bytes;
        if (!(d.flags & kFlagIdentity)) {
            const Band b = tile_band(a, d, g);
            if (b.fits && b.groups <= int(blockDim.x)) {
                if (d.channels == 3)
                    clip_pair_pass<OutT, 3, true>(a, d, g, b, off0, off1, out, column, band);
                else
                    clip_pair_pass<OutT, 4, true>(a, d, g, b, off0, off1, out, column, band);
                return;
            }
        }
        tile_pass<OutT, 0, true>(a, d, g, off0, out, column, band);
        __syncthreads();  // the first frame's band is no longer read
        tile_pass<OutT, 1, true>(a, d, g, off1, out, column, band);
    }
}

// Column-order gather: one workgroup copies one merge unit (4 contiguous
// rows) from its merge-order position to its column-order position, one
// wavefront per row; units go to XCDs in contiguous runs, as the fused
// kernel's tiles do (4.55 ms for 2 x 12.9 GB, against 4.93 ms for a
// wavefront per unit in dispatch order with one load in flight).
template <typename OutT>
__global__ __launch_bounds__(kThreads) void column_permute_kernel(PermArgs a) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t unit = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    if (unit >= a.total_units) return;  // workgroup-uniform
    const int64_t drow = unit * kRowsPerUnit;
    const int img = find_segment(a.row_begin, a.n, drow);
    const DevImage d = a.images[img];
    const int units = d.blocks_h * d.blocks_w;  // per temporal patch
    const int ju = int((drow - d.row_offset) / kRowsPerUnit);  // column-order unit index
    const int t = ju / units;
    const int j = ju - t * units;
    const int bc = div_small(j, d.blocks_h, d.inv_blocks_h);
    const int br = j - bc * d.blocks_h;
    const int64_t src_row =
        d.row_offset + (int64_t(t) * units + int64_t(br) * d.blocks_w + bc) * kRowsPerUnit;
    static_assert(kWaves == kRowsPerUnit, "one wavefront per row of the unit");
    constexpr int kPerLane = kRowLen * int(sizeof(OutT)) / 16 / 64;  // 16-byte vectors: 6 (fp32) or 3 (bf16)
    const u32x4 *in = reinterpret_cast<const u32x4 *>(static_cast<const OutT *>(a.in) + (src_row + wave) * kRowLen);
    u32x4 *out = reinterpret_cast<u32x4 *>(static_cast<OutT *>(a.out) + (drow + wave) * kRowLen);
    // All of the row's loads go out before any store: the compiler cannot
    // move a load above a store to `out` (it may alias `in`), so a plain
    // load-store loop would keep one load in flight.
    u32x4 v[kPerLane];
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) v[k] = __builtin_nontemporal_load(in + k * 64 + lane);
#pragma unroll
    for (int k = 0; k < kPerLane; ++k) __builtin_nontemporal_store(v[k], out + k * 64 + lane);
}

// ------------------------------------------------------------- host side

// Conservative size of the LDS band one tile of R rows needs, in dwords.
int64_t band_estimate(const DevImage &d, int R) {
    const int out_rows = R >= kRowsPerUnit ? kUnitPx : kPatch;
    const int out_cols = R >= kRowsPerUnit ? kUnitPx * (R / kRowsPerUnit) : kPatch * R;
    if (d.flags & kFlagIdentity) return int64_t(out_rows) * (4 * ((out_cols + 3) / 4));
    const double rows = std::min<double>(d.src_h, std::ceil((out_rows - 1.0) * d.scale_y) + 4.0);
    const double cols = std::min<double>(d.src_w, std::ceil((out_cols - 1.0) * d.scale_x) + 4.0);
    return int64_t(rows) * (4 * ((int64_t(cols) + 3) / 4 + 1));
}

// Builds the workspace image -- DevImage records, tile prefix, row prefix --
// into `bytes` (ws_total_bytes(n) bytes, zeroed by the caller).
int build_tables_into(int32_t n, const mimo_image_desc *desc, const Tiling &tiling, uint8_t *bytes,
                      BuiltTables &out) {
    DevImage *img = reinterpret_cast<DevImage *>(bytes);
    int64_t *tile_begin = reinterpret_cast<int64_t *>(bytes + ws_images_bytes(n));
    int64_t *row_begin = reinterpret_cast<int64_t *>(bytes + ws_images_bytes(n) + ws_prefix_bytes(n));
    const int R = tiling.rows_per_tile;
    int64_t tiles = 0, rows = 0, band = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mimo_image_desc &s = desc[i];
        DevImage d;
        std::memset(&d, 0, sizeof(d));
        tile_begin[i] = tiles;
        row_begin[i] = rows;
        d.src_offset = s.src_offset;
        d.row_offset = rows;
        d.tiles_per_brow = 1;
        if (s.status != MIMO_OK || s.rows == 0) {
            img[i] = d;
            continue;
        }
        if (s.src_h < 1 || s.src_w < 1 || (s.channels != 3 && s.channels != 4) || s.frames < 1 ||
            s.dst_h < kUnitPx || s.dst_w < kUnitPx || s.dst_h % kUnitPx || s.dst_w % kUnitPx ||
            s.grid_t != (s.frames + kTemporal - 1) / kTemporal || s.grid_h * kPatch != s.dst_h ||
            s.grid_w * kPatch != s.dst_w ||
            s.rows != int64_t(s.grid_t) * s.grid_h * s.grid_w || s.rows > kMaxRowsPerImage ||
            s.row_offset != rows || s.src_offset < 0)
            return set_error(MIMO_E_INVALID, "descriptor " + std::to_string(i) +
                                                 " is not a plan of the 16/2/2 kernels");
        if (s.src_h > kMaxSide || s.src_w > kMaxSide || s.dst_h > kMaxSide || s.dst_w > kMaxSide)
            return set_error(MIMO_E_TOO_LARGE, "descriptor " + std::to_string(i) + ": side too large");
        d.src_h = s.src_h;
        d.src_w = s.src_w;
        d.channels = s.channels;
        d.frames = s.frames;
        out.clips = out.clips || s.frames > 1;
        d.blocks_h = s.dst_h / kUnitPx;
        d.blocks_w = s.dst_w / kUnitPx;
        d.scale_y = float(s.src_h) / float(s.dst_h);
        d.scale_x = float(s.src_w) / float(s.dst_w);
        d.flags = (s.src_h == s.dst_h && s.src_w == s.dst_w) ? kFlagIdentity : 0;
        const int64_t est = band_estimate(d, R);
        if (est <= kBandBudgetDwords) band = std::max(band, est);  // else: direct reads
        const int64_t brow_rows = int64_t(d.blocks_w) * kRowsPerUnit;
        d.tiles_per_brow = int32_t((brow_rows + R - 1) / R);
        d.inv_tiles_per_brow = 1.0f / float(d.tiles_per_brow);
        d.inv_blocks_h = 1.0f / float(d.blocks_h);
        img[i] = d;
        tiles += int64_t(s.grid_t) * d.blocks_h * d.tiles_per_brow;
        rows += s.rows;
    }
    tile_begin[n] = tiles;
    row_begin[n] = rows;
    out.total_tiles = tiles;
    out.total_rows = rows;
    out.band_capacity = int32_t((std::max<int64_t>(band, 4) + 3) & ~int64_t(3));  // the x-tap table follows, 16-byte aligned
    return MIMO_OK;
}

// The same, into out.bytes.
int build_tables(int32_t n, const mimo_image_desc *desc, const Tiling &tiling, BuiltTables &out) {
    out.bytes.assign(ws_total_bytes(n), 0);
    return build_tables_into(n, desc, tiling, out.bytes.data(), out);
}

// ------------------------------------------- allocation-free entry point

// Device scratch of mimo_preprocess_batch_noalloc: the descriptor tables of
// one call (at most MIMO_NOALLOC_MAX_IMAGES images), one copy per GPU, held
// until the process ends.  Host code never uses this name as an address
// (on the host it is only a stand-in for the symbol): each device's copy is
// reached through the pointer hipGetSymbolAddress returns for it.
constexpr size_t kNoAllocScratchBytes = ws_total_bytes_const(MIMO_NOALLOC_MAX_IMAGES);
static_assert(kNoAllocScratchBytes == MIMO_NOALLOC_SCRATCH_BYTES, "scratch size as declared");
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// One piece of a descriptor table carried in a kernel's arguments: the host
// hands the tables over with no staging buffer of its own.
constexpr int kChunkWords = 768;  // 3 KB per launch
struct TableChunk {
    uint32_t *dst;
    uint32_t words;  // <= kChunkWords
    uint32_t pad;
    uint32_t data[kChunkWords];
};

__global__ __launch_bounds__(256) void table_fill_kernel(TableChunk c) {
    for (uint32_t i = threadIdx.x; i < c.words; i += blockDim.x) c.dst[i] = c.data[i];
}

// The device address of this device's scratch, looked up once per device
// (with that device current) and kept.
hipError_t scratch_address(uint8_t **out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = static_cast<uint8_t *>(addr[dev]);
    return hipSuccess;
}

// Copies `bytes` (a multiple of 4) from host memory to device memory on
// `stream` through the arguments of table_fill_kernel launches.
hipError_t fill_by_arguments(const uint8_t *host, size_t bytes, uint8_t *dev, hipStream_t stream) {
    TableChunk c;
    c.pad = 0;
    for (size_t off = 0; off < bytes; off += 4 * size_t(kChunkWords)) {
        c.words = uint32_t(std::min<size_t>(kChunkWords, (bytes - off) / 4));
        c.dst = reinterpret_cast<uint32_t *>(dev + off);
        std::memcpy(c.data, host + off, 4 * size_t(c.words));
        hipLaunchKernelGGL(table_fill_kernel, dim3(1), dim3(256), 0, stream, c);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

namespace {

// Where a call's descriptor tables go: the caller's workspace, uploaded
// through the pinned staging ring, or this device's scratch, filled through
// kernel arguments.
enum class TableHome { kWorkspace, kScratch };

int preprocess_common(const char *who, int32_t n, const mimo_image_desc *desc, const uint8_t *src,
                      int64_t src_capacity, const float *mean255, const float *std255,
                      int32_t out_dtype, void *rows, void *rows_col, int64_t capacity_rows,
                      void *workspace, size_t workspace_bytes, void *stream, TableHome home) {
    const std::string w(who);
    if (n < 0 || (n > 0 && !desc) || !mean255 || !std255)
        return set_error(MIMO_E_INVALID, w + ": bad n or null pointer");
    if (home == TableHome::kScratch && n > MIMO_NOALLOC_MAX_IMAGES)
        return set_error(MIMO_E_CAPACITY, w + ": " + std::to_string(n) + " images, above the scratch's " +
                                              std::to_string(MIMO_NOALLOC_MAX_IMAGES));
    if (out_dtype != MIMO_F32 && out_dtype != MIMO_BF16)
        return set_error(MIMO_E_INVALID, w + ": out_dtype must be MIMO_F32 or MIMO_BF16");
    if (!rows && !rows_col)
        return set_error(MIMO_E_INVALID, w + ": both outputs are null");
    if ((rows && !check_ptr_align(rows, 16)) || (rows_col && !check_ptr_align(rows_col, 16)))
        return set_error(MIMO_E_INVALID, w + ": outputs must be 16-byte aligned");
    if (n == 0) return MIMO_OK;
    if (!src || !check_ptr_align(src, 4))
        return set_error(MIMO_E_INVALID, w + ": src must be non-null and 4-byte aligned");
    if (home == TableHome::kWorkspace) {
        if (!workspace || !check_ptr_align(workspace, 16))
            return set_error(MIMO_E_INVALID, w + ": workspace must be non-null and 16-byte aligned");
        if (workspace_bytes < ws_total_bytes(n))
            return set_error(MIMO_E_CAPACITY, w + ": workspace smaller than mimo_workspace_bytes(n)");
    }
    PreArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int c = 0; c < 3; ++c) {
        if (!(std255[c] > 0.0f) || !std::isfinite(std255[c]) || !std::isfinite(mean255[c]))
            return set_error(MIMO_E_INVALID, w + ": std255 must be > 0 and finite");
        a.inv_std[c] = float(1.0 / double(std255[c]));
        a.mean[c] = mean255[c];
    }
    bool clips = false;
    for (int32_t i = 0; i < n; ++i) clips = clips || (desc[i].status == MIMO_OK && desc[i].frames > 1);
    const Tiling tiling = Tiling::choose(rows != nullptr, rows_col != nullptr, clips);
    // The tables are built on the host: into a vector for the workspace
    // path; for the scratch path into a static host buffer (held under its
    // lock until the launches that carry it have been issued), so that the
    // call allocates nothing.
    static std::mutex host_mu;
    static uint8_t host_tables[kNoAllocScratchBytes];
    std::unique_lock<std::mutex> host_lock(host_mu, std::defer_lock);
    BuiltTables t;
    const uint8_t *table = nullptr;
    int st;
    if (home == TableHome::kScratch) {
        host_lock.lock();
        std::memset(host_tables, 0, ws_total_bytes(n));
        st = build_tables_into(n, desc, tiling, host_tables, t);
        table = host_tables;
    } else {
        st = build_tables(n, desc, tiling, t);
        table = t.bytes.data();
    }
    if (st != MIMO_OK) return st;
    int64_t src_needed = 0;
    for (int32_t i = 0; i < n; ++i)
        if (desc[i].status == MIMO_OK && desc[i].rows > 0)
            src_needed = std::max<int64_t>(src_needed, desc[i].src_offset +
                                                           int64_t(desc[i].frames) * desc[i].src_h *
                                                               desc[i].src_w * desc[i].channels);
    if (src_capacity < ((src_needed + 15) & ~int64_t(15)))
        return set_error(MIMO_E_CAPACITY, w + ": src_capacity below the packed size rounded up to 16");
    if (t.total_rows > capacity_rows)
        return set_error(MIMO_E_CAPACITY, w + ": capacity_rows " + std::to_string(capacity_rows) +
                                              " < " + std::to_string(t.total_rows) + " rows");
    if (t.total_tiles == 0) return MIMO_OK;
    if (t.total_tiles * tiling.passes > 0x7FFFFFFFll)
        return set_error(MIMO_E_TOO_LARGE, w + ": more than 2^31-1 tiles");

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (n <= kInlineImages) {
        // small batch: the tables travel in the kernel arguments
        std::memcpy(a.inl_images, table, sizeof(DevImage) * size_t(n));
        std::memcpy(a.inl_tile_begin, table + ws_images_bytes(n), sizeof(int64_t) * (size_t(n) + 1));
        a.images = nullptr;
        a.tile_begin = nullptr;
    } else {
        uint8_t *ws = nullptr;
        if (home == TableHome::kScratch) {
            e = scratch_address(&ws);
            if (e != hipSuccess) return hip_error(e, (w + ": scratch address").c_str());
            e = fill_by_arguments(table, ws_total_bytes(n), ws, s);
        } else {
            ws = static_cast<uint8_t *>(workspace);
            e = upload_table(table, ws_total_bytes(n), ws, s);
        }
        if (e != hipSuccess) return hip_error(e, (w + ": table upload").c_str());
        a.images = reinterpret_cast<const DevImage *>(ws);
        a.tile_begin = reinterpret_cast<const int64_t *>(ws + ws_images_bytes(n));
    }

    a.src = src;
    a.src_end = src_capacity;
    a.rows = rows;
    a.rows_col = rows_col;
    a.n = n;
    a.band_capacity = t.band_capacity;
    a.rows_per_tile = tiling.rows_per_tile;
    a.xcd_order = tiling.xcd_order;
    a.tiles_per_pass = rows ? t.total_tiles : int64_t(1) << 62;
    // band, then the x-tap table, then (clip instance) the y-tap table
    const size_t lds = (size_t(t.band_capacity) + 3 * kMaxTileCols + (t.clips ? 4 * kMaxTileRows : 0)) * 4;
    const dim3 grid{unsigned(t.total_tiles * tiling.passes), 1, 1},
        block{unsigned(tiling.threads()), 1, 1};
    const bool inl = n <= kInlineImages;
    e = timed_launch(s, [&] {
#define MIMO_LAUNCH(T, C)                                                                   \
    do {                                                                                    \
        if (inl)                                                                            \
            hipLaunchKernelGGL((preprocess_kernel<T, C, true>), grid, block, lds, s, a);    \
        else                                                                                \
            hipLaunchKernelGGL((preprocess_kernel<T, C, false>), grid, block, lds, s, a);   \
    } while (0)
        if (out_dtype == MIMO_F32) {
            if (t.clips)
                MIMO_LAUNCH(float, true);
            else
                MIMO_LAUNCH(float, false);
        } else {
            if (t.clips)
                MIMO_LAUNCH(uint16_t, true);
            else
                MIMO_LAUNCH(uint16_t, false);
        }
#undef MIMO_LAUNCH
    });
    if (e != hipSuccess) return hip_error(e, (w + ": kernel launch").c_str());
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

}  // namespace
}  // namespace mimo

using namespace mimo;

extern "C" {

int mimo_preprocess_batch(int32_t n, const mimo_image_desc *desc, const uint8_t *src,
                          int64_t src_capacity, const float *mean255, const float *std255,
                          int32_t out_dtype, void *rows, void *rows_col, int64_t capacity_rows,
                          void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    return preprocess_common("preprocess_batch", n, desc, src, src_capacity, mean255, std255, out_dtype,
                             rows, rows_col, capacity_rows, workspace, workspace_bytes, stream,
                             TableHome::kWorkspace);
}

int mimo_preprocess_batch_noalloc(int32_t n, const mimo_image_desc *desc, const uint8_t *src,
                                  int64_t src_capacity, const float *mean255, const float *std255,
                                  int32_t out_dtype, void *rows, void *rows_col, int64_t capacity_rows,
                                  void *stream) {
    clear_error();
    return preprocess_common("preprocess_batch_noalloc", n, desc, src, src_capacity, mean255, std255,
                             out_dtype, rows, rows_col, capacity_rows, nullptr, 0, stream,
                             TableHome::kScratch);
}

int mimo_column_permute(int32_t n, const mimo_image_desc *desc, const void *rows_in,
                        void *rows_out, int32_t out_dtype, int64_t capacity_rows,
                        void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    if (n < 0 || (n > 0 && !desc))
        return set_error(MIMO_E_INVALID, "column_permute: bad n or null pointer");
    if (out_dtype != MIMO_F32 && out_dtype != MIMO_BF16)
        return set_error(MIMO_E_INVALID, "column_permute: out_dtype must be MIMO_F32 or MIMO_BF16");
    if (n == 0) return MIMO_OK;
    if (!rows_in || !rows_out || rows_in == rows_out || !check_ptr_align(rows_in, 16) ||
        !check_ptr_align(rows_out, 16))
        return set_error(MIMO_E_INVALID, "column_permute: need distinct 16-byte aligned buffers");
    if (!workspace || !check_ptr_align(workspace, 16))
        return set_error(MIMO_E_INVALID, "column_permute: workspace must be non-null and 16-byte aligned");
    if (workspace_bytes < ws_total_bytes(n))
        return set_error(MIMO_E_CAPACITY, "column_permute: workspace smaller than mimo_workspace_bytes(n)");
    BuiltTables t;
    int st = build_tables(n, desc, Tiling(), t);
    if (st != MIMO_OK) return st;
    if (t.total_rows > capacity_rows)
        return set_error(MIMO_E_CAPACITY, "column_permute: capacity_rows below the total rows");
    if (t.total_rows == 0) return MIMO_OK;
    const int64_t units = t.total_rows / kRowsPerUnit;
    const int64_t blocks = units;
    if (blocks > 0x7FFFFFFFll)
        return set_error(MIMO_E_TOO_LARGE, "column_permute: too many merge units");

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = upload_table(t.bytes.data(), t.bytes.size(), workspace, s);
    if (e != hipSuccess) return hip_error(e, "column_permute: table upload");
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    PermArgs a;
    a.images = reinterpret_cast<const DevImage *>(ws);
    a.row_begin = reinterpret_cast<const int64_t *>(ws + ws_images_bytes(n) + ws_prefix_bytes(n));
    a.in = rows_in;
    a.out = rows_out;
    a.total_units = units;
    a.n = n;
    const dim3 grid{unsigned(blocks), 1, 1}, block{unsigned(kThreads), 1, 1};
    e = timed_launch(s, [&] {
        if (out_dtype == MIMO_F32)
            hipLaunchKernelGGL(column_permute_kernel<float>, grid, block, 0, s, a);
        else
            hipLaunchKernelGGL(column_permute_kernel<uint16_t>, grid, block, 0, s, a);
    });
    if (e != hipSuccess) return hip_error(e, "column_permute: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

}  // extern "C"
