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

#include "internal.h"

namespace mimo {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// LDS budget for one tile's source band, in dwords (one dword per pixel).
constexpr int kBandBudgetDwords = 12288;  // 48 KB
constexpr int kMaxUnitsPerTile = 4;
// Buffer resource word 3 for raw (untyped) buffer loads on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;

struct PreArgs {
    const uint8_t *src;
    const DevImage *images;
    const int64_t *tile_begin;  // [n + 1]
    void *rows;                 // merge-block order, nullable
    void *rows_col;             // column order, nullable
    int64_t src_end;            // bytes readable from src
    int32_t n;
    int32_t band_capacity;      // dwords of dynamic LDS
    float inv_std[3];           // 1 / std255, rounded once
    float mean[3];              // mean255
};

struct PermArgs {
    const DevImage *images;
    const int64_t *row_begin;  // [n + 1]
    const void *in;
    void *out;
    int64_t total_units;
    int32_t n;
};

// ---------------------------------------------------------------- helpers

// Largest i in [0, n) with begin[i] <= key (begin non-decreasing,
// begin[0] = 0 <= key).  Each round one wavefront compares 64 evenly spaced
// entries and keeps the bracket that holds the key.  Result is wave-uniform.
__device__ __forceinline__ int find_segment(const int64_t *__restrict__ begin, int n, int64_t key) {
    const int lane = threadIdx.x & 63;
    int lo = 0, hi = n;
    while (hi - lo > 1) {
        const int step = (hi - lo + 63) >> 6;
        const int idx = lo + lane * step;
        const bool le = idx < hi && begin[idx] <= key;
        const uint64_t mask = __ballot(le);
        const int k = __popcll(mask) - 1;
        lo = lo + k * step;
        hi = min(lo + step, hi);
    }
    return __builtin_amdgcn_readfirstlane(lo);
}

struct Tap {
    int i0, i1;
    float l0, l1;
};

// Half-pixel source taps for destination index d on an axis of n_in source
// samples (align_corners=False, clamped below at 0).
__device__ __forceinline__ Tap make_tap(float scale, int d, int n_in) {
    float s = __builtin_fmaf(scale, float(d) + 0.5f, -0.5f);
    s = s < 0.0f ? 0.0f : s;
    int i0 = int(s);  // s >= 0: truncation is floor
    i0 = i0 < n_in - 1 ? i0 : n_in - 1;
    Tap t;
    t.i0 = i0;
    t.i1 = i0 < n_in - 1 ? i0 + 1 : i0;
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

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {__bf16(lo), __bf16(hi)};  // hardware round-to-nearest-even
    return __builtin_bit_cast(uint32_t, v);
}

// Stores one lane's 4 consecutive values of channel c into both frames of a
// row.  row_ptr points at the row's element (py*16 + 4q).
template <typename OutT>
__device__ __forceinline__ void store_both_frames(OutT *row_ptr, int c, const float (&v)[4]);

template <>
__device__ __forceinline__ void store_both_frames<float>(float *row_ptr, int c, const float (&v)[4]) {
    const f32x4 q = {v[0], v[1], v[2], v[3]};
    float *p = row_ptr + c * (kTemporal * kPlane);
    __builtin_nontemporal_store(q, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store(q, reinterpret_cast<f32x4 *>(p + kPlane));
}

template <>
__device__ __forceinline__ void store_both_frames<uint16_t>(uint16_t *row_ptr, int c,
                                                            const float (&v)[4]) {
    const u32x2 q = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    uint16_t *p = row_ptr + c * (kTemporal * kPlane);
    __builtin_nontemporal_store(q, reinterpret_cast<u32x2 *>(p));
    __builtin_nontemporal_store(q, reinterpret_cast<u32x2 *>(p + kPlane));
}

// Pixel sources for the compute loop: LDS band or direct global reads.
struct LdsPixels {
    const uint32_t *band;
    int pitch, r_lo, c_lo;
    __device__ __forceinline__ uint32_t at(int y, int x) const {
        return band[(y - r_lo) * pitch + (x - c_lo)];
    }
};

struct GlobalPixels {
    const uint8_t *img;
    int64_t row_bytes;
    int channels;
    __device__ __forceinline__ uint32_t at(int y, int x) const {
        const uint8_t *p = img + int64_t(y) * row_bytes + int64_t(x) * channels;
        const uint32_t px = uint32_t(p[0]) | (uint32_t(p[1]) << 8) | (uint32_t(p[2]) << 16);
        return channels == 4 ? flatten_rgba(px | (uint32_t(p[3]) << 24)) : px;
    }
};

// Output rows one wavefront task writes: merge order and column order.
template <typename OutT>
struct RowSinks {
    OutT *merge;   // nullable
    OutT *column;  // nullable
};

// One wavefront computes output row (unit u of the tile, mh, mw): a 16x16
// patch, 3 channels, and stores it for both frames.
template <typename OutT, bool kIdentity, typename Pixels>
__device__ __forceinline__ void compute_patch(const Pixels &px, const DevImage &d, const PreArgs &a,
                                              int br, int bc, int mh, int mw, RowSinks<OutT> sinks) {
    const int lane = threadIdx.x & 63;
    const int py = lane >> 2;
    const int q = lane & 3;
    const int oy = (br * kMerge + mh) * kPatch + py;
    const int ox0 = (bc * kMerge + mw) * kPatch + 4 * q;

    float v[3][4];
    if constexpr (kIdentity) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t p = px.at(oy, ox0 + j);
#pragma unroll
            for (int c = 0; c < 3; ++c) v[c][j] = (chan(p, c) - a.mean[c]) * a.inv_std[c];
        }
    } else {
        const Tap ty = make_tap(d.scale_y, oy, d.src_h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const Tap tx = make_tap(d.scale_x, ox0 + j, d.src_w);
            const uint32_t p00 = px.at(ty.i0, tx.i0);
            const uint32_t p01 = px.at(ty.i0, tx.i1);
            const uint32_t p10 = px.at(ty.i1, tx.i0);
            const uint32_t p11 = px.at(ty.i1, tx.i1);
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                const float top = __builtin_fmaf(tx.l0, chan(p00, c), tx.l1 * chan(p01, c));
                const float bot = __builtin_fmaf(tx.l0, chan(p10, c), tx.l1 * chan(p11, c));
                const float val = __builtin_fmaf(ty.l0, top, ty.l1 * bot);
                v[c][j] = (val - a.mean[c]) * a.inv_std[c];
            }
        }
    }

    const int within = mh * kMerge + mw;
    const int elem = py * kPatch + 4 * q;
    if (sinks.merge) {
        const int64_t row = d.row_offset + int64_t(br * d.blocks_w + bc) * kRowsPerUnit + within;
        OutT *base = sinks.merge + row * kRowLen + elem;
#pragma unroll
        for (int c = 0; c < 3; ++c) store_both_frames<OutT>(base, c, v[c]);
    }
    if (sinks.column) {
        const int64_t row = d.row_offset + int64_t(bc * d.blocks_h + br) * kRowsPerUnit + within;
        OutT *base = sinks.column + row * kRowLen + elem;
#pragma unroll
        for (int c = 0; c < 3; ++c) store_both_frames<OutT>(base, c, v[c]);
    }
}

template <typename OutT, bool kIdentity, typename Pixels>
__device__ __forceinline__ void compute_tile(const Pixels &px, const DevImage &d, const PreArgs &a,
                                             int br, int bc0, int nb) {
    const int wave = threadIdx.x >> 6;
    RowSinks<OutT> sinks{static_cast<OutT *>(a.rows), static_cast<OutT *>(a.rows_col)};
    for (int p = wave; p < nb * kRowsPerUnit; p += kWaves) {
        const int u = p >> 2;
        compute_patch<OutT, kIdentity>(px, d, a, br, bc0 + u, (p >> 1) & 1, p & 1, sinks);
    }
}

// Copies source rows [r_lo, r_lo+rows) x columns [c_lo, c_lo + 4*groups) of
// one image into LDS as one dword per pixel (R | G<<8 | B<<16), flattening
// RGBA onto white.  Loads are dword-aligned 16-byte buffer loads (plus one
// dword for RGBA) realigned with v_alignbyte; reads past the buffer end
// return zero and only feed pixels outside the band.
__device__ __forceinline__ void stage_band(uint32_t *band, const PreArgs &a, const DevImage &d,
                                           int r_lo, int c_lo, int rows, int groups, int pitch) {
    const int C = d.channels;
    const int64_t row_bytes = int64_t(d.src_w) * C;
    const uint64_t first = reinterpret_cast<uint64_t>(a.src) + uint64_t(d.src_offset) +
                           uint64_t(int64_t(r_lo) * row_bytes + int64_t(c_lo) * C);
    const uint64_t base = first & ~uint64_t(3);
    const uint64_t end = reinterpret_cast<uint64_t>(a.src) + uint64_t(a.src_end);
    const uint64_t avail = end - base;
    const int num = avail > 0x7FFFFFF0ull ? 0x7FFFFFF0 : int(avail);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(base), 0, num, kBufferWord3);
    const uint32_t lead = uint32_t(first - base);
    const int total = rows * groups;
    for (int i = threadIdx.x; i < total; i += kThreads) {
        const int r = i / groups;
        const int g = i - r * groups;
        const uint32_t off = lead + uint32_t(int64_t(r) * row_bytes) + uint32_t(g * 4 * C);
        const uint32_t al = off & ~3u;
        const uint32_t sh = off & 3u;
        const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(al), 0, 0));
        uint32_t p0, p1, p2, p3;
        if (C == 3) {
            const uint32_t u0 = __builtin_amdgcn_alignbyte(w.y, w.x, sh);
            const uint32_t u1 = __builtin_amdgcn_alignbyte(w.z, w.y, sh);
            const uint32_t u2 = __builtin_amdgcn_alignbyte(w.w, w.z, sh);
            p0 = u0 & 0x00FFFFFFu;
            p1 = (u0 >> 24) | ((u1 & 0xFFFFu) << 8);
            p2 = (u1 >> 16) | ((u2 & 0xFFu) << 16);
            p3 = u2 >> 8;
        } else {
            const uint32_t w4 = __builtin_amdgcn_raw_buffer_load_b32(rsrc, int(al) + 16, 0, 0);
            p0 = flatten_rgba(__builtin_amdgcn_alignbyte(w.y, w.x, sh));
            p1 = flatten_rgba(__builtin_amdgcn_alignbyte(w.z, w.y, sh));
            p2 = flatten_rgba(__builtin_amdgcn_alignbyte(w.w, w.z, sh));
            p3 = flatten_rgba(__builtin_amdgcn_alignbyte(w4, w.w, sh));
        }
        const u32x4 out = {p0, p1, p2, p3};
        *reinterpret_cast<u32x4 *>(band + r * pitch + 4 * g) = out;
    }
}

template <typename OutT>
__global__ __launch_bounds__(kThreads) void preprocess_kernel(PreArgs a) {
    extern __shared__ uint32_t band[];
    const int64_t tile = blockIdx.x;
    const int img = find_segment(a.tile_begin, a.n, tile);
    const DevImage d = a.images[img];
    const int local = int(tile - a.tile_begin[img]);
    const int br = local / d.tiles_per_brow;
    const int bc0 = (local - br * d.tiles_per_brow) * d.units_per_tile;
    const int nb = min(d.units_per_tile, d.blocks_w - bc0);
    const bool identity = (d.flags & kFlagIdentity) != 0;

    // Source band touched by this tile: taps are monotone in the output
    // index, so the first and last output rows/columns bound it.
    const int oy_first = br * kUnitPx, oy_last = oy_first + kUnitPx - 1;
    const int ox_first = bc0 * kUnitPx, ox_last = (bc0 + nb) * kUnitPx - 1;
    int r_lo, r_hi, c_lo, c_hi;
    if (identity) {
        r_lo = oy_first; r_hi = oy_last; c_lo = ox_first; c_hi = ox_last;
    } else {
        r_lo = make_tap(d.scale_y, oy_first, d.src_h).i0;
        r_hi = make_tap(d.scale_y, oy_last, d.src_h).i1;
        c_lo = make_tap(d.scale_x, ox_first, d.src_w).i0;
        c_hi = make_tap(d.scale_x, ox_last, d.src_w).i1;
    }
    const int rows = r_hi - r_lo + 1;
    const int groups = (c_hi - c_lo + 4) >> 2;
    const int pitch = 4 * groups;
    const int64_t band_bytes = int64_t(rows) * d.src_w * d.channels;
    const bool fits = int64_t(rows) * pitch <= a.band_capacity && band_bytes < 0x7FFF0000ll;

    if (fits) {
        stage_band(band, a, d, r_lo, c_lo, rows, groups, pitch);
        __syncthreads();
        const LdsPixels px{band, pitch, r_lo, c_lo};
        if (identity) compute_tile<OutT, true>(px, d, a, br, bc0, nb);
        else compute_tile<OutT, false>(px, d, a, br, bc0, nb);
    } else {
        const GlobalPixels px{a.src + d.src_offset, int64_t(d.src_w) * d.channels, d.channels};
        if (identity) compute_tile<OutT, true>(px, d, a, br, bc0, nb);
        else compute_tile<OutT, false>(px, d, a, br, bc0, nb);
    }
}

// Column-order gather: one wavefront copies one merge unit (4 contiguous
// rows) from its merge-order position to its column-order position.
template <typename OutT>
__global__ __launch_bounds__(kThreads) void column_permute_kernel(PermArgs a) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t unit = int64_t(blockIdx.x) * kWaves + wave;
    if (unit >= a.total_units) return;  // wave-uniform
    const int64_t drow = unit * kRowsPerUnit;
    const int img = find_segment(a.row_begin, a.n, drow);
    const DevImage d = a.images[img];
    const int64_t j = (drow - d.row_offset) / kRowsPerUnit;  // column-order unit index
    const int64_t bc = j / d.blocks_h, br = j - bc * d.blocks_h;
    const int64_t src_row = d.row_offset + (br * d.blocks_w + bc) * kRowsPerUnit;
    constexpr int kVecs = kRowsPerUnit * kRowLen * int(sizeof(OutT)) / 16;  // 16-byte vectors per unit
    const u32x4 *in = reinterpret_cast<const u32x4 *>(static_cast<const OutT *>(a.in) + src_row * kRowLen);
    u32x4 *out = reinterpret_cast<u32x4 *>(static_cast<OutT *>(a.out) + drow * kRowLen);
#pragma unroll 4
    for (int i = lane; i < kVecs; i += 64) {
        const u32x4 v = __builtin_nontemporal_load(in + i);
        __builtin_nontemporal_store(v, out + i);
    }
}

// ------------------------------------------------------------- host side

std::atomic<int64_t> g_dispatches{0};

// Pinned host staging for the per-call descriptor tables: a small ring per
// device, each slot fenced by an event so a slot is rewritten only after
// its previous copy has executed.
class TableStaging {
  public:
    struct Slot {
        void *host = nullptr;
        size_t cap = 0;
        hipEvent_t done = nullptr;
        bool pending = false;
    };
    static constexpr int kSlots = 8;

    // Copies bytes from `table` to device `dst` on `stream`, asynchronously.
    hipError_t upload(const void *table, size_t bytes, void *dst, hipStream_t stream) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        std::lock_guard<std::mutex> lock(mu_);
        if (int(rings_.size()) <= dev) rings_.resize(dev + 1);
        Ring &ring = rings_[dev];
        Slot &s = ring.slots[ring.next];
        ring.next = (ring.next + 1) % kSlots;
        if (s.pending) {
            e = hipEventSynchronize(s.done);
            if (e != hipSuccess) return e;
            s.pending = false;
        }
        if (!s.done) {
            e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
        if (s.cap < bytes) {
            if (s.host) (void)hipHostFree(s.host);
            s.host = nullptr;
            s.cap = 0;
            e = hipHostMalloc(&s.host, bytes, hipHostMallocDefault);
            if (e != hipSuccess) return e;
            s.cap = bytes;
        }
        std::memcpy(s.host, table, bytes);
        e = hipMemcpyAsync(dst, s.host, bytes, hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return e;
        e = hipEventRecord(s.done, stream);
        if (e != hipSuccess) return e;
        s.pending = true;
        return hipSuccess;
    }

  private:
    struct Ring {
        Slot slots[kSlots];
        int next = 0;
    };
    std::mutex mu_;
    std::vector<Ring> rings_;
};

TableStaging &staging() {
    static TableStaging *s = new TableStaging();  // lives until process exit
    return *s;
}

int hip_error(hipError_t e, const char *what) {
    return set_error(MIMO_E_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                                     hipGetErrorString(e) + ")");
}

// Conservative size of the LDS band one tile of k units needs, in dwords.
int64_t band_estimate(const DevImage &d, int k) {
    if (d.flags & kFlagIdentity) return int64_t(kUnitPx) * (4 * ((kUnitPx * k + 3) / 4));
    const double rows = std::min<double>(d.src_h, std::ceil(31.0 * d.scale_y) + 4.0);
    const double cols = std::min<double>(d.src_w, std::ceil((kUnitPx * k - 1.0) * d.scale_x) + 4.0);
    return int64_t(rows) * (4 * ((int64_t(cols) + 3) / 4 + 1));
}

struct BuiltTables {
    std::vector<uint8_t> bytes;  // workspace image
    int64_t total_tiles = 0;
    int64_t total_rows = 0;
    int32_t band_capacity = 0;  // dwords
};

// Builds the workspace image: DevImage records, tile prefix, row prefix.
int build_tables(int32_t n, const mimo_image_desc *desc, BuiltTables &out) {
    out.bytes.assign(ws_total_bytes(n), 0);
    DevImage *img = reinterpret_cast<DevImage *>(out.bytes.data());
    int64_t *tile_begin = reinterpret_cast<int64_t *>(out.bytes.data() + ws_images_bytes(n));
    int64_t *row_begin =
        reinterpret_cast<int64_t *>(out.bytes.data() + ws_images_bytes(n) + ws_prefix_bytes(n));
    int64_t tiles = 0, rows = 0, band = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mimo_image_desc &s = desc[i];
        DevImage d;
        std::memset(&d, 0, sizeof(d));
        tile_begin[i] = tiles;
        row_begin[i] = rows;
        d.src_offset = s.src_offset;
        d.row_offset = rows;
        if (s.status != MIMO_OK || s.rows == 0) {
            d.tiles_per_brow = 1;
            d.units_per_tile = 1;
            img[i] = d;
            continue;
        }
        if (s.src_h < 1 || s.src_w < 1 || (s.channels != 3 && s.channels != 4) ||
            s.dst_h < kUnitPx || s.dst_w < kUnitPx || s.dst_h % kUnitPx || s.dst_w % kUnitPx ||
            s.grid_t != 1 || s.grid_h * kPatch != s.dst_h || s.grid_w * kPatch != s.dst_w ||
            s.rows != int64_t(s.grid_h) * s.grid_w || s.row_offset != rows || s.src_offset < 0)
            return set_error(MIMO_E_INVALID, "descriptor " + std::to_string(i) +
                                                 " is not a plan of the 16/2/2 kernels");
        if (s.src_h > kMaxSide || s.src_w > kMaxSide || s.dst_h > kMaxSide || s.dst_w > kMaxSide)
            return set_error(MIMO_E_TOO_LARGE, "descriptor " + std::to_string(i) + ": side too large");
        d.src_h = s.src_h;
        d.src_w = s.src_w;
        d.channels = s.channels;
        d.blocks_h = s.dst_h / kUnitPx;
        d.blocks_w = s.dst_w / kUnitPx;
        d.scale_y = float(s.src_h) / float(s.dst_h);
        d.scale_x = float(s.src_w) / float(s.dst_w);
        d.flags = (s.src_h == s.dst_h && s.src_w == s.dst_w) ? kFlagIdentity : 0;
        int k = kMaxUnitsPerTile;
        while (k > 1 && band_estimate(d, k) > kBandBudgetDwords) k >>= 1;
        if (band_estimate(d, k) <= kBandBudgetDwords) band = std::max(band, band_estimate(d, k));
        d.units_per_tile = std::min(k, d.blocks_w);
        d.tiles_per_brow = (d.blocks_w + d.units_per_tile - 1) / d.units_per_tile;
        img[i] = d;
        tiles += int64_t(d.blocks_h) * d.tiles_per_brow;
        rows += s.rows;
    }
    tile_begin[n] = tiles;
    row_begin[n] = rows;
    out.total_tiles = tiles;
    out.total_rows = rows;
    out.band_capacity = int32_t(std::max<int64_t>(band, 4));
    return MIMO_OK;
}

int check_ptr_align(const void *p, uintptr_t align) {
    return (reinterpret_cast<uintptr_t>(p) & (align - 1)) == 0;
}

}  // namespace mimo

using namespace mimo;

extern "C" {

int64_t mimo_dispatch_count(void) { return g_dispatches.load(); }

int mimo_preprocess_batch(int32_t n, const mimo_image_desc *desc, const uint8_t *src,
                          int64_t src_capacity, const float *mean255, const float *std255,
                          int32_t out_dtype, void *rows, void *rows_col, int64_t capacity_rows,
                          void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    if (n < 0 || (n > 0 && !desc) || !mean255 || !std255)
        return set_error(MIMO_E_INVALID, "preprocess_batch: bad n or null pointer");
    if (out_dtype != MIMO_F32 && out_dtype != MIMO_BF16)
        return set_error(MIMO_E_INVALID, "preprocess_batch: out_dtype must be MIMO_F32 or MIMO_BF16");
    if (!rows && !rows_col)
        return set_error(MIMO_E_INVALID, "preprocess_batch: both outputs are null");
    if ((rows && !check_ptr_align(rows, 16)) || (rows_col && !check_ptr_align(rows_col, 16)))
        return set_error(MIMO_E_INVALID, "preprocess_batch: outputs must be 16-byte aligned");
    if (n == 0) return MIMO_OK;
    if (!src || !check_ptr_align(src, 4))
        return set_error(MIMO_E_INVALID, "preprocess_batch: src must be non-null and 4-byte aligned");
    if (!workspace || !check_ptr_align(workspace, 16))
        return set_error(MIMO_E_INVALID, "preprocess_batch: workspace must be non-null and 16-byte aligned");
    if (workspace_bytes < ws_total_bytes(n))
        return set_error(MIMO_E_CAPACITY, "preprocess_batch: workspace smaller than mimo_workspace_bytes(n)");
    PreArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int c = 0; c < 3; ++c) {
        if (!(std255[c] > 0.0f) || !std::isfinite(std255[c]) || !std::isfinite(mean255[c]))
            return set_error(MIMO_E_INVALID, "preprocess_batch: std255 must be > 0 and finite");
        a.inv_std[c] = float(1.0 / double(std255[c]));
        a.mean[c] = mean255[c];
    }
    BuiltTables t;
    int st = build_tables(n, desc, t);
    if (st != MIMO_OK) return st;
    int64_t src_needed = 0;
    for (int32_t i = 0; i < n; ++i)
        if (desc[i].status == MIMO_OK && desc[i].rows > 0)
            src_needed = std::max<int64_t>(src_needed, desc[i].src_offset + int64_t(desc[i].src_h) *
                                                                             desc[i].src_w * desc[i].channels);
    if (src_capacity < ((src_needed + 15) & ~int64_t(15)))
        return set_error(MIMO_E_CAPACITY, "preprocess_batch: src_capacity below the packed size rounded up to 16");
    if (t.total_rows > capacity_rows)
        return set_error(MIMO_E_CAPACITY, "preprocess_batch: capacity_rows " + std::to_string(capacity_rows) +
                                              " < " + std::to_string(t.total_rows) + " rows");
    if (t.total_tiles == 0) return MIMO_OK;
    if (t.total_tiles > 0x7FFFFFFFll)
        return set_error(MIMO_E_TOO_LARGE, "preprocess_batch: more than 2^31-1 tiles");

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = staging().upload(t.bytes.data(), t.bytes.size(), workspace, s);
    if (e != hipSuccess) return hip_error(e, "preprocess_batch: table upload");

    uint8_t *ws = static_cast<uint8_t *>(workspace);
    a.src = src;
    a.src_end = src_capacity;
    a.images = reinterpret_cast<const DevImage *>(ws);
    a.tile_begin = reinterpret_cast<const int64_t *>(ws + ws_images_bytes(n));
    a.rows = rows;
    a.rows_col = rows_col;
    a.n = n;
    a.band_capacity = t.band_capacity;
    const size_t lds = size_t(t.band_capacity) * 4;
    const dim3 grid{unsigned(t.total_tiles), 1, 1}, block{unsigned(kThreads), 1, 1};
    if (out_dtype == MIMO_F32)
        hipLaunchKernelGGL(preprocess_kernel<float>, grid, block, lds, s, a);
    else
        hipLaunchKernelGGL(preprocess_kernel<uint16_t>, grid, block, lds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "preprocess_batch: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
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
    int st = build_tables(n, desc, t);
    if (st != MIMO_OK) return st;
    if (t.total_rows > capacity_rows)
        return set_error(MIMO_E_CAPACITY, "column_permute: capacity_rows below the total rows");
    if (t.total_rows == 0) return MIMO_OK;
    const int64_t units = t.total_rows / kRowsPerUnit;
    const int64_t blocks = (units + kWaves - 1) / kWaves;
    if (blocks > 0x7FFFFFFFll)
        return set_error(MIMO_E_TOO_LARGE, "column_permute: too many merge units");

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = staging().upload(t.bytes.data(), t.bytes.size(), workspace, s);
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
    if (out_dtype == MIMO_F32)
        hipLaunchKernelGGL(column_permute_kernel<float>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(column_permute_kernel<uint16_t>, grid, block, 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "column_permute: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

}  // extern "C"
