// internal.h -- definitions shared by the host planner and the HIP kernels of
// the MiMo-V2 pixel path library (not part of the public ABI).
#pragma once

#include <cstdint>
#include <string>

#include "mimo_pre.h"

namespace mimo {

// Kernel geometry: patch 16, merge 2, two frames (processing page,
// MimoV2ImageProcessor defaults; cortiq mimo_vision: factor 32, T = 2,
// rows flattened as (c, tt, py, px)).
constexpr int kPatch = 16;
constexpr int kMerge = 2;
constexpr int kTemporal = 2;
constexpr int kUnitPx = kPatch * kMerge;                       // 32 output pixels per merge unit side
constexpr int kRowLen = 3 * kTemporal * kPatch * kPatch;        // 1536 values per row
constexpr int kRowsPerUnit = kMerge * kMerge;                   // 4 rows per merge unit
constexpr int kPlane = kPatch * kPatch;                         // 256 values per (c, tt) plane

// Largest side the kernels index: coordinates are formed as float(d) + 0.5
// and float(n_in), which are exact below 2^23.
constexpr int64_t kMaxSide = (int64_t(1) << 23) - 1;
// Largest row count of one image: per-image row and tile indices are formed
// in 32-bit arithmetic with float-reciprocal quotients, exact below 2^24.
constexpr int64_t kMaxRowsPerImage = int64_t(1) << 24;

// Per-image record the fused kernel reads (64 bytes, one per image).
struct DevImage {
    int64_t src_offset;     // byte offset of the image in the packed sources
    int64_t row_offset;     // first output row (merge-block order)
    int32_t src_h, src_w;
    int32_t channels;       // 3 or 4
    int32_t flags;          // kFlag* bits
    int32_t blocks_h;       // merge units per column  (grid_h / 2)
    int32_t blocks_w;       // merge units per row     (grid_w / 2)
    int32_t tiles_per_brow; // tiles along one block row (4 * blocks_w rows)
    float inv_tiles_per_brow;  // 1 / tiles_per_brow (quotient estimate, corrected exactly)
    float scale_y;          // float32(src_h) / float32(dst_h)
    float scale_x;          // float32(src_w) / float32(dst_w)
    float inv_blocks_h;     // 1 / blocks_h
    int32_t frames;         // source frames (1 for a still image)
};
static_assert(sizeof(DevImage) == 64, "DevImage must stay 64 bytes");

constexpr int32_t kFlagIdentity = 1;  // dst == src on both axes

// Workspace layout: [DevImage x n][int64 tile_begin x (n+1)][int64 row_begin x (n+1)],
// each part 256-byte aligned.
constexpr size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
constexpr size_t ws_images_bytes(int32_t n) { return align256(sizeof(DevImage) * size_t(n)); }
constexpr size_t ws_prefix_bytes(int32_t n) { return align256(sizeof(int64_t) * (size_t(n) + 1)); }
constexpr size_t ws_total_bytes(int32_t n) { return ws_images_bytes(n) + 2 * ws_prefix_bytes(n); }
constexpr size_t ws_total_bytes_const(int32_t n) { return ws_total_bytes(n); }

// Thread-local error reporting.
int set_error(int code, const std::string &msg);
void clear_error();

}  // namespace mimo
