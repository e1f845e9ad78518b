// tables.h -- the per-call descriptor tables the pixel kernels read (one
// DevImage per image, the tile and row prefix sums), built on the host from
// a plan; shared by the pixel kernel (preprocess.hip) and the fused pixel
// embedding (pixel_embed.hip).
#pragma once

#include <algorithm>
#include <cstdint>
#include <vector>

#include "internal.h"

namespace mimo {

// Tiling policy: rows per tile (1, 2 or a multiple of 4) and whether
// workgroups are mapped to XCD-contiguous runs of tiles.  Small tiles keep
// the output each workgroup writes small, which the HBM write path favours.
// With both outputs requested the grid holds two passes of tiles (merge
// order, then column order), so each output is written as a dense stream.
#ifndef MIMO_ROWS_PER_TILE
#define MIMO_ROWS_PER_TILE 4
#endif
#ifndef MIMO_ROWS_PER_TILE_DUAL
#define MIMO_ROWS_PER_TILE_DUAL 1
#endif
#ifndef MIMO_ROWS_PER_TILE_CLIPS
#define MIMO_ROWS_PER_TILE_CLIPS 12
#endif
#ifndef MIMO_XCD_ORDER
#define MIMO_XCD_ORDER 1
#endif
struct Tiling {
    int rows_per_tile = MIMO_ROWS_PER_TILE;
    int xcd_order = MIMO_XCD_ORDER;
    int passes = 1;
    // clips: the batch holds an item with two or more frames.  A clip tile
    // stages and resamples its two frames one after the other; three merge
    // units per tile amortise the two band loads and barriers better than
    // one (measured on 64-frame 1280x720 clips, bf16: 0.62 vs 0.70 ms).
    static Tiling choose(bool merge, bool column, bool clips) {
        Tiling t;
        if (clips) t.rows_per_tile = MIMO_ROWS_PER_TILE_CLIPS;
        if (merge && column) {
            t.passes = 2;
            t.rows_per_tile = std::min(MIMO_ROWS_PER_TILE_DUAL, kRowsPerUnit);
        } else if (column) {
            t.rows_per_tile = std::min(t.rows_per_tile, kRowsPerUnit);
        }
        return t;
    }
    int threads() const { return 64 * std::min(rows_per_tile, kRowsPerUnit); }
};

struct BuiltTables {
    std::vector<uint8_t> bytes;  // workspace image (build_tables)
    int64_t total_tiles = 0;
    int64_t total_rows = 0;
    int32_t band_capacity = 0;  // dwords
    bool clips = false;         // some item has two or more frames
};

// Builds the workspace image -- DevImage records, tile prefix, row prefix --
// into `bytes` (ws_total_bytes(n) bytes, zeroed by the caller).
int build_tables_into(int32_t n, const mimo_image_desc *desc, const Tiling &tiling, uint8_t *bytes,
                      BuiltTables &out);
// The same, into out.bytes.
int build_tables(int32_t n, const mimo_image_desc *desc, const Tiling &tiling, BuiltTables &out);

}  // namespace mimo
