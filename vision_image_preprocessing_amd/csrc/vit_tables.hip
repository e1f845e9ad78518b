// vit_tables.hip -- ViT index tables for the rows the pixel path emits:
// per-row rotary positions with their cos/sin tables, and the merge-unit
// window index, for AMD Instinct MI355X (gfx950).
//
// What is computed (NeMo Automodel "mimo_v2_flash.vision":
// MiMoVisionRotaryEmbedding(dim, theta), MiMoVisionTransformer
// ._rotary_positions, ._get_window_index(grid_thw, column_major),
// ._apply_merge_index; docs.rs "cortiq_engine::mimo_vision" module
// conventions): a row of merge-block order (t, block row, block col, mh, mw)
// covers the patch at grid row 2 * block row + mh and grid column
// 2 * block col + mw; type-1 window blocks list whole merge units by
// (t, block col, block row) and the RoPE tables follow the rows; every
// temporal slice is its own chunk.
//
// Both kernels are output streams with no reads beyond a 64-byte record per
// item: a workgroup owns a run of rows (or merge units) of one item, found
// with the same 64-ary wavefront search over tile prefix sums as the pixel
// kernel, and writes every output byte once.  The rotary kernel gives each
// lane four consecutive table columns of one row, so a wavefront's cos and
// sin stores are contiguous 1 KB runs.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "device_util.h"
#include "internal.h"
#include "runtime.h"

namespace mimo {
namespace {

constexpr int kTableThreads = 256;
constexpr int kRowsPerTableTile = 128;     // rows of one item per rotary workgroup (64: 107 us, 128: 93, 256: 109 on 2 M rows)
constexpr int kUnitsPerIndexTile = 256;    // merge units of one item per index workgroup

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

struct RotaryArgs {
    const DevImage *images;
    const int64_t *tile_begin;  // [n + 1]
    const int64_t *row_begin;   // [n + 1]
    int32_t *pos;               // [rows][2] or null
    float *cos_out;             // [rows][dim] or null
    float *sin_out;             // [rows][dim] or null
    int32_t n;
    int32_t column;             // rows listed in column order
    int32_t dim;                // table width (rope_dim)
    int32_t chunks;             // dim / 4 columns groups per row
    float inv_chunks;           // 1 / chunks
    float inv_freq[MIMO_ROPE_DIM_MAX / 2];
};

struct WindowArgs {
    const DevImage *images;
    const int64_t *tile_begin;  // [n + 1]
    const int64_t *row_begin;   // [n + 1]
    int64_t *index;             // [units] or null
    int64_t *inverse;           // [units] or null
    int32_t n;
    int32_t column_major;
};

// Grid position (h, w) of row `local` of an item, in merge-block order or,
// with `column`, in column order.  local < 2^24.
__device__ __forceinline__ void row_position(const DevImage &d, int local, bool column, int &h,
                                             int &w) {
    const int bh = d.blocks_h, bw = d.blocks_w;
    const int per_slice = kRowsPerUnit * bh * bw;
    const int t = div_small(local, per_slice, 1.0f / float(per_slice));
    const int in_slice = local - t * per_slice;
    const int unit = in_slice / kRowsPerUnit;
    const int k = in_slice - unit * kRowsPerUnit;  // (mh, mw) = divmod(k, merge)
    int br, bc;
    if (column) {
        bc = div_small(unit, bh, d.inv_blocks_h);
        br = unit - bc * bh;
    } else {
        br = div_small(unit, bw, 1.0f / float(bw));
        bc = unit - br * bw;
    }
    h = br * kMerge + k / kMerge;
    w = bc * kMerge + k % kMerge;
}

__global__ __launch_bounds__(kTableThreads) void rotary_tables_kernel(RotaryArgs a) {
    const int64_t tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    const int img = find_segment(a.tile_begin, a.n, tile);
    const DevImage d = a.images[img];
    const int rows_i = int(a.row_begin[img + 1] - a.row_begin[img]);
    const int first = int(tile - a.tile_begin[img]) * kRowsPerTableTile;
    const int count = min(kRowsPerTableTile, rows_i - first);
    const int half = a.dim >> 1;
    const bool column = a.column != 0;
    for (int idx = threadIdx.x; idx < count * a.chunks; idx += blockDim.x) {
        const int r = div_small(idx, a.chunks, a.inv_chunks);
        const int c = idx - r * a.chunks;
        int h, w;
        row_position(d, first + r, column, h, w);
        const int64_t row = d.row_offset + first + r;
        if (a.pos && c == 0) {
            const i32x2 hw = {h, w};
            *reinterpret_cast<i32x2 *>(a.pos + 2 * row) = hw;
        }
        if (!a.cos_out && !a.sin_out) continue;
        // columns [4c, 4c + 4) lie in one half (half is a multiple of 4):
        // the h half first, then the w half
        const int col = 4 * c;
        const bool w_half = col >= half;
        const float p = float(w_half ? w : h);
        const int k0 = w_half ? col - half : col;
        float cs[4], sn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float angle = p * a.inv_freq[k0 + j];  // one float32 rounding
            sincosf(angle, &sn[j], &cs[j]);
        }
        const int64_t off = row * a.dim + col;
        if (a.cos_out) {
            const f32x4 v = {cs[0], cs[1], cs[2], cs[3]};
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(a.cos_out + off));
        }
        if (a.sin_out) {
            const f32x4 v = {sn[0], sn[1], sn[2], sn[3]};
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(a.sin_out + off));
        }
    }
}

__global__ __launch_bounds__(kTableThreads) void window_index_kernel(WindowArgs a) {
    const int64_t tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    const int img = find_segment(a.tile_begin, a.n, tile);
    const DevImage d = a.images[img];
    const int units_i = int((a.row_begin[img + 1] - a.row_begin[img]) / kRowsPerUnit);
    const int u = int(tile - a.tile_begin[img]) * kUnitsPerIndexTile + int(threadIdx.x);
    if (u >= units_i) return;
    int src = u;
    if (a.column_major) {
        const int per_slice = d.blocks_h * d.blocks_w;
        const int t = div_small(u, per_slice, 1.0f / float(per_slice));
        const int j = u - t * per_slice;
        const int bc = div_small(j, d.blocks_h, d.inv_blocks_h);
        const int br = j - bc * d.blocks_h;
        src = t * per_slice + br * d.blocks_w + bc;
    }
    const int64_t base = d.row_offset / kRowsPerUnit;
    if (a.index) a.index[base + u] = base + src;
    if (a.inverse) a.inverse[base + src] = base + u;
}

// Per-item records and tile prefix sums for the table kernels: tiles of
// `per_tile` rows (units = false) or merge units (units = true) of one item.
struct ItemTables {
    std::vector<uint8_t> bytes;  // workspace image (same layout as the pixel kernel's)
    int64_t tiles = 0;
    int64_t rows = 0;
};

int build_item_tables(int32_t n, const mimo_image_desc *desc, int per_tile, bool units,
                      const char *who, ItemTables &out) {
    out.bytes.assign(ws_total_bytes(n), 0);
    DevImage *img = reinterpret_cast<DevImage *>(out.bytes.data());
    int64_t *tile_begin = reinterpret_cast<int64_t *>(out.bytes.data() + ws_images_bytes(n));
    int64_t *row_begin =
        reinterpret_cast<int64_t *>(out.bytes.data() + ws_images_bytes(n) + ws_prefix_bytes(n));
    int64_t tiles = 0, rows = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mimo_image_desc &s = desc[i];
        DevImage d;
        std::memset(&d, 0, sizeof(d));
        tile_begin[i] = tiles;
        row_begin[i] = rows;
        d.row_offset = rows;
        if (s.status != MIMO_OK || s.rows == 0) {
            img[i] = d;
            continue;
        }
        if (s.grid_t < 1 || s.grid_h < kMerge || s.grid_w < kMerge || s.grid_h % kMerge ||
            s.grid_w % kMerge || s.rows != int64_t(s.grid_t) * s.grid_h * s.grid_w ||
            s.row_offset != rows)
            return set_error(MIMO_E_INVALID, std::string(who) + ": descriptor " + std::to_string(i) +
                                                 " is not a plan of the 16/2/2 kernels");
        if (s.rows > kMaxRowsPerImage)
            return set_error(MIMO_E_TOO_LARGE, std::string(who) + ": descriptor " + std::to_string(i) +
                                                   " has more than 2^24 rows");
        d.blocks_h = s.grid_h / kMerge;
        d.blocks_w = s.grid_w / kMerge;
        d.inv_blocks_h = 1.0f / float(d.blocks_h);
        d.frames = s.frames;
        img[i] = d;
        const int64_t count = units ? s.rows / kRowsPerUnit : s.rows;
        tiles += (count + per_tile - 1) / per_tile;
        rows += s.rows;
    }
    tile_begin[n] = tiles;
    row_begin[n] = rows;
    out.tiles = tiles;
    out.rows = rows;
    return MIMO_OK;
}

int check_workspace(int32_t n, void *workspace, size_t workspace_bytes, const char *who) {
    if (!workspace || !check_ptr_align(workspace, 16))
        return set_error(MIMO_E_INVALID, std::string(who) + ": workspace must be non-null and 16-byte aligned");
    if (workspace_bytes < ws_total_bytes(n))
        return set_error(MIMO_E_CAPACITY, std::string(who) + ": workspace smaller than mimo_workspace_bytes(n)");
    return MIMO_OK;
}

}  // namespace
}  // namespace mimo

using namespace mimo;

extern "C" {

int mimo_rotary_tables(int32_t n, const mimo_image_desc *desc, int32_t order, int32_t rope_dim,
                       double theta, int32_t *pos_hw, float *rope_cos, float *rope_sin,
                       int64_t capacity_rows, void *workspace, size_t workspace_bytes,
                       void *stream) {
    clear_error();
    if (n < 0 || (n > 0 && !desc))
        return set_error(MIMO_E_INVALID, "rotary_tables: bad n or null desc");
    if (order != MIMO_ORDER_MERGE && order != MIMO_ORDER_COLUMN)
        return set_error(MIMO_E_INVALID, "rotary_tables: order must be MIMO_ORDER_MERGE or MIMO_ORDER_COLUMN");
    if (rope_dim < 8 || rope_dim > MIMO_ROPE_DIM_MAX || rope_dim % 8)
        return set_error(MIMO_E_INVALID, "rotary_tables: rope_dim must be a multiple of 8 in [8, 256]");
    if (!pos_hw && !rope_cos && !rope_sin)
        return set_error(MIMO_E_INVALID, "rotary_tables: no output given");
    if ((pos_hw && !check_ptr_align(pos_hw, 8)) || (rope_cos && !check_ptr_align(rope_cos, 16)) ||
        (rope_sin && !check_ptr_align(rope_sin, 16)))
        return set_error(MIMO_E_INVALID, "rotary_tables: pos_hw must be 8-byte and the tables 16-byte aligned");
    RotaryArgs a;
    std::memset(&a, 0, sizeof(a));
    int st = mimo_rope_inv_freq(rope_dim, theta, a.inv_freq);
    if (st != MIMO_OK) return st;
    if (n == 0) return MIMO_OK;
    st = check_workspace(n, workspace, workspace_bytes, "rotary_tables");
    if (st != MIMO_OK) return st;
    ItemTables t;
    st = build_item_tables(n, desc, kRowsPerTableTile, false, "rotary_tables", t);
    if (st != MIMO_OK) return st;
    if (t.rows > capacity_rows)
        return set_error(MIMO_E_CAPACITY, "rotary_tables: capacity_rows below the plan's total rows");
    if (t.tiles == 0) return MIMO_OK;
    if (t.tiles > 0x7FFFFFFFll)
        return set_error(MIMO_E_TOO_LARGE, "rotary_tables: more than 2^31 - 1 tiles");

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = upload_table(t.bytes.data(), t.bytes.size(), workspace, s);
    if (e != hipSuccess) return hip_error(e, "rotary_tables: table upload");
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    a.images = reinterpret_cast<const DevImage *>(ws);
    a.tile_begin = reinterpret_cast<const int64_t *>(ws + ws_images_bytes(n));
    a.row_begin = reinterpret_cast<const int64_t *>(ws + ws_images_bytes(n) + ws_prefix_bytes(n));
    a.pos = pos_hw;
    a.cos_out = rope_cos;
    a.sin_out = rope_sin;
    a.n = n;
    a.column = order == MIMO_ORDER_COLUMN;
    a.dim = rope_dim;
    a.chunks = rope_dim / 4;
    a.inv_chunks = 1.0f / float(a.chunks);
    const dim3 grid{unsigned(t.tiles), 1, 1}, block{unsigned(kTableThreads), 1, 1};
    e = timed_launch(s, [&] { hipLaunchKernelGGL(rotary_tables_kernel, grid, block, 0, s, a); });
    if (e != hipSuccess) return hip_error(e, "rotary_tables: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

int mimo_window_index(int32_t n, const mimo_image_desc *desc, int32_t column_major,
                      int64_t *index, int64_t *inverse, int64_t capacity_units, void *workspace,
                      size_t workspace_bytes, void *stream) {
    clear_error();
    if (n < 0 || (n > 0 && !desc))
        return set_error(MIMO_E_INVALID, "window_index: bad n or null desc");
    if (column_major != 0 && column_major != 1)
        return set_error(MIMO_E_INVALID, "window_index: column_major must be 0 or 1");
    if (!index && !inverse)
        return set_error(MIMO_E_INVALID, "window_index: no output given");
    if ((index && !check_ptr_align(index, 8)) || (inverse && !check_ptr_align(inverse, 8)))
        return set_error(MIMO_E_INVALID, "window_index: outputs must be 8-byte aligned");
    if (n == 0) return MIMO_OK;
    int st = check_workspace(n, workspace, workspace_bytes, "window_index");
    if (st != MIMO_OK) return st;
    ItemTables t;
    st = build_item_tables(n, desc, kUnitsPerIndexTile, true, "window_index", t);
    if (st != MIMO_OK) return st;
    if (t.rows / kRowsPerUnit > capacity_units)
        return set_error(MIMO_E_CAPACITY, "window_index: capacity_units below the plan's merge units");
    if (t.tiles == 0) return MIMO_OK;
    if (t.tiles > 0x7FFFFFFFll)
        return set_error(MIMO_E_TOO_LARGE, "window_index: more than 2^31 - 1 tiles");

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = upload_table(t.bytes.data(), t.bytes.size(), workspace, s);
    if (e != hipSuccess) return hip_error(e, "window_index: table upload");
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    WindowArgs a;
    a.images = reinterpret_cast<const DevImage *>(ws);
    a.tile_begin = reinterpret_cast<const int64_t *>(ws + ws_images_bytes(n));
    a.row_begin = reinterpret_cast<const int64_t *>(ws + ws_images_bytes(n) + ws_prefix_bytes(n));
    a.index = index;
    a.inverse = inverse;
    a.n = n;
    a.column_major = column_major;
    const dim3 grid{unsigned(t.tiles), 1, 1}, block{unsigned(kTableThreads), 1, 1};
    e = timed_launch(s, [&] { hipLaunchKernelGGL(window_index_kernel, grid, block, 0, s, a); });
    if (e != hipSuccess) return hip_error(e, "window_index: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

}  // extern "C"
