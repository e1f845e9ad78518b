/*
 * mimo_pre.h -- C ABI of the MI355X (gfx950) MiMo-V2 image pixel path.
 *
 * The pixel path, as defined on the pages this library implements:
 *   NeMo Automodel "mimo_v2_flash.processing" (module docstring, the
 *   MimoV2ImageProcessor class docstring and defaults, smart_resize, _to_rgb,
 *   get_number_of_image_patches) and docs.rs "cortiq_engine::mimo_vision"
 *   (module conventions, resize_bilinear, column_permutation, smart_resize):
 *
 *   uint8 RGB or RGBA image -> RGBA flattened onto white -> float 0-255 ->
 *   bilinear resize (align_corners=False, no antialias, no 8-bit round trip)
 *   to the smart_resize target -> (x - mean255[c]) / std255[c] -> two
 *   identical frames -> rows of 3*2*16*16 = 1536 values, the Conv3d kernel
 *   flattened as (c, tt, py, px), listed in merge-block order
 *   (t, block row, block col, mh, mw); optionally also in column order
 *   (t, block col, block row), each merge unit's 4 rows kept together.
 *
 * Conventions for every entry point:
 *   - Plain C types only.  "device" pointers are HIP device memory on the
 *     current device; "host" pointers are ordinary host memory.
 *   - The caller owns every buffer.  The library never frees caller memory.
 *   - Functions return MIMO_OK (0) or a negative MIMO_E_* code; nothing is
 *     thrown across the ABI.  mimo_last_error() gives a message for the last
 *     failure on the calling thread.
 *   - GPU work is enqueued on the given stream (a hipStream_t passed as
 *     void*, NULL = the null stream) and is asynchronous: outputs are valid
 *     once the stream has reached the enqueued work.
 *   - Thread safety: all entry points may be called concurrently from
 *     different threads.
 */
#ifndef MIMO_PRE_H
#define MIMO_PRE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MIMO_OK 0
#define MIMO_E_INVALID (-1)     /* bad argument: size <= 0, null pointer, std <= 0, ... */
#define MIMO_E_ASPECT (-2)      /* long/short side ratio above max_aspect (short side >= factor) */
#define MIMO_E_DEGENERATE (-3)  /* shrink to max_pixels floors a side to zero */
#define MIMO_E_UNSUPPORTED (-4) /* parameters the kernels do not implement */
#define MIMO_E_CAPACITY (-5)    /* an output or workspace buffer is too small */
#define MIMO_E_HIP (-6)         /* HIP runtime error (message in mimo_last_error) */
#define MIMO_E_TOO_LARGE (-7)   /* a side >= 2^23 or an image of more than 2^24 rows */

/* ---- output element types ---------------------------------------------- */
#define MIMO_F32 0  /* float32 */
#define MIMO_BF16 1 /* bfloat16, rounded to nearest even from the float32 value */

/*
 * Processor knobs (processing page, MimoV2ImageProcessor signature; cortiq
 * MimoProcessorConfig).  factor = patch_size * merge_size.
 * The kernels implement patch_size 16, merge_size 2, temporal_patch_size 2
 * (rows of 1536 values); the geometry functions accept any positive values.
 * max_aspect is the aspect guard of the Qwen2-VL smart_resize (200); a ratio
 * strictly above it is rejected on the branch whose short side is >= factor.
 */
typedef struct mimo_params {
    int32_t patch_size;          /* 16 */
    int32_t merge_size;          /* 2 */
    int32_t temporal_patch_size; /* 2 */
    int32_t reserved0;           /* must be 0 */
    int64_t min_pixels;          /* 8192: lower bound on the resized area */
    int64_t max_pixels;          /* 8388608: upper bound on the resized area */
    double max_aspect;           /* 200 */
} mimo_params;

/* Fills *p with the defaults above. */
void mimo_default_params(mimo_params *p);

/*
 * Per-item plan, produced by mimo_plan_geometry / mimo_plan_frames and
 * consumed unchanged by mimo_preprocess_batch and mimo_column_permute.  An
 * item is a still image (frames = 1) or a video of `frames` frames of one
 * size.  64 bytes.
 *   src_offset  byte offset of the item in the packed source buffer; items
 *               are packed back to back in batch order, each frame row-major
 *               uint8 [src_h][src_w][channels], the frames of a video back
 *               to back.
 *   row_offset  first output row of this image (rows of all images are
 *               concatenated in batch order).
 *   rows        grid_t * grid_h * grid_w (get_number_of_image_patches);
 *               placeholder tokens = rows / merge_size^2.
 *   dst_h/dst_w smart_resize target; grid_h = dst_h / patch_size,
 *               grid_w = dst_w / patch_size, grid_t = ceil(frames / 2):
 *               consecutive frames pair into temporal patches, an odd count
 *               repeating its last frame (so a still image is two identical
 *               frames, grid_t = 1).  (grid_t, grid_h, grid_w) is
 *               image_grid_thw / video_grid_thw.
 *   status      MIMO_OK or the item's MIMO_E_* code; a failed item has
 *               rows = 0 and contributes no output.
 *   frames      source frames of the item (1 for a still image).
 */
typedef struct mimo_image_desc {
    int64_t src_offset;
    int64_t row_offset;
    int64_t rows;
    int32_t src_h, src_w, channels;
    int32_t dst_h, dst_w;
    int32_t grid_t, grid_h, grid_w;
    int32_t status;
    int32_t frames;
} mimo_image_desc;

/*
 * smart_resize (processing page; cortiq smart_resize): resize target for one
 * h x w image with factor = patch_size * merge_size.  Round each side to the
 * nearest multiple of factor (ties to even); if the area exceeds max_pixels
 * shrink both sides by sqrt(h*w/max_pixels) and floor to the factor; if it
 * is below min_pixels grow by sqrt(min_pixels/(h*w)) and ceil.  A short side
 * below factor is first scaled up to factor (both sides by the same ratio)
 * and that branch skips the aspect guard; a shrink that floors a side to
 * zero is rejected.
 * Host only.  Returns MIMO_OK, MIMO_E_INVALID (h, w < 1 or bad params),
 * MIMO_E_ASPECT or MIMO_E_DEGENERATE; *out_h, *out_w untouched on error.
 */
int mimo_smart_resize(int64_t h, int64_t w, const mimo_params *params, int64_t *out_h,
                      int64_t *out_w);

/*
 * Plans a batch of n images (host only, no allocation).
 *   hwc        host int32 [n][3]: height, width, channels (3 = RGB, 4 = RGBA).
 *   params     NULL for the defaults.
 *   out        host [n] descriptors, written in batch order.
 *   total_rows host, nullable: sum of rows (the pixel_values row count).
 *   total_src_bytes host, nullable: packed source size in bytes.
 * Every image is planned; a failing image gets its code in out[i].status and
 * rows = 0.  Returns MIMO_OK, or the first failing image's code.
 */
int mimo_plan_geometry(int32_t n, const int32_t *hwc, const mimo_params *params,
                       mimo_image_desc *out, int64_t *total_rows, int64_t *total_src_bytes);

/*
 * Plans a batch of still images and videos (host only, no allocation).
 *   fhwc       host int32 [n][4]: frames, height, width, channels.  frames = 1
 *              is a still image; a video's frames share one size.
 *   max_pixels host int64 [n], nullable: a per-item ceiling on the resized
 *              area used instead of params->max_pixels (prepare_video_frames:
 *              the per-frame budget from mimo_video_max_pixels); entries <= 0
 *              mean params->max_pixels.
 * One smart_resize per item serves all its frames (cortiq
 * prepare_video_frames).  Otherwise as mimo_plan_geometry.
 */
int mimo_plan_frames(int32_t n, const int32_t *fhwc, const int64_t *max_pixels,
                     const mimo_params *params, mimo_image_desc *out, int64_t *total_rows,
                     int64_t *total_src_bytes);

/*
 * cortiq video_max_pixels: per-frame pixel ceiling for n_sampled frames,
 * max(min_pixels, min(total_max * temporal_patch_size // n_sampled,
 * max_pixels)).  total_max is the video's total pixel budget (the pages do
 * not print a default).  Returns the ceiling, or MIMO_E_INVALID.
 */
int64_t mimo_video_max_pixels(int64_t n_sampled, int64_t total_max, const mimo_params *params);

/*
 * cortiq smart_nframes: frame count for `total` source frames at fps_src
 * sampled at fps: total / fps_src * fps, held inside [min_frames,
 * max_frames], then capped at total, then rounded down to an even count.  Returns the
 * count, or MIMO_E_INVALID.
 */
int64_t mimo_smart_nframes(int64_t total, double fps_src, double fps, int64_t min_frames,
                           int64_t max_frames);

/*
 * cortiq sample_frames: indices unique(int64(linspace(0, total - 1, n))) and
 * timestamps float32(index) / fps_src.  idx (int64) and ts (float) are host
 * arrays of at least n entries.  Returns the number of indices written, or
 * MIMO_E_INVALID.
 */
int64_t mimo_sample_frames(int64_t total, int64_t n, double fps_src, int64_t *idx, float *ts);

/*
 * Statistics in 0-255 units (processing page, MimoV2ImageProcessor: the
 * image_mean / image_std it is given are 0-1 values, and standardisation
 * runs on 0-255 floats with mean and std scaled by 255).
 *   mean01, std01    host double[3]: the processor's per-channel statistics.
 *   mean255, std255  host float[3]: float32(255 * v), the product formed in
 *                    float64 and rounded once -- what mimo_preprocess_batch
 *                    takes.
 * Host only.  Returns MIMO_OK, or MIMO_E_INVALID for a null pointer, a
 * non-finite value or std <= 0 (outputs untouched).
 */
int mimo_stats255(const double *mean01, const double *std01, float *mean255, float *std255);

/* Bytes of device workspace mimo_preprocess_batch / mimo_column_permute need
 * for n images (descriptor tables copied from the host on each call). */
size_t mimo_workspace_bytes(int32_t n);

/*
 * The fused pixel path for a whole batch: flatten, cast, bilinear resize,
 * standardise, two frames, patch rows -- one kernel launch (after one
 * asynchronous host-to-device copy of the descriptor tables into the
 * workspace).
 *   n, desc      host: the plan from mimo_plan_geometry (params must be the
 *                defaults' patch/merge/temporal sizes).  Images whose status
 *                is not MIMO_OK are skipped.
 *   src          device: packed uint8 sources, 4-byte aligned.
 *   src_capacity bytes readable at src; must be >= the packed size rounded
 *                up to a multiple of 16 (the kernels read whole 16-byte
 *                words; bytes past the images are read and ignored).
 *   mean255, std255  host float[3]: per-channel statistics in 0-255 units
 *                (255 * mean, 255 * std); std255 > 0.
 *   out_dtype    MIMO_F32 or MIMO_BF16.
 *   rows         device, nullable: [capacity_rows][1536] merge-block order.
 *   rows_col     device, nullable: [capacity_rows][1536] column order.  At
 *                least one of rows / rows_col is non-null.  16-byte aligned.
 *   capacity_rows rows available in each non-null output (>= total rows).
 *   workspace    device, >= mimo_workspace_bytes(n) bytes, 16-byte aligned;
 *                must stay untouched until the kernel has run.
 *   stream       hipStream_t.
 * Returns MIMO_OK, MIMO_E_INVALID, MIMO_E_UNSUPPORTED, MIMO_E_CAPACITY,
 * MIMO_E_TOO_LARGE or MIMO_E_HIP.
 */
int mimo_preprocess_batch(int32_t n, const mimo_image_desc *desc, const uint8_t *src,
                          int64_t src_capacity, const float *mean255, const float *std255,
                          int32_t out_dtype, void *rows, void *rows_col, int64_t capacity_rows,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * mimo_preprocess_batch for callers that cannot allocate memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc:
 * the same kernel, with the descriptor tables kept in a device scratch array
 * inside the library instead of a caller's workspace.  Neither this call nor
 * anything it calls allocates: the scratch is static device memory of
 * MIMO_NOALLOC_SCRATCH_BYTES (640.5 KiB) per GPU, held until the process
 * ends, and the host hands the tables over in the arguments of small copy
 * kernels (one per 3 KB of table, on `stream`, before the main kernel).
 *   n   at most MIMO_NOALLOC_MAX_IMAGES images; more returns
 *       MIMO_E_CAPACITY before anything is enqueued.
 * Other arguments, results and errors as for mimo_preprocess_batch.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's tables: calls on one stream are ordered and safe, but calls that
 * overlap on one GPU (several streams, or host threads on different
 * streams) race on the scratch and must be serialised by the caller.
 */
#define MIMO_NOALLOC_MAX_IMAGES 8192
#define MIMO_NOALLOC_SCRATCH_BYTES 655872 /* mimo_workspace_bytes(MIMO_NOALLOC_MAX_IMAGES) */
int mimo_preprocess_batch_noalloc(int32_t n, const mimo_image_desc *desc, const uint8_t *src,
                                  int64_t src_capacity, const float *mean255, const float *std255,
                                  int32_t out_dtype, void *rows, void *rows_col, int64_t capacity_rows,
                                  void *stream);

/*
 * column_permutation (cortiq mimo_vision): for one image with grid
 * (grid_t, grid_h, grid_w) and merge size m, perm[dst] = src lists the merge
 * units by (t, block col, block row), each unit's m*m rows kept together.
 * Host only.  perm: host int64 [grid_t*grid_h*grid_w].  Returns MIMO_OK or
 * MIMO_E_INVALID (non-positive sizes, grid not divisible by m).
 */
int mimo_column_permutation(int64_t grid_t, int64_t grid_h, int64_t grid_w, int64_t merge,
                            int64_t *perm);

/*
 * Gather kernel: rows_out[row_offset_i + d] = rows_in[row_offset_i + perm_i[d]]
 * for every image i (perm_i from mimo_column_permutation), i.e. merge-order
 * rows -> column-order rows.  Not in place (rows_out != rows_in).
 *   n, desc      host plan (as for mimo_preprocess_batch).
 *   rows_in, rows_out  device [capacity_rows][1536] of out_dtype, 16-byte aligned.
 *   workspace    device, >= mimo_workspace_bytes(n).
 * Returns MIMO_OK, MIMO_E_INVALID, MIMO_E_CAPACITY or MIMO_E_HIP.
 */
int mimo_column_permute(int32_t n, const mimo_image_desc *desc, const void *rows_in,
                        void *rows_out, int32_t out_dtype, int64_t capacity_rows,
                        void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * ViT index tables.  NeMo Automodel "mimo_v2_flash.vision":
 * MiMoVisionRotaryEmbedding(dim, theta = 10000) with dim = head_dim / 2,
 * MiMoVisionTransformer._rotary_positions, _get_window_index(grid_thw,
 * column_major) and _apply_merge_index; docs.rs "cortiq_engine::mimo_vision"
 * module conventions: type-1 window blocks run in column order, the RoPE
 * tables follow the same permutation as the rows, and no two frames share a
 * chunk.  They describe the rows mimo_preprocess_batch emits, in either
 * order, so a consumer can run rotary attention on them directly.
 * ------------------------------------------------------------------------ */

#define MIMO_ORDER_MERGE 0   /* rows in merge-block order (t, block row, block col, mh, mw) */
#define MIMO_ORDER_COLUMN 1  /* rows in column order (t, block col, block row, mh, mw) */
#define MIMO_ROPE_DIM_MAX 256

/*
 * inv_freq of MiMoVisionRotaryEmbedding(rope_dim, theta): rope_dim / 2
 * floats theta^-(2i / rope_dim), evaluated as a float32 module does (float32
 * exponent, power rounded to float32, reciprocal rounded to float32).
 *   inv  host [rope_dim / 2].
 * Returns MIMO_OK, or MIMO_E_INVALID unless rope_dim is even, in [2,
 * MIMO_ROPE_DIM_MAX], and theta > 1.
 */
int mimo_rope_inv_freq(int32_t rope_dim, double theta, float *inv);

/*
 * Rotary tables of every row of a planned batch, in the order the rows are
 * emitted (one kernel launch, after one table upload).  Row r of item i
 * (global index row_offset_i + r) covers the patch at grid position (h, w):
 * h = 2 * block row + mh, w = 2 * block col + mw of that row, whatever t.
 *   n, desc    host plan (mimo_plan_geometry / mimo_plan_frames); items with
 *              a non-zero status are skipped.
 *   order      MIMO_ORDER_MERGE or MIMO_ORDER_COLUMN.
 *   rope_dim   table width: a multiple of 8 in [8, MIMO_ROPE_DIM_MAX]
 *              (head_dim / 2 of the tower; 32 for head_dim 64).
 *   theta      rotary base (10000 in the tower).
 *   pos_hw     device int32 [rows][2] (h, w), 8-byte aligned, or NULL.
 *   rope_cos, rope_sin  device float32 [rows][rope_dim], or NULL: column k <
 *              rope_dim / 2 holds cos / sin of float32(h * inv_freq[k]),
 *              column rope_dim / 2 + k the same for w (the h half, then the w
 *              half, as the positions index the frequency table).  16-byte
 *              aligned.
 *   capacity_rows  rows the outputs hold (>= the plan's total).
 *   workspace  device, >= mimo_workspace_bytes(n), 16-byte aligned.
 * At least one output must be given.  Returns MIMO_OK, MIMO_E_INVALID,
 * MIMO_E_CAPACITY, MIMO_E_TOO_LARGE (an item with more than 2^24 rows, or
 * more than 2^31 - 1 workgroup tiles) or MIMO_E_HIP.
 */
int mimo_rotary_tables(int32_t n, const mimo_image_desc *desc, int32_t order, int32_t rope_dim,
                       double theta, int32_t *pos_hw, float *rope_cos, float *rope_sin,
                       int64_t capacity_rows, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * Merge-unit index of a planned batch for the windowed blocks
 * (_get_window_index): units are the 4-row groups of the merge-order rows,
 * numbered globally (unit u = rows 4u .. 4u + 3).  index[dst] = src: with
 * column_major = 0 the identity; with column_major = 1, within each item and
 * temporal slice, units listed by (block col, block row) -- the unit-level
 * form of mimo_column_permutation.  inverse[src] = dst undoes it.
 * Applying it (_apply_merge_index) is a gather of whole units.
 *   index, inverse  device int64 [units], 8-byte aligned; either may be NULL
 *              (not both).
 *   capacity_units  entries the outputs hold (>= total rows / 4).
 *   workspace  device, >= mimo_workspace_bytes(n), 16-byte aligned.
 * Returns MIMO_OK, MIMO_E_INVALID, MIMO_E_CAPACITY, MIMO_E_TOO_LARGE (as for
 * mimo_rotary_tables) or MIMO_E_HIP.
 */
int mimo_window_index(int32_t n, const mimo_image_desc *desc, int32_t column_major,
                      int64_t *index, int64_t *inverse, int64_t capacity_units, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * Attention chunk boundaries (host): every temporal slice of every item is
 * its own chunk of grid_h * grid_w rows.  cu[0] = 0, cu[k + 1] = cu[k] +
 * rows of chunk k, over the items with status MIMO_OK in batch order.
 *   cu  host int32 [capacity]; needs sum(grid_t) + 1 entries.
 * Returns the number of chunks, MIMO_E_INVALID, MIMO_E_CAPACITY, or
 * MIMO_E_TOO_LARGE if a boundary exceeds 2^31 - 1.
 */
int64_t mimo_chunk_seqlens(int32_t n, const mimo_image_desc *desc, int32_t *cu, int64_t capacity);

/* ------------------------------------------------------------------------
 * Stock-HF contrast path.  NeMo Automodel "mimo_v2_flash.processing", module
 * docstring: the stock Qwen2-VL processor that AutoProcessor resolves for
 * these checkpoints drops alpha, resizes with PIL's antialiased bicubic back
 * to bytes, normalises in 0-1 units, and its smart_resize clamps each side
 * on its own instead of scaling a short side up first.  The page calls these
 * the wrong pixels for the model; they are here so the shift can be measured
 * and reproduced.
 * ------------------------------------------------------------------------ */

/* The stock smart_resize (round each side to the factor; shrink with floor,
 * each side at least one factor; grow with ceil; aspect guard always).
 * Returns MIMO_OK, MIMO_E_INVALID, MIMO_E_ASPECT or MIMO_E_TOO_LARGE. */
int mimo_hf_smart_resize(int64_t h, int64_t w, const mimo_params *params, int64_t *out_h,
                         int64_t *out_w);

/* mimo_plan_geometry with the stock geometry (frames = 1, grid_t = 1). */
int mimo_plan_hf(int32_t n, const int32_t *hwc, const mimo_params *params, mimo_image_desc *out,
                 int64_t *total_rows, int64_t *total_src_bytes);

/* Device workspace bytes mimo_preprocess_hf_batch needs for this plan (the
 * per-item records, a normalisation table, and the resize taps). */
size_t mimo_hf_workspace_bytes(int32_t n, const mimo_image_desc *desc);

/*
 * The stock processor's pixels for a planned batch (mimo_plan_hf), one
 * kernel launch after one upload of the tables.  Alpha is ignored; each
 * resampled axis uses PIL's antialiased bicubic with 22-bit fixed-point
 * weights and a rounded byte result (horizontal first, each pass only if
 * that side changes); bytes v become float32(float64(v) / 255), then
 * (x - mean01[c]) / std01[c] in float32; rows as mimo_preprocess_batch
 * writes them (two identical frames, either or both orders).  Results equal
 * the stock processor's bit for bit.
 *   mean01, std01  host float[3], statistics in 0-1 units.
 *   workspace      device, >= mimo_hf_workspace_bytes(n, desc), 16-byte aligned.
 * Other arguments as for mimo_preprocess_batch.  Returns MIMO_OK,
 * MIMO_E_INVALID, MIMO_E_CAPACITY, MIMO_E_UNSUPPORTED (a downscale beyond
 * the kernel's LDS band: one output row's taps over more than 256 source
 * rows, or one tile's 32 output columns over more than 4096 source
 * columns),
 * MIMO_E_TOO_LARGE or MIMO_E_HIP.
 */
int mimo_preprocess_hf_batch(int32_t n, const mimo_image_desc *desc, const uint8_t *src,
                             int64_t src_capacity, const float *mean01, const float *std01,
                             int32_t out_dtype, void *rows, void *rows_col, int64_t capacity_rows,
                             void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Patch embedding.  NeMo Automodel "mimo_v2_flash.vision",
 * MiMoVisionPatchEmbed: the rows' consumer, a Conv3d whose kernel and stride
 * are both (T, P, P) = (2, 16, 16), so each row is one window and the
 * convolution is out[r][e] = bias[e] + sum_k rows[r][k] * W[e][k] with the
 * weight [E][3][2][16][16] flattened in the rows' (c, tt, py, px) order.
 * Runs on the matrix cores in bf16 with float32 accumulation.
 * ------------------------------------------------------------------------ */

/*
 * Folded weight for rows whose two temporal slots are equal (still images):
 * w_folded[e][c][p] = bf16(W[e][c][0][p] + W[e][c][1][p]) (sum in float32,
 * one rounding to nearest even), so the embedding needs K = 768 instead of
 * 1536 (mimo_patch_embed with folded = 1).
 *   w         device bf16 [embed_dim][1536], 16-byte aligned.
 *   w_folded  device bf16 [embed_dim][768], 16-byte aligned, not w.
 * One kernel launch.  Returns MIMO_OK, MIMO_E_INVALID or MIMO_E_HIP.
 */
int mimo_fold_patch_weights(int32_t embed_dim, const void *w, void *w_folded, void *stream);

/*
 * out = rows * W^T (+ bias) for n_rows rows, one kernel launch.
 *   rows       device bf16 [n_rows][1536] (mimo_preprocess_batch output with
 *              MIMO_BF16, either row order), 16-byte aligned.
 *   embed_dim  E: a multiple of 256 in [256, 65536].
 *   w          device bf16 [E][1536] (folded = 0), or the folded weight
 *              [E][768] (folded = 1: only the tt = 0 half of every row is
 *              read, which is exact only for rows whose two frames are
 *              equal), 16-byte aligned.
 *   bias       device float32 [E], 16-byte aligned, or NULL.
 *   out        device [n_rows][E] of out_dtype (MIMO_F32 or MIMO_BF16,
 *              rounded to nearest even), 16-byte aligned.
 * Returns MIMO_OK, MIMO_E_INVALID, MIMO_E_TOO_LARGE or MIMO_E_HIP.
 */
int mimo_patch_embed(int64_t n_rows, const void *rows, int32_t embed_dim, const void *w,
                     int32_t folded, const float *bias, int32_t out_dtype, void *out,
                     void *stream);

/* ------------------------------------------------------------------------
 * The pixel path and the patch embedding in one kernel, for still images:
 * NeMo Automodel "mimo_v2_flash.vision", MiMoVisionPatchEmbed, applied to the
 * rows of NeMo Automodel "mimo_v2_flash.processing", MimoV2ImageProcessor,
 * without writing the rows.  A still image's two frames are equal, so the
 * weight's two temporal halves are summed (K = 768); the standardisation is
 * affine, so it moves into the weight and bias:
 *   sum_k a_k W'_k = sum_k x_k (s_c W'_k) - sum_k mean255[c] (s_c W'_k),
 * a = (x - mean255[c]) * s_c, s_c = 1 / std255[c], x the resized 0-255 value.
 * ------------------------------------------------------------------------ */

/*
 * Prepares the weight and bias for mimo_pixel_embed (one kernel launch):
 *   w_pixels[e][(py*16 + px)*3 + c] = bf16(s_c * (W[e][c][0][py][px] + W[e][c][1][py][px]))
 *     (sum and product in float32, s_c = float32(1 / std255[c]), one rounding
 *     to nearest even) -- the (py, px, c) order of the source bytes;
 *   bias_pixels[e] = bias[e] - sum_k mean255[c(k)] * w_pixels[e][k]
 *     (float64, rounded once to float32; bias NULL counts as zeros).
 *   w           device bf16 [embed_dim][1536] (the Conv3d weight flattened as
 *               (c, tt, py, px)), 16-byte aligned.
 *   bias        device float32 [embed_dim], or NULL.
 *   mean255, std255  host float[3], 0-255 units (mimo_stats255); std255 > 0.
 *   w_pixels    device bf16 [embed_dim][768], 16-byte aligned, not w.
 *   bias_pixels device float32 [embed_dim].
 * Returns MIMO_OK, MIMO_E_INVALID or MIMO_E_HIP.
 */
int mimo_prepare_pixel_embed(int32_t embed_dim, const void *w, const float *bias, const float *mean255,
                             const float *std255, void *w_pixels, float *bias_pixels, void *stream);

/*
 * Patch embeddings of a planned batch of still images straight from their
 * packed uint8 sources: out[r][e] = bias_pixels[e] + sum_k bf16(x_r[k]) *
 * w_pixels[e][k] over the 768 resized 0-255 values x_r of row r's patch in
 * (py, px, c) order (RGBA flattened onto white, the bilinear resize of
 * mimo_preprocess_batch in float32, then one rounding to bf16 -- exact for an
 * image whose smart_resize target is its own size), float32 accumulation on
 * the matrix cores.  Rows in merge-block order, as mimo_preprocess_batch
 * lists them.  One kernel launch after one table upload; no pixel row is
 * written.
 *   n, desc      host plan (mimo_plan_geometry); items must be still images
 *                (frames = 1), else MIMO_E_UNSUPPORTED.
 *   src, src_capacity  as for mimo_preprocess_batch.
 *   embed_dim    E: a multiple of 256 in [256, 65536].
 *   w_pixels, bias_pixels  from mimo_prepare_pixel_embed (16-byte aligned).
 *   out          device [capacity_rows][E] of out_dtype (MIMO_F32 or
 *                MIMO_BF16, rounded to nearest even), 16-byte aligned.
 *   workspace    device, >= mimo_workspace_bytes(n), 16-byte aligned.
 * A batch whose every item is RGB and not resampled runs the fast producer
 * (source bytes straight into the matrix-core tiles); any other batch runs
 * a producer that evaluates each value from global memory (correct, slower).
 * Returns MIMO_OK, MIMO_E_INVALID, MIMO_E_UNSUPPORTED, MIMO_E_CAPACITY,
 * MIMO_E_TOO_LARGE (more than 2^31 - 1 tiles, or one tile's images spanning
 * more than 2^31 source bytes) or MIMO_E_HIP.
 */
int mimo_pixel_embed(int32_t n, const mimo_image_desc *desc, const uint8_t *src, int64_t src_capacity,
                     int32_t embed_dim, const void *w_pixels, const float *bias_pixels, int32_t out_dtype,
                     void *out, int64_t capacity_rows, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * Instrumentation.  When start and stop are non-null hipEvent_t handles
 * (passed as void*), every later kernel launch that the library makes on the
 * calling thread records `start` on the launch stream immediately before
 * the kernel and `stop` immediately after it, so the pair times the kernel
 * alone (the descriptor upload falls outside).  NULL, NULL switches it off.
 * Thread-local; the caller owns the events.  Returns MIMO_OK, or MIMO_E_INVALID if only one is null.
 */
int mimo_set_launch_events(void *start, void *stop);

/* Static text for a status code. */
const char *mimo_status_string(int status);

/* Message for the last failure on the calling thread ("" if none). */
const char *mimo_last_error(void);

/* Number of kernel launches this process has made through the library (a
 * proof that timings come from the GPU path). */
int64_t mimo_dispatch_count(void);

/* Number of mimo_preprocess_hf_batch launches that ran the contrast kernel's
 * matrix-core instance (every resized tile within 64 source columns and 64
 * band rows, at most 12 taps per output on each axis) rather than its
 * dot-product instance.  A diagnostic: both give the same bytes. */
int64_t mimo_hf_matrix_dispatch_count(void);

#ifdef __cplusplus
}
#endif

#endif /* MIMO_PRE_H */
