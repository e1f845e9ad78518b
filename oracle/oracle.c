/*
 * oracle.c -- plain, slow CPU oracle of the MiMo-V2 image pixel path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library under vision_image_preprocessing_amd/) never calls it and
 * shares no code, header, table or helper with it.
 *
 * Every function follows the definition on the pages, step by step, with
 * materialised intermediates and no blocking or fusion:
 *
 *   - NeMo Automodel "nemo_automodel.components.models.mimo_v2_flash.processing"
 *     (module docstring; MimoV2ImageProcessor class docstring and defaults;
 *      smart_resize; _to_rgb; get_number_of_image_patches),
 *   - docs.rs "cortiq_engine::mimo_vision" (module conventions list;
 *      resize_bilinear; column_permutation; smart_resize; the video helpers
 *      prepare_video_frames, smart_nframes, sample_frames, video_max_pixels),
 *   - the processing page's module docstring for the stock-HF contrast path
 *     (PIL bicubic with antialias, uint8 round trip, 0-1 normalisation),
 *   - NeMo Automodel "nemo_automodel.components.models.mimo_v2_flash.vision"
 *     (MiMoVisionRotaryEmbedding; MiMoVisionTransformer._rotary_positions,
 *      _get_window_index, _apply_merge_index) for the ViT index tables.
 *
 * Precision: the pages fix the resize as torch F.interpolate(bilinear,
 * align_corners=False) on a float32 tensor of 0-255 values, so the resize and
 * standardisation are carried out in float32 with the coordinate and weight
 * arithmetic torch uses (fp32 scale, single-rounded fused multiply-add for the
 * source coordinate, fp32 weights, W taps nested inside H taps).  Geometry is
 * done in float64 exactly as Python evaluates it.  Build with
 * -ffp-contract=off so that the only fused operations are the explicit fmaf.
 *
 * Parity pins (tests/test_oracle_*.py): geometry against the transformers
 * Qwen2-VL smart_resize and hand-derived cases; flatten against PIL on all
 * 65,536 (value, alpha) pairs; resize against torch CPU F.interpolate and
 * against a float64 evaluation within a derived bound; layout against a
 * coded image and a tensor reshape formulation; permutation against brute
 * force; bf16 rounding against torch; the stock-HF contrast path against
 * PIL's bicubic resize and transformers' Qwen2-VL processor and smart_resize,
 * bitwise; video helpers against numpy linspace
 * and hand-derived cases, frames against a torch composition; ViT tables
 * against reshapes, brute-force sorts, a coded image and torch's float32
 * inv_freq / outer product.  No function here is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_INVALID (-1)
#define ORC_E_ASPECT (-2)
#define ORC_E_DEGENERATE (-3)
#define ORC_E_NOMEM (-4)

/* ------------------------------------------------------------------------ */
/* Geometry: smart_resize with the MiMo / sglang semantics.                  */
/* ------------------------------------------------------------------------ */

/* Python's built-in round() on a float: nearest integer, ties to even. */
static double py_round(double v)
{
    double f = floor(v);
    double frac = v - f;
    if (frac < 0.5)
        return f;
    if (frac > 0.5)
        return f + 1.0;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/*
 * smart_resize(height, width, factor, min_pixels, max_pixels) -> (h, w).
 *
 * processing page, smart_resize: the Qwen2-VL algorithm (round each side to
 * a multiple of factor; if the area is above max_pixels shrink by
 * beta = sqrt(h*w/max) and floor; if below min_pixels grow by
 * beta = sqrt(min/(h*w)) and ceil) with two changes:
 *   (i)  a short side below factor is first scaled up to factor, both sides
 *        by the same ratio, and that branch skips the aspect guard;
 *   (ii) a shrink that floors a side to zero is rejected, not clamped.
 * Readings where the pages are silent: the aspect guard rejects a long/short
 * ratio strictly above max_aspect (200 in the Qwen2-VL routine); the
 * upscaled sides are the exact ratios side*factor/short, rounded once to
 * float64, and they replace the originals in every later step.
 */
int oracle_smart_resize(int64_t height, int64_t width, int64_t factor,
                        int64_t min_pixels, int64_t max_pixels,
                        double max_aspect, int64_t *out_h, int64_t *out_w)
{
    if (height < 1 || width < 1 || factor < 1 || min_pixels < 0 ||
        max_pixels < 1 || min_pixels > max_pixels)
        return ORC_E_INVALID;

    int64_t short_side = height < width ? height : width;
    int64_t long_side = height < width ? width : height;
    double h, w;
    if (short_side < factor) {
        /* upscale branch: the short side becomes exactly factor */
        h = (double)(height * factor) / (double)short_side;
        w = (double)(width * factor) / (double)short_side;
    } else {
        if ((double)long_side / (double)short_side > max_aspect)
            return ORC_E_ASPECT;
        h = (double)height;
        w = (double)width;
    }

    double f = (double)factor;
    double h_bar = py_round(h / f) * f;
    double w_bar = py_round(w / f) * f;
    if (h_bar * w_bar > (double)max_pixels) {
        double beta = sqrt(h * w / (double)max_pixels);
        h_bar = floor(h / beta / f) * f;
        w_bar = floor(w / beta / f) * f;
        if (h_bar == 0.0 || w_bar == 0.0)
            return ORC_E_DEGENERATE;
    } else if (h_bar * w_bar < (double)min_pixels) {
        double beta = sqrt((double)min_pixels / (h * w));
        h_bar = ceil(h * beta / f) * f;
        w_bar = ceil(w * beta / f) * f;
    }
    *out_h = (int64_t)h_bar;
    *out_w = (int64_t)w_bar;
    return ORC_OK;
}

/*
 * Grid, patch and token counts for one image.
 * get_number_of_image_patches: grid_h*grid_w patches before the merge**2
 * reduction; rows of pixel_values = grid_t*grid_h*grid_w; each image is
 * temporal_patch_size identical frames, so grid_t = 1; placeholder tokens
 * are patches / merge**2.
 */
int oracle_image_grid(int64_t height, int64_t width, int64_t patch,
                      int64_t merge, int64_t min_pixels, int64_t max_pixels,
                      double max_aspect, int64_t *grid_thw /* [3] */,
                      int64_t *rows, int64_t *tokens)
{
    int64_t rh, rw;
    int st = oracle_smart_resize(height, width, patch * merge, min_pixels,
                                 max_pixels, max_aspect, &rh, &rw);
    if (st != ORC_OK)
        return st;
    grid_thw[0] = 1;
    grid_thw[1] = rh / patch;
    grid_thw[2] = rw / patch;
    *rows = grid_thw[0] * grid_thw[1] * grid_thw[2];
    *tokens = *rows / (merge * merge);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Colour: RGBA flattened onto white (_to_rgb).                               */
/* ------------------------------------------------------------------------ */

/*
 * One channel of a pixel composited over an opaque white background with
 * coverage a/255, rounded to the nearest 8-bit value:
 *   out = value * a/255 + 255 * (1 - a/255).
 * The compositing happens on 8-bit pixels, before the float cast.
 */
static uint8_t flatten_on_white(uint8_t value, uint8_t alpha)
{
    double cover = (double)alpha / 255.0;
    double mixed = (double)value * cover + 255.0 * (1.0 - cover);
    return (uint8_t)floor(mixed + 0.5);
}

void oracle_flatten_rgba(const uint8_t *rgba, int64_t npix, uint8_t *rgb)
{
    for (int64_t i = 0; i < npix; ++i) {
        uint8_t a = rgba[4 * i + 3];
        for (int c = 0; c < 3; ++c)
            rgb[3 * i + c] = flatten_on_white(rgba[4 * i + c], a);
    }
}

/* ------------------------------------------------------------------------ */
/* Resize: F.interpolate(bilinear, align_corners=False), no antialias.       */
/* ------------------------------------------------------------------------ */

/*
 * Half-pixel source coordinate for destination index d on an axis mapped
 * from n_in to n_out samples, clamped below at zero, and its two taps:
 *   scale = n_in / n_out                     (float32 division)
 *   src   = scale * (d + 0.5) - 0.5          (one fused multiply-add)
 *   i0 = floor(src), l1 = src - i0, l0 = 1 - l1,
 *   i1 = i0 + 1, or i0 at the last sample.
 */
static void bilinear_tap(int64_t n_in, int64_t n_out, int64_t d, int64_t *i0,
                         int64_t *i1, float *l0, float *l1)
{
    float scale = (float)n_in / (float)n_out;
    float src = fmaf(scale, (float)d + 0.5f, -0.5f);
    if (src < 0.0f)
        src = 0.0f;
    float fl = floorf(src);
    int64_t lo = (int64_t)fl;
    if (lo > n_in - 1)
        lo = n_in - 1;
    *i0 = lo;
    *i1 = lo < n_in - 1 ? lo + 1 : lo;
    *l1 = src - (float)lo;
    *l0 = 1.0f - *l1;
}

/*
 * Planar float32 [C][H][W] -> [C][OH][OW].  For each output sample:
 * interpolate along W on the two source rows, then along H:
 *   t_y = l0x * v[y][x0] + l1x * v[y][x1]
 *   out = l0y * t_y0    + l1y * t_y1
 * each evaluated as fmaf(first weight, first value, second product).
 */
void oracle_resize_bilinear(const float *src, int64_t C, int64_t H, int64_t W,
                            float *dst, int64_t OH, int64_t OW)
{
    for (int64_t c = 0; c < C; ++c) {
        const float *plane = src + c * H * W;
        for (int64_t y = 0; y < OH; ++y) {
            int64_t y0, y1;
            float ly0, ly1;
            bilinear_tap(H, OH, y, &y0, &y1, &ly0, &ly1);
            for (int64_t x = 0; x < OW; ++x) {
                int64_t x0, x1;
                float lx0, lx1;
                bilinear_tap(W, OW, x, &x0, &x1, &lx0, &lx1);
                float top = fmaf(lx0, plane[y0 * W + x0],
                                 lx1 * plane[y0 * W + x1]);
                float bot = fmaf(lx0, plane[y1 * W + x0],
                                 lx1 * plane[y1 * W + x1]);
                dst[(c * OH + y) * OW + x] = fmaf(ly0, top, ly1 * bot);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* bf16: round to nearest, ties to even.                                      */
/* ------------------------------------------------------------------------ */

static float bits_to_float(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/*
 * The two bf16 values bracketing x are the float32 values whose low 16
 * mantissa bits are zero: truncation toward zero and the next one away from
 * zero.  Pick the nearer; on a tie pick the one with an even last bit.
 * (Inputs here are finite.)
 */
void oracle_to_bf16(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &x[i], 4);
        uint32_t toward = u >> 16;
        uint32_t away = toward + 1;
        double dx = (double)x[i];
        double d_toward = fabs(dx - (double)bits_to_float(toward << 16));
        double d_away = fabs((double)bits_to_float(away << 16) - dx);
        uint32_t pick;
        if (d_toward < d_away)
            pick = toward;
        else if (d_away < d_toward)
            pick = away;
        else
            pick = (toward & 1u) ? away : toward;
        out[i] = (uint16_t)pick;
    }
}

/* ------------------------------------------------------------------------ */
/* One image through the whole pixel path (_process_one / prepare_image).    */
/* ------------------------------------------------------------------------ */

/*
 * hwc: uint8 [H][W][C], C = 3 (RGB) or 4 (RGBA).  (OH, OW) is the
 * smart_resize target.  mean255/std255 are the per-channel statistics in
 * 0-255 units.  Output: (OH/patch)*(OW/patch) rows of
 * 3*temporal*patch*patch float32 values.
 *
 * Steps, in the order of the MimoV2ImageProcessor docstring:
 *  1. RGBA flattened onto white (RGB passes through);
 *  2. cast to float32, 0-255, planar [3][H][W];
 *  3. bilinear resize to [3][OH][OW];
 *  4. standardise (x - mean255[c]) / std255[c] in float32;
 *  5. duplicate the frame temporal times (T identical frames);
 *  6. patchify: row r = ((br*Bw + bc)*merge + mh)*merge + mw lists the patch
 *     at patch row br*merge+mh, patch column bc*merge+mw (merge-block order,
 *     (t, block row, block col, mh, mw)); element
 *     e = ((c*temporal + tt)*patch + py)*patch + px is the Conv3d kernel
 *     flattened as (c, tt, py, px).
 */
int oracle_preprocess_image(const uint8_t *hwc, int64_t H, int64_t W,
                            int64_t C, int64_t OH, int64_t OW, int64_t patch,
                            int64_t merge, int64_t temporal,
                            const float *mean255, const float *std255,
                            float *rows_out)
{
    if (H < 1 || W < 1 || (C != 3 && C != 4) || patch < 1 || merge < 1 ||
        temporal < 1 || OH % (patch * merge) != 0 || OW % (patch * merge) != 0 ||
        OH < 1 || OW < 1)
        return ORC_E_INVALID;

    int64_t npix = H * W;
    uint8_t *rgb = (uint8_t *)malloc((size_t)(npix * 3));
    float *planar = (float *)malloc(sizeof(float) * (size_t)(3 * npix));
    float *resized = (float *)malloc(sizeof(float) * (size_t)(3 * OH * OW));
    float *frames = (float *)malloc(sizeof(float) * (size_t)(temporal * 3 * OH * OW));
    if (!rgb || !planar || !resized || !frames) {
        free(rgb);
        free(planar);
        free(resized);
        free(frames);
        return ORC_E_NOMEM;
    }

    /* 1. colour */
    if (C == 4)
        oracle_flatten_rgba(hwc, npix, rgb);
    else
        memcpy(rgb, hwc, (size_t)(npix * 3));

    /* 2. cast, HWC -> planar CHW */
    for (int64_t c = 0; c < 3; ++c)
        for (int64_t i = 0; i < npix; ++i)
            planar[c * npix + i] = (float)rgb[3 * i + c];

    /* 3. resize */
    oracle_resize_bilinear(planar, 3, H, W, resized, OH, OW);

    /* 4. standardise */
    for (int64_t c = 0; c < 3; ++c)
        for (int64_t i = 0; i < OH * OW; ++i)
            resized[c * OH * OW + i] = (resized[c * OH * OW + i] - mean255[c]) / std255[c];

    /* 5. duplicate along the temporal axis */
    for (int64_t t = 0; t < temporal; ++t)
        memcpy(frames + t * 3 * OH * OW, resized, sizeof(float) * (size_t)(3 * OH * OW));

    /* 6. patchify in merge-block order */
    int64_t gh = OH / patch, gw = OW / patch;
    int64_t bh = gh / merge, bw = gw / merge;
    int64_t row_len = 3 * temporal * patch * patch;
    for (int64_t br = 0; br < bh; ++br)
        for (int64_t bc = 0; bc < bw; ++bc)
            for (int64_t mh = 0; mh < merge; ++mh)
                for (int64_t mw = 0; mw < merge; ++mw) {
                    int64_t r = ((br * bw + bc) * merge + mh) * merge + mw;
                    float *row = rows_out + r * row_len;
                    for (int64_t c = 0; c < 3; ++c)
                        for (int64_t tt = 0; tt < temporal; ++tt)
                            for (int64_t py = 0; py < patch; ++py)
                                for (int64_t px = 0; px < patch; ++px) {
                                    int64_t y = (br * merge + mh) * patch + py;
                                    int64_t x = (bc * merge + mw) * patch + px;
                                    int64_t e = ((c * temporal + tt) * patch + py) * patch + px;
                                    row[e] = frames[((tt * 3 + c) * OH + y) * OW + x];
                                }
                }

    free(rgb);
    free(planar);
    free(resized);
    free(frames);
    return ORC_OK;
}

/*
 * The same values as oracle_preprocess_image, computed one output element at
 * a time for a range of rows, without materialising the image.  Used to
 * check sampled rows of batches too large to run through the full path.
 */
static float source_value(const uint8_t *hwc, int64_t W, int64_t C, int64_t y,
                          int64_t x, int64_t c)
{
    const uint8_t *p = hwc + (y * W + x) * C;
    uint8_t v = C == 4 ? flatten_on_white(p[c], p[3]) : p[c];
    return (float)v;
}

int oracle_preprocess_rows(const uint8_t *hwc, int64_t H, int64_t W, int64_t C,
                           int64_t OH, int64_t OW, int64_t patch,
                           int64_t merge, int64_t temporal,
                           const float *mean255, const float *std255,
                           int64_t row_begin, int64_t row_count,
                           float *rows_out)
{
    if (H < 1 || W < 1 || (C != 3 && C != 4) || patch < 1 || merge < 1 ||
        temporal < 1 || OH % (patch * merge) != 0 || OW % (patch * merge) != 0)
        return ORC_E_INVALID;
    int64_t gh = OH / patch, gw = OW / patch;
    int64_t bw = gw / merge;
    int64_t unit = merge * merge;
    int64_t row_len = 3 * temporal * patch * patch;
    if (row_begin < 0 || row_count < 0 || row_begin + row_count > gh * gw)
        return ORC_E_INVALID;

    for (int64_t k = 0; k < row_count; ++k) {
        int64_t r = row_begin + k;
        /* invert r = ((br*bw + bc)*merge + mh)*merge + mw */
        int64_t block = r / unit, in_unit = r % unit;
        int64_t br = block / bw, bc = block % bw;
        int64_t mh = in_unit / merge, mw = in_unit % merge;
        float *row = rows_out + k * row_len;
        for (int64_t c = 0; c < 3; ++c)
            for (int64_t tt = 0; tt < temporal; ++tt)
                for (int64_t py = 0; py < patch; ++py)
                    for (int64_t px = 0; px < patch; ++px) {
                        int64_t y = (br * merge + mh) * patch + py;
                        int64_t x = (bc * merge + mw) * patch + px;
                        int64_t y0, y1, x0, x1;
                        float ly0, ly1, lx0, lx1;
                        bilinear_tap(H, OH, y, &y0, &y1, &ly0, &ly1);
                        bilinear_tap(W, OW, x, &x0, &x1, &lx0, &lx1);
                        float top = fmaf(lx0, source_value(hwc, W, C, y0, x0, c),
                                         lx1 * source_value(hwc, W, C, y0, x1, c));
                        float bot = fmaf(lx0, source_value(hwc, W, C, y1, x0, c),
                                         lx1 * source_value(hwc, W, C, y1, x1, c));
                        float v = fmaf(ly0, top, ly1 * bot);
                        int64_t e = ((c * temporal + tt) * patch + py) * patch + px;
                        row[e] = (v - mean255[c]) / std255[c];
                    }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* column_permutation (cortiq_engine::mimo_vision).                           */
/* ------------------------------------------------------------------------ */

/*
 * Rows of one image reordered into column order: merge units listed by
 * (t, block col, block row) instead of (t, block row, block col), each
 * unit's merge**2 rows kept together in their own order.  perm[dst] = src.
 */
int oracle_column_permutation(int64_t grid_t, int64_t grid_h, int64_t grid_w,
                              int64_t merge, int64_t *perm)
{
    if (grid_t < 1 || grid_h < 1 || grid_w < 1 || merge < 1 ||
        grid_h % merge != 0 || grid_w % merge != 0)
        return ORC_E_INVALID;
    int64_t bh = grid_h / merge, bw = grid_w / merge, unit = merge * merge;
    int64_t dst = 0;
    for (int64_t t = 0; t < grid_t; ++t)
        for (int64_t bc = 0; bc < bw; ++bc)
            for (int64_t br = 0; br < bh; ++br)
                for (int64_t k = 0; k < unit; ++k)
                    perm[dst++] = ((t * bh + br) * bw + bc) * unit + k;
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Video frames (cortiq_engine::mimo_vision: video_max_pixels, smart_nframes, */
/* sample_frames, prepare_video_frames).                                     */
/* ------------------------------------------------------------------------ */

/*
 * Per-frame pixel ceiling for n sampled frames:
 *   max(min_pixels, min(total_max * T // n, max_pixels)),
 * with T the temporal patch size and // floor division.
 */
int64_t oracle_video_max_pixels(int64_t n_sampled, int64_t total_max, int64_t temporal,
                                int64_t min_pixels, int64_t max_pixels)
{
    if (n_sampled < 1)
        return ORC_E_INVALID;
    int64_t per_frame = (total_max * temporal) / n_sampled;
    int64_t capped = per_frame < max_pixels ? per_frame : max_pixels;
    return capped > min_pixels ? capped : min_pixels;
}

/*
 * Frame count for `total` source frames at `fps_src` sampled at `fps`:
 * total / fps_src * fps, held inside [min_frames, max_frames], then to at
 * most total, then floored to an even count.
 */
int64_t oracle_smart_nframes(int64_t total, double fps_src, double fps, int64_t min_frames,
                             int64_t max_frames)
{
    if (total < 1 || !(fps_src > 0.0) || !(fps > 0.0) || min_frames > max_frames)
        return ORC_E_INVALID;
    double n = (double)total / fps_src * fps;
    if (n < (double)min_frames)
        n = (double)min_frames;
    if (n > (double)max_frames)
        n = (double)max_frames;
    if (n > (double)total)
        n = (double)total;
    return (int64_t)(floor(n / 2.0) * 2.0);
}

/*
 * Sampled frame indices unique(int64(linspace(0, total - 1, n))) and their
 * timestamps float32(idx) / fps_src.  linspace as numpy evaluates it:
 * step = (stop - start) / (n - 1), value_i = i * step + start, and the last
 * value set to stop exactly.  Returns the number of unique indices.
 */
int64_t oracle_sample_frames(int64_t total, int64_t n, double fps_src, int64_t *idx, float *ts)
{
    if (total < 1 || n < 1 || !(fps_src > 0.0))
        return ORC_E_INVALID;
    double start = 0.0, stop = (double)(total - 1);
    int64_t count = 0;
    for (int64_t i = 0; i < n; ++i) {
        double v;
        if (n == 1)
            v = start;
        else if (i == n - 1)
            v = stop;
        else
            v = (double)i * ((stop - start) / (double)(n - 1)) + start;
        int64_t k = (int64_t)v; /* truncation toward zero, as an int64 cast */
        /* values are non-decreasing: unique keeps the first of each run */
        if (count == 0 || idx[count - 1] != k)
            idx[count++] = k;
    }
    float fps32 = (float)fps_src;
    for (int64_t j = 0; j < count; ++j)
        ts[j] = (float)idx[j] / fps32;
    return count;
}

/*
 * prepare_video_frames, pixel part: n frames of one size (uint8 [H][W][C]
 * each, back to back), all resized to the same (OH, OW).  The frame list
 * is padded to a multiple of `temporal` by repeating the last frame; frame
 * f = t*temporal + tt forms temporal slot tt of temporal patch t.  Rows are
 * listed by (t, block row, block col, mh, mw); each row holds
 * (c, tt, py, px).  A single frame gives the image path (T identical
 * frames).
 */
int oracle_preprocess_video(const uint8_t *frames, int64_t n_frames, int64_t H, int64_t W,
                            int64_t C, int64_t OH, int64_t OW, int64_t patch, int64_t merge,
                            int64_t temporal, const float *mean255, const float *std255,
                            float *rows_out)
{
    if (n_frames < 1 || H < 1 || W < 1 || (C != 3 && C != 4) || patch < 1 || merge < 1 ||
        temporal < 1 || OH % (patch * merge) != 0 || OW % (patch * merge) != 0 || OH < 1 ||
        OW < 1)
        return ORC_E_INVALID;
    int64_t padded = (n_frames + temporal - 1) / temporal * temporal;
    int64_t npix = H * W;
    uint8_t *rgb = (uint8_t *)malloc((size_t)(npix * 3));
    float *planar = (float *)malloc(sizeof(float) * (size_t)(3 * npix));
    float *resized = (float *)malloc(sizeof(float) * (size_t)(padded * 3 * OH * OW));
    if (!rgb || !planar || !resized) {
        free(rgb);
        free(planar);
        free(resized);
        return ORC_E_NOMEM;
    }
    for (int64_t f = 0; f < padded; ++f) {
        int64_t src_f = f < n_frames ? f : n_frames - 1; /* repeat the last frame */
        const uint8_t *hwc = frames + src_f * npix * C;
        if (C == 4)
            oracle_flatten_rgba(hwc, npix, rgb);
        else
            memcpy(rgb, hwc, (size_t)(npix * 3));
        for (int64_t c = 0; c < 3; ++c)
            for (int64_t i = 0; i < npix; ++i)
                planar[c * npix + i] = (float)rgb[3 * i + c];
        float *out_f = resized + f * 3 * OH * OW;
        oracle_resize_bilinear(planar, 3, H, W, out_f, OH, OW);
        for (int64_t c = 0; c < 3; ++c)
            for (int64_t i = 0; i < OH * OW; ++i)
                out_f[c * OH * OW + i] = (out_f[c * OH * OW + i] - mean255[c]) / std255[c];
    }
    int64_t gt = padded / temporal;
    int64_t gh = OH / patch, gw = OW / patch;
    int64_t bh = gh / merge, bw = gw / merge;
    int64_t row_len = 3 * temporal * patch * patch;
    for (int64_t t = 0; t < gt; ++t)
        for (int64_t br = 0; br < bh; ++br)
            for (int64_t bc = 0; bc < bw; ++bc)
                for (int64_t mh = 0; mh < merge; ++mh)
                    for (int64_t mw = 0; mw < merge; ++mw) {
                        int64_t r = (((t * bh + br) * bw + bc) * merge + mh) * merge + mw;
                        float *row = rows_out + r * row_len;
                        for (int64_t c = 0; c < 3; ++c)
                            for (int64_t tt = 0; tt < temporal; ++tt)
                                for (int64_t py = 0; py < patch; ++py)
                                    for (int64_t px = 0; px < patch; ++px) {
                                        int64_t f = t * temporal + tt;
                                        int64_t y = (br * merge + mh) * patch + py;
                                        int64_t x = (bc * merge + mw) * patch + px;
                                        int64_t e = ((c * temporal + tt) * patch + py) * patch + px;
                                        row[e] = resized[((f * 3 + c) * OH + y) * OW + x];
                                    }
                    }
    free(rgb);
    free(planar);
    free(resized);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* ViT index tables (NeMo Automodel "...mimo_v2_flash.vision":               */
/* MiMoVisionTransformer._rotary_positions, _get_window_index,               */
/* _apply_merge_index, MiMoVisionRotaryEmbedding; docs.rs                    */
/* "cortiq_engine::mimo_vision" module conventions on window blocks).        */
/* ------------------------------------------------------------------------ */

/*
 * Rotary patch coordinates of every row of one item.  Rows are listed in
 * merge-block order (t, block row, block col, mh, mw), and the row's patch
 * sits at grid row h = block row * merge + mh and grid column
 * w = block col * merge + mw, whatever t.  In column order (column != 0)
 * the same coordinates follow the rows: pos_col[dst] = pos[perm[dst]] with
 * perm the column permutation.  pos[2r] = h, pos[2r + 1] = w.
 */
int oracle_rotary_positions(int64_t grid_t, int64_t grid_h, int64_t grid_w, int64_t merge,
                            int column, int32_t *pos)
{
    if (grid_t < 1 || grid_h < 1 || grid_w < 1 || merge < 1 ||
        grid_h % merge != 0 || grid_w % merge != 0)
        return ORC_E_INVALID;
    int64_t rows = grid_t * grid_h * grid_w;
    int32_t *merge_order = malloc((size_t)rows * 2 * sizeof(int32_t));
    if (!merge_order)
        return ORC_E_NOMEM;
    int64_t bh = grid_h / merge, bw = grid_w / merge, r = 0;
    for (int64_t t = 0; t < grid_t; ++t)
        for (int64_t br = 0; br < bh; ++br)
            for (int64_t bc = 0; bc < bw; ++bc)
                for (int64_t mh = 0; mh < merge; ++mh)
                    for (int64_t mw = 0; mw < merge; ++mw) {
                        merge_order[2 * r] = (int32_t)(br * merge + mh);
                        merge_order[2 * r + 1] = (int32_t)(bc * merge + mw);
                        ++r;
                    }
    if (!column) {
        memcpy(pos, merge_order, (size_t)rows * 2 * sizeof(int32_t));
        free(merge_order);
        return ORC_OK;
    }
    int64_t *perm = malloc((size_t)rows * sizeof(int64_t));
    if (!perm) {
        free(merge_order);
        return ORC_E_NOMEM;
    }
    int st = oracle_column_permutation(grid_t, grid_h, grid_w, merge, perm);
    if (st == ORC_OK)
        for (int64_t dst = 0; dst < rows; ++dst) {
            pos[2 * dst] = merge_order[2 * perm[dst]];
            pos[2 * dst + 1] = merge_order[2 * perm[dst] + 1];
        }
    free(perm);
    free(merge_order);
    return st;
}

/*
 * inv_freq of MiMoVisionRotaryEmbedding(dim, theta): dim / 2 entries
 * theta^-(2i / dim), as a float32 module evaluates them: the exponent
 * 2i / dim in float32, the power rounded to float32, then its reciprocal
 * rounded to float32.  The power is evaluated in float64, whose error is far
 * below half a float32 ulp, so it is the correctly rounded float32 power.
 */
int oracle_rope_inv_freq(int64_t dim, double theta, float *inv)
{
    if (dim < 2 || dim % 2 != 0 || !(theta > 1.0))
        return ORC_E_INVALID;
    for (int64_t i = 0; i < dim / 2; ++i) {
        float e = (float)(2 * i) / (float)dim;
        float p = (float)pow(theta, (double)e);
        inv[i] = 1.0f / p;
    }
    return ORC_OK;
}

/*
 * Rotary angles of every row and their cosine and sine: a row whose patch
 * sits at (h, w) gets, for k < dim / 2, the angle float32(h * inv[k]) in
 * column k and float32(w * inv[k]) in column dim / 2 + k (h half first,
 * then w half), the float32 outer product of positions and inv_freq.
 * cos and sin are taken in float64 of that float32 angle.
 */
int oracle_rope_tables(const int32_t *pos, int64_t rows, int64_t dim, const float *inv,
                       float *angle, double *cos_out, double *sin_out)
{
    if (rows < 0 || dim < 2 || dim % 2 != 0)
        return ORC_E_INVALID;
    int64_t half = dim / 2;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t axis = 0; axis < 2; ++axis) {
            float p = (float)pos[2 * r + axis];
            for (int64_t k = 0; k < half; ++k) {
                float a = p * inv[k];
                int64_t col = r * dim + axis * half + k;
                angle[col] = a;
                cos_out[col] = cos((double)a);
                sin_out[col] = sin((double)a);
            }
        }
    return ORC_OK;
}

/*
 * Merge-unit index of a batch for the windowed blocks: index[dst] = src over
 * the batch's merge units, numbered globally with the items back to back in
 * batch order and each item's units in merge-block order.  column_major = 0
 * keeps that order (the identity); column_major = 1 lists, within each item
 * and each temporal slice, the units by (block col, block row).  thw holds
 * (grid_t, grid_h, grid_w) per item.
 */
int oracle_window_index(int64_t n, const int64_t *thw, int64_t merge, int column_major,
                        int64_t *index)
{
    if (n < 0 || merge < 1)
        return ORC_E_INVALID;
    int64_t base = 0, dst = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t gt = thw[3 * i], gh = thw[3 * i + 1], gw = thw[3 * i + 2];
        if (gt < 1 || gh < 1 || gw < 1 || gh % merge != 0 || gw % merge != 0)
            return ORC_E_INVALID;
        int64_t bh = gh / merge, bw = gw / merge;
        for (int64_t t = 0; t < gt; ++t) {
            if (column_major) {
                for (int64_t bc = 0; bc < bw; ++bc)
                    for (int64_t br = 0; br < bh; ++br)
                        index[dst++] = base + (t * bh + br) * bw + bc;
            } else {
                for (int64_t br = 0; br < bh; ++br)
                    for (int64_t bc = 0; bc < bw; ++bc)
                        index[dst++] = base + (t * bh + br) * bw + bc;
            }
        }
        base += gt * bh * bw;
    }
    return ORC_OK;
}

/*
 * Attention chunks of a batch: every temporal slice of every item is its
 * own chunk of grid_h * grid_w rows (frames never share a chunk).
 * cu[0] = 0 and cu[k + 1] = cu[k] + rows of chunk k.  Returns the number of
 * chunks; cu must hold sum(grid_t) + 1 entries.
 */
int64_t oracle_chunk_seqlens(int64_t n, const int64_t *thw, int64_t *cu)
{
    if (n < 0)
        return ORC_E_INVALID;
    int64_t k = 0;
    cu[0] = 0;
    for (int64_t i = 0; i < n; ++i) {
        int64_t gt = thw[3 * i], gh = thw[3 * i + 1], gw = thw[3 * i + 2];
        if (gt < 1 || gh < 1 || gw < 1)
            return ORC_E_INVALID;
        for (int64_t t = 0; t < gt; ++t) {
            cu[k + 1] = cu[k] + gh * gw;
            ++k;
        }
    }
    return k;
}

/* ------------------------------------------------------------------------ */
/* Patch embedding (NeMo Automodel "...mimo_v2_flash.vision":                */
/* MiMoVisionPatchEmbed): a Conv3d whose kernel and stride are both          */
/* (T, P, P), applied to rows that are exactly one kernel window each.       */
/* ------------------------------------------------------------------------ */

/*
 * out[r][e] = bias[e] + sum over k of rows[r][k] * w[e][k], where w is the
 * Conv3d weight [embed_dim][C][T][P][P] flattened in the rows' own
 * (c, tt, py, px) order, so the convolution at the one window position is
 * this dot product.  Accumulated in float64 (the float inputs convert
 * exactly).  bias may be NULL.
 */
int oracle_patch_embed(const float *rows, int64_t n_rows, int64_t row_len, const float *w,
                       int64_t embed_dim, const float *bias, double *out)
{
    if (n_rows < 0 || row_len < 1 || embed_dim < 1)
        return ORC_E_INVALID;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int64_t e = 0; e < embed_dim; ++e) {
            double acc = bias ? (double)bias[e] : 0.0;
            for (int64_t k = 0; k < row_len; ++k)
                acc += (double)rows[r * row_len + k] * (double)w[e * row_len + k];
            out[r * embed_dim + e] = acc;
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Stock-HF contrast path (NeMo Automodel "mimo_v2_flash.processing", module */
/* docstring): the stock Qwen2-VL processor resizes with PIL bicubic         */
/* (antialiased, back to uint8), normalises in 0-1 units, drops alpha, and   */
/* its smart_resize clamps each side on its own instead of upscaling a short */
/* side first.                                                               */
/* ------------------------------------------------------------------------ */

/*
 * Stock smart_resize: round each side to the factor (ties to even); if the
 * area is above max_pixels shrink by beta = sqrt(h*w/max) with floor, each
 * side clamped to at least factor; else if below min_pixels grow by
 * beta = sqrt(min/(h*w)) with ceil.  Aspect above max_aspect is an error.
 */
int oracle_hf_smart_resize(int64_t h, int64_t w, int64_t factor, int64_t min_pixels,
                           int64_t max_pixels, double max_aspect, int64_t *out_h, int64_t *out_w)
{
    if (h < 1 || w < 1 || factor < 1 || min_pixels < 0 || max_pixels < 1)
        return ORC_E_INVALID;
    double hd = (double)h, wd = (double)w, f = (double)factor;
    double big = hd > wd ? hd : wd, small = hd > wd ? wd : hd;
    if (big / small > max_aspect)
        return ORC_E_ASPECT;
    double hb = py_round(hd / f) * f, wb = py_round(wd / f) * f;
    if (hb * wb > (double)max_pixels) {
        double beta = sqrt((hd * wd) / (double)max_pixels);
        hb = floor(hd / beta / f) * f;
        wb = floor(wd / beta / f) * f;
        if (hb < f)
            hb = f;
        if (wb < f)
            wb = f;
    } else if (hb * wb < (double)min_pixels) {
        double beta = sqrt((double)min_pixels / (hd * wd));
        hb = ceil(hd * beta / f) * f;
        wb = ceil(wd * beta / f) * f;
    }
    *out_h = (int64_t)hb;
    *out_w = (int64_t)wb;
    return ORC_OK;
}

/* Keys' cubic convolution kernel with a = -0.5 (the bicubic of PIL). */
static double keys_cubic(double x)
{
    const double a = -0.5;
    if (x < 0.0)
        x = -x;
    if (x < 1.0)
        return ((a + 2.0) * x - (a + 3.0)) * x * x + 1.0;
    if (x < 2.0)
        return (((x - 5.0) * x + 8.0) * x - 4.0) * a;
    return 0.0;
}

#define PIL_BITS 22 /* fractional bits of the 8-bit resampler's weights */

/*
 * Taps of one axis for PIL's antialiased bicubic, n_in -> n_out samples:
 * scale = n_in / n_out; the kernel is widened by max(scale, 1) (support
 * 2 * that); output i centred at (i + 0.5) * scale takes inputs
 * [first, first + count) with weights keys((j - centre + 0.5) / widening),
 * normalised to sum 1 and rounded half away from zero to PIL_BITS bits.
 * first[i], count[i], weight[i * ksize + j]; returns ksize.
 */
static int64_t pil_axis_taps(int64_t n_in, int64_t n_out, int64_t **first_out,
                             int64_t **count_out, int32_t **weight_out)
{
    double scale = (double)n_in / (double)n_out;
    double widen = scale < 1.0 ? 1.0 : scale;
    double support = 2.0 * widen;
    int64_t ksize = (int64_t)ceil(support) * 2 + 1;
    int64_t *first = malloc(sizeof(int64_t) * (size_t)n_out);
    int64_t *count = malloc(sizeof(int64_t) * (size_t)n_out);
    int32_t *weight = calloc((size_t)(n_out * ksize), sizeof(int32_t));
    double *k = malloc(sizeof(double) * (size_t)ksize);
    if (!first || !count || !weight || !k) {
        free(first);
        free(count);
        free(weight);
        free(k);
        return ORC_E_NOMEM;
    }
    for (int64_t i = 0; i < n_out; ++i) {
        double centre = ((double)i + 0.5) * scale;
        int64_t lo = (int64_t)(centre - support + 0.5);
        if (lo < 0)
            lo = 0;
        int64_t hi = (int64_t)(centre + support + 0.5);
        if (hi > n_in)
            hi = n_in;
        int64_t n = hi - lo;
        double total = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            k[j] = keys_cubic(((double)(j + lo) - centre + 0.5) / widen);
            total += k[j];
        }
        for (int64_t j = 0; j < n; ++j) {
            double v = total != 0.0 ? k[j] / total : k[j];
            double fixed = v * (double)(1 << PIL_BITS);
            weight[i * ksize + j] = (int32_t)(v < 0.0 ? fixed - 0.5 : fixed + 0.5);
        }
        first[i] = lo;
        count[i] = n;
    }
    free(k);
    *first_out = first;
    *count_out = count;
    *weight_out = weight;
    return ksize;
}

/* (acc + half) >> PIL_BITS clamped to a byte: the resampler's rounding. */
static uint8_t pil_round_clip(int32_t acc)
{
    int32_t v = (acc + (1 << (PIL_BITS - 1))) >> PIL_BITS;
    return (uint8_t)(v < 0 ? 0 : (v > 255 ? 255 : v));
}

/*
 * PIL's 8-bit antialiased bicubic resize of an interleaved uint8 image
 * [h][w][c] to [oh][ow][c]: a horizontal pass (only if ow != w) to bytes,
 * then a vertical pass (only if oh != h) to bytes, each output the rounded,
 * clamped fixed-point sum over its taps.
 */
int oracle_pil_resize_bicubic(const uint8_t *src, int64_t h, int64_t w, int64_t c, int64_t oh,
                              int64_t ow, uint8_t *dst)
{
    if (h < 1 || w < 1 || c < 1 || oh < 1 || ow < 1)
        return ORC_E_INVALID;
    uint8_t *mid = malloc((size_t)(h * ow * c));
    if (!mid)
        return ORC_E_NOMEM;
    if (ow != w) {
        int64_t *first, *count;
        int32_t *wt;
        int64_t ks = pil_axis_taps(w, ow, &first, &count, &wt);
        if (ks < 0) {
            free(mid);
            return (int)ks;
        }
        for (int64_t y = 0; y < h; ++y)
            for (int64_t x = 0; x < ow; ++x)
                for (int64_t ch = 0; ch < c; ++ch) {
                    int32_t acc = 0;
                    for (int64_t j = 0; j < count[x]; ++j)
                        acc += (int32_t)src[(y * w + first[x] + j) * c + ch] * wt[x * ks + j];
                    mid[(y * ow + x) * c + ch] = pil_round_clip(acc);
                }
        free(first);
        free(count);
        free(wt);
    } else {
        memcpy(mid, src, (size_t)(h * w * c));
    }
    if (oh != h) {
        int64_t *first, *count;
        int32_t *wt;
        int64_t ks = pil_axis_taps(h, oh, &first, &count, &wt);
        if (ks < 0) {
            free(mid);
            return (int)ks;
        }
        for (int64_t y = 0; y < oh; ++y)
            for (int64_t x = 0; x < ow; ++x)
                for (int64_t ch = 0; ch < c; ++ch) {
                    int32_t acc = 0;
                    for (int64_t j = 0; j < count[y]; ++j)
                        acc += (int32_t)mid[((first[y] + j) * ow + x) * c + ch] * wt[y * ks + j];
                    dst[(y * ow + x) * c + ch] = pil_round_clip(acc);
                }
        free(first);
        free(count);
        free(wt);
    } else {
        memcpy(dst, mid, (size_t)(oh * ow * c));
    }
    free(mid);
    return ORC_OK;
}

/*
 * The stock processor's pixel path for one image: the alpha channel (if any)
 * is dropped, the RGB bytes resized with PIL bicubic to (oh, ow), each byte
 * v rescaled as float32(float64(v) * (1 / 255)) and normalised in float32 as
 * (x - mean01[c]) / std01[c], then rows laid out as in the MiMo path
 * (T identical frames, (c, tt, py, px), merge-block order).
 */
int oracle_hf_preprocess_image(const uint8_t *src, int64_t h, int64_t w, int64_t c, int64_t oh,
                               int64_t ow, int64_t patch, int64_t merge, int64_t temporal,
                               const float *mean01, const float *std01, float *rows)
{
    if ((c != 3 && c != 4) || oh % (patch * merge) || ow % (patch * merge))
        return ORC_E_INVALID;
    uint8_t *rgb = malloc((size_t)(h * w * 3));
    uint8_t *res = malloc((size_t)(oh * ow * 3));
    float *planar = malloc(sizeof(float) * (size_t)(3 * oh * ow));
    if (!rgb || !res || !planar) {
        free(rgb);
        free(res);
        free(planar);
        return ORC_E_NOMEM;
    }
    for (int64_t i = 0; i < h * w; ++i)
        for (int64_t ch = 0; ch < 3; ++ch)
            rgb[i * 3 + ch] = src[i * c + ch];
    int st = oracle_pil_resize_bicubic(rgb, h, w, 3, oh, ow, res);
    if (st == ORC_OK) {
        const double rescale = 1.0 / 255.0;
        for (int64_t ch = 0; ch < 3; ++ch)
            for (int64_t i = 0; i < oh * ow; ++i) {
                float x = (float)((double)res[i * 3 + ch] * rescale);
                planar[ch * oh * ow + i] = (x - mean01[ch]) / std01[ch];
            }
        int64_t gh = oh / patch, gw = ow / patch, bh = gh / merge, bw = gw / merge;
        int64_t row_len = 3 * temporal * patch * patch, r = 0;
        for (int64_t br = 0; br < bh; ++br)
            for (int64_t bc = 0; bc < bw; ++bc)
                for (int64_t mh = 0; mh < merge; ++mh)
                    for (int64_t mw = 0; mw < merge; ++mw) {
                        float *row = rows + r * row_len;
                        int64_t y0 = (br * merge + mh) * patch, x0 = (bc * merge + mw) * patch;
                        for (int64_t ch = 0; ch < 3; ++ch)
                            for (int64_t tt = 0; tt < temporal; ++tt)
                                for (int64_t py = 0; py < patch; ++py)
                                    for (int64_t px = 0; px < patch; ++px)
                                        row[((ch * temporal + tt) * patch + py) * patch + px] =
                                            planar[ch * oh * ow + (y0 + py) * ow + x0 + px];
                        ++r;
                    }
    }
    free(rgb);
    free(res);
    free(planar);
    return st;
}
