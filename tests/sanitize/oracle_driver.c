/* oracle_driver.c -- drives the oracle's C functions (oracle/oracle.c) over
 * small random images and edge-case sizes, for a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer.  It checks no values (the oracle's pins do
 * that); a sanitizer report or a non-zero exit fails it. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_smart_resize(int64_t, int64_t, int64_t, int64_t, int64_t, double, int64_t *, int64_t *);
int oracle_image_grid(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, double, int64_t *,
                      int64_t *, int64_t *);
void oracle_flatten_rgba(const uint8_t *, int64_t, uint8_t *);
void oracle_to_bf16(const float *, int64_t, uint16_t *);
int oracle_preprocess_image(const uint8_t *, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                            int64_t, int64_t, const float *, const float *, float *);
int oracle_preprocess_rows(const uint8_t *, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                           int64_t, int64_t, const float *, const float *, int64_t, int64_t, float *);
int oracle_column_permutation(int64_t, int64_t, int64_t, int64_t, int64_t *);
int64_t oracle_video_max_pixels(int64_t, int64_t, int64_t, int64_t, int64_t);
int64_t oracle_smart_nframes(int64_t, double, double, int64_t, int64_t);
int64_t oracle_sample_frames(int64_t, int64_t, double, int64_t *, float *);
int oracle_preprocess_video(const uint8_t *, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                            int64_t, int64_t, int64_t, const float *, const float *, float *);
int oracle_rotary_positions(int64_t, int64_t, int64_t, int64_t, int, int32_t *);
int oracle_rope_inv_freq(int64_t, double, float *);
int oracle_rope_tables(const int32_t *, int64_t, int64_t, const float *, float *, double *, double *);
int oracle_window_index(int64_t, const int64_t *, int64_t, int, int64_t *);
int64_t oracle_chunk_seqlens(int64_t, const int64_t *, int64_t *);
int oracle_patch_embed(const float *, int64_t, int64_t, const float *, int64_t, const float *, double *);
int oracle_hf_smart_resize(int64_t, int64_t, int64_t, int64_t, int64_t, double, int64_t *, int64_t *);
int oracle_pil_resize_bicubic(const uint8_t *, int64_t, int64_t, int64_t, int64_t, int64_t, uint8_t *);
int oracle_hf_preprocess_image(const uint8_t *, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                               int64_t, int64_t, const float *, const float *, float *);

static uint64_t g_state = 0x2545F4914F6CDD1Dull;
static double g_sum = 0.0; /* keeps every result observable */

static uint64_t next_u64(void) /* xorshift64 */
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return g_state;
}

static int64_t uniform(int64_t lo, int64_t hi) { return lo + (int64_t)(next_u64() % (uint64_t)(hi - lo + 1)); }

static void *xmalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void image_case(int64_t h, int64_t w, int64_t c, int64_t oh, int64_t ow)
{
    const float m255[3] = {123.675f, 116.28f, 103.53f}, s255[3] = {58.395f, 57.12f, 57.375f};
    const float m01[3] = {0.485f, 0.456f, 0.406f}, s01[3] = {0.229f, 0.224f, 0.225f};
    uint8_t *img = xmalloc((size_t)(h * w * c));
    for (int64_t i = 0; i < h * w * c; ++i) img[i] = (uint8_t)next_u64();
    const int64_t rows = (oh / 16) * (ow / 16);
    float *out = xmalloc((size_t)rows * 1536 * sizeof(float));
    g_sum += oracle_preprocess_image(img, h, w, c, oh, ow, 16, 2, 2, m255, s255, out);
    g_sum += out[0] + out[rows * 1536 - 1];
    if (rows > 2) {
        g_sum += oracle_preprocess_rows(img, h, w, c, oh, ow, 16, 2, 2, m255, s255, 1, rows - 2, out);
        g_sum += out[(rows - 2) * 1536 - 1];
    }
    uint16_t *bf = xmalloc((size_t)rows * 1536 * sizeof(uint16_t));
    oracle_to_bf16(out, rows * 1536, bf);
    g_sum += bf[rows * 1536 - 1];
    if (c == 4) {
        uint8_t *rgb = xmalloc((size_t)(h * w * 3));
        oracle_flatten_rgba(img, h * w, rgb);
        g_sum += rgb[h * w * 3 - 1];
        free(rgb);
    }
    uint8_t *small = xmalloc((size_t)(oh * ow * c));
    g_sum += oracle_pil_resize_bicubic(img, h, w, c, oh, ow, small);
    g_sum += oracle_hf_preprocess_image(img, h, w, c, oh, ow, 16, 2, 2, m01, s01, out);
    g_sum += out[rows * 1536 - 1];
    /* three frames: an odd count, the last repeated */
    uint8_t *clip = xmalloc((size_t)(3 * h * w * c));
    for (int64_t i = 0; i < 3 * h * w * c; ++i) clip[i] = (uint8_t)next_u64();
    float *vout = xmalloc((size_t)(2 * rows) * 1536 * sizeof(float));
    g_sum += oracle_preprocess_video(clip, 3, h, w, c, oh, ow, 16, 2, 2, m255, s255, vout);
    g_sum += vout[2 * rows * 1536 - 1];
    free(vout);
    free(clip);
    free(small);
    free(bf);
    free(out);
    free(img);
}

int main(void)
{
    const int64_t edge[][2] = {{0, 5}, {1, 8193}, {32, 6401}, {1, 8192}, {16, 192}, {8, 500},
                               {31, 31}, {1, 64}, {4000, 6000}, {1, 1}};
    for (size_t i = 0; i < sizeof edge / sizeof edge[0]; ++i) {
        int64_t oh = -1, ow = -1, grid[3], rows, tok;
        g_sum += oracle_smart_resize(edge[i][0], edge[i][1], 32, 8192, 8388608, 200.0, &oh, &ow);
        g_sum += oracle_hf_smart_resize(edge[i][0], edge[i][1], 32, 8192, 8388608, 200.0, &oh, &ow);
        g_sum += oracle_image_grid(edge[i][0], edge[i][1], 16, 2, 8192, 8388608, 200.0, grid, &rows, &tok);
    }
    for (int i = 0; i < 5000; ++i) {
        int64_t oh, ow;
        g_sum += oracle_smart_resize(uniform(1, 9000), uniform(1, 9000), 32, 8192, 8388608, 200.0, &oh, &ow);
        g_sum += oracle_hf_smart_resize(uniform(1, 9000), uniform(1, 9000), 32, uniform(0, 9000),
                                        8388608, 200.0, &oh, &ow);
    }
    /* pixel paths on small images: resized to sizes around and off the source */
    for (int i = 0; i < 24; ++i) {
        const int64_t h = uniform(1, 90), w = uniform(1, 90), c = uniform(3, 4);
        const int64_t oh = 32 * uniform(1, 4), ow = 32 * uniform(1, 4);
        image_case(h, w, c, oh, ow);
    }
    image_case(64, 64, 3, 64, 64);
    /* permutation, video helpers, vision-tower tables, patch embedding */
    for (int i = 0; i < 200; ++i) {
        const int64_t gt = uniform(1, 3), gh = 2 * uniform(1, 12), gw = 2 * uniform(1, 12);
        int64_t *perm = xmalloc((size_t)(gt * gh * gw) * sizeof(int64_t));
        g_sum += oracle_column_permutation(gt, gh, gw, 2, perm);
        int32_t *pos = xmalloc((size_t)(gt * gh * gw) * 2 * sizeof(int32_t));
        g_sum += oracle_rotary_positions(gt, gh, gw, 2, i & 1, pos);
        float inv[16];
        g_sum += oracle_rope_inv_freq(32, 10000.0, inv);
        float *angle = xmalloc((size_t)(gt * gh * gw) * 32 * sizeof(float));
        double *cs = xmalloc((size_t)(gt * gh * gw) * 32 * sizeof(double));
        double *sn = xmalloc((size_t)(gt * gh * gw) * 32 * sizeof(double));
        g_sum += oracle_rope_tables(pos, gt * gh * gw, 32, inv, angle, cs, sn);
        const int64_t thw[6] = {gt, gh, gw, 1, 2, 4};
        int64_t *index = xmalloc((size_t)(gt * gh * gw / 4 + 2) * sizeof(int64_t));
        g_sum += oracle_window_index(2, thw, 2, i & 1, index);
        int64_t cu[8];
        g_sum += (double)oracle_chunk_seqlens(2, thw, cu);
        free(index);
        free(sn);
        free(cs);
        free(angle);
        free(pos);
        free(perm);
    }
    for (int i = 0; i < 300; ++i) {
        const int64_t total = uniform(1, 3000), n = uniform(1, 200);
        int64_t *idx = xmalloc((size_t)n * sizeof(int64_t));
        float *ts = xmalloc((size_t)n * sizeof(float));
        g_sum += (double)oracle_sample_frames(total, n, 30.0, idx, ts);
        g_sum += (double)oracle_smart_nframes(total, 30.0, 2.0, 4, 768);
        g_sum += (double)oracle_video_max_pixels(n, 1 << 24, 2, 8192, 8388608);
        free(ts);
        free(idx);
    }
    {
        const int64_t n = 9, k = 1536, e = 33;
        float *x = xmalloc((size_t)(n * k) * sizeof(float)), *wt = xmalloc((size_t)(e * k) * sizeof(float));
        float bias[33];
        double *out = xmalloc((size_t)(n * e) * sizeof(double));
        for (int64_t i = 0; i < n * k; ++i) x[i] = (float)(int64_t)(next_u64() % 512) / 256.0f - 1.0f;
        for (int64_t i = 0; i < e * k; ++i) wt[i] = (float)(int64_t)(next_u64() % 512) / 4096.0f;
        for (int64_t i = 0; i < e; ++i) bias[i] = (float)i;
        g_sum += oracle_patch_embed(x, n, k, wt, e, bias, out);
        g_sum += out[n * e - 1];
        free(out);
        free(wt);
        free(x);
    }
    printf("oracle driver done %.17g\n", g_sum);
    return 0;
}
