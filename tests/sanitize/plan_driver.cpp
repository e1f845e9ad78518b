// plan_driver.cpp -- drives every host entry point of the planner
// (csrc/plan.cpp) over random and edge-case arguments, for a build with
// AddressSanitizer and UndefinedBehaviorSanitizer.  It checks no values
// (the parity tests do that); a sanitizer report or a non-zero exit fails it.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "mimo_pre.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;

uint64_t next_u64() {  // xorshift64
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return g_state;
}

int64_t uniform(int64_t lo, int64_t hi) { return lo + int64_t(next_u64() % uint64_t(hi - lo + 1)); }

uint64_t g_sum = 0;  // keeps every result observable (wraps)

void note(int64_t v) { g_sum = g_sum * 31u + uint64_t(v); }

void sizes(const mimo_params *p) {
    const int64_t edge[][2] = {{0, 5},       {-1, 5},         {1, 8193},      {32, 6401},
                               {1, 8192},    {16, 192},       {8, 500},       {31, 31},
                               {1, 64},      {1, 1},          {4000, 6000},   {8388607, 1},
                               {INT32_MAX, 3}, {INT64_MAX / 4, 7}, {1, INT64_MAX / 4}};
    for (const auto &e : edge) {
        int64_t oh = -9, ow = -9;
        note(mimo_smart_resize(e[0], e[1], p, &oh, &ow));
        note(oh + ow);
        note(mimo_hf_smart_resize(e[0], e[1], p, &oh, &ow));
        note(oh + ow);
    }
    for (int i = 0; i < 20000; ++i) {
        const int64_t h = i % 3 == 0 ? uniform(1, 40) : uniform(1, 9000);
        const int64_t w = i % 5 == 0 ? uniform(1, 40) : uniform(1, 9000);
        int64_t oh = 0, ow = 0;
        note(mimo_smart_resize(h, w, p, &oh, &ow));
        note(oh ^ ow);
        note(mimo_hf_smart_resize(h, w, p, &oh, &ow));
        note(oh ^ ow);
    }
    note(mimo_smart_resize(5, 5, p, nullptr, nullptr));
}

void plans(const mimo_params *p) {
    for (int batch = 0; batch < 40; ++batch) {
        const int32_t n = int32_t(uniform(0, 300));
        std::vector<int32_t> hwc(3 * size_t(n) + 1), fhwc(4 * size_t(n) + 1);
        std::vector<int64_t> ceil(size_t(n) + 1);
        for (int32_t i = 0; i < n; ++i) {
            hwc[3 * i] = int32_t(i % 7 == 0 ? uniform(-2, 40) : uniform(1, 5000));
            hwc[3 * i + 1] = int32_t(uniform(1, 5000));
            hwc[3 * i + 2] = int32_t(i % 11 == 0 ? uniform(0, 6) : uniform(3, 4));
            fhwc[4 * i] = int32_t(i % 13 == 0 ? uniform(-1, 1) : uniform(1, 9));
            fhwc[4 * i + 1] = hwc[3 * i];
            fhwc[4 * i + 2] = hwc[3 * i + 1];
            fhwc[4 * i + 3] = hwc[3 * i + 2];
            ceil[i] = i % 3 ? 0 : uniform(-5, 1 << 24);
        }
        std::vector<mimo_image_desc> desc(size_t(n) + 1);
        int64_t rows = 0, src = 0;
        note(mimo_plan_geometry(n, hwc.data(), p, desc.data(), &rows, &src));
        note(rows + src);
        note(mimo_plan_geometry(n, hwc.data(), nullptr, desc.data(), nullptr, nullptr));
        note(mimo_plan_frames(n, fhwc.data(), ceil.data(), p, desc.data(), &rows, &src));
        note(mimo_plan_frames(n, fhwc.data(), nullptr, p, desc.data(), &rows, &src));
        note(int64_t(mimo_workspace_bytes(n)));
        std::vector<int32_t> cu(size_t(n) * 5 + 2);
        note(mimo_chunk_seqlens(n, desc.data(), cu.data(), int64_t(cu.size())));
        note(mimo_chunk_seqlens(n, desc.data(), cu.data(), 1));
        note(mimo_plan_hf(n, hwc.data(), p, desc.data(), &rows, &src));
    }
    note(mimo_plan_geometry(-1, nullptr, p, nullptr, nullptr, nullptr));
    note(mimo_plan_geometry(3, nullptr, p, nullptr, nullptr, nullptr));
}

void helpers() {
    for (int i = 0; i < 3000; ++i) {
        const int64_t total = uniform(-2, 5000);
        const double fps_src = double(uniform(0, 120)) / 2.0, fps = double(uniform(0, 8)) / 2.0;
        note(mimo_smart_nframes(total, fps_src, fps, uniform(-1, 8), uniform(-1, 800)));
        note(mimo_video_max_pixels(uniform(-1, 900), uniform(-1, int64_t(1) << 30), nullptr));
        const int64_t n = uniform(-1, 300);
        std::vector<int64_t> idx(size_t(n > 0 ? n : 1));
        std::vector<float> ts(idx.size());
        note(mimo_sample_frames(total, n, fps_src, idx.data(), ts.data()));
        const int64_t gt = uniform(0, 3), gh = 2 * uniform(0, 20), gw = 2 * uniform(0, 20);
        std::vector<int64_t> perm(size_t(gt > 0 && gh > 0 && gw > 0 ? gt * gh * gw : 1));
        note(mimo_column_permutation(gt, gh, gw, 2, perm.data()));
        note(mimo_column_permutation(gt, gh + 1, gw, 2, perm.data()));
    }
    float inv[MIMO_ROPE_DIM_MAX];
    for (int d = -2; d <= MIMO_ROPE_DIM_MAX + 2; ++d) note(mimo_rope_inv_freq(d, 10000.0, inv));
    const double m[3] = {0.485, 0.456, 0.406}, s[3] = {0.229, 0.224, 0.225}, z[3] = {0.2, 0.0, 0.2};
    float m255[3], s255[3];
    note(mimo_stats255(m, s, m255, s255));
    note(mimo_stats255(m, z, m255, s255));
    note(mimo_stats255(nullptr, s, m255, s255));
    for (int code = 1; code >= -9; --code) note(int64_t(mimo_status_string(code)[0]));
    note(int64_t(mimo_last_error()[0]));
}

}  // namespace

int main() {
    mimo_params p;
    mimo_default_params(&p);
    sizes(&p);
    sizes(nullptr);
    mimo_params bad = p;
    bad.reserved0 = 1;
    sizes(&bad);
    plans(&p);
    helpers();
    std::printf("plan driver done %llu\n", static_cast<unsigned long long>(g_sum));
    return 0;
}
