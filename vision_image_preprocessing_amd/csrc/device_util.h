// device_util.h -- small device helpers shared by the library's kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace mimo {

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

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

// n / d for 0 <= n < 2^24 and d >= 1, given inv = float(1 / d): the float
// estimate is within one of the quotient and is corrected exactly.
__device__ __forceinline__ int div_small(int n, int d, float inv) {
    int q = int(float(n) * inv);
    const int r = n - q * d;
    q += (r >= d) - (r < 0);
    return q;
}

// Tile order: workgroup b is dispatched to XCD b % 8; tile t = (b % 8) * per
// + b / 8 gives each XCD one contiguous run of tiles (and so of output
// rows), which keeps each XCD's write stream and its source reads local.
__device__ __forceinline__ int64_t xcd_contiguous_tile(int64_t b, int64_t grid) {
    const int64_t per = grid / kXcds;
    return b < per * kXcds ? (b % kXcds) * per + b / kXcds : b;
}

}  // namespace mimo
