// embed_tile.h -- the matrix-core tile shared by the patch-embedding GEMMs
// (patch_embed.hip over materialised rows, pixel_embed.hip straight from the
// source pixels): a 256 x 256 output tile per 4-wave workgroup, each wave a
// 128 x 128 quarter as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16, K staged
// through LDS 64 at a time in 128-byte rows whose 16-byte chunks are
// XOR-swizzled, and the fp32 accumulators written back through LDS with
// 16-byte non-temporal stores (bias added on the way out).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_util.h"

namespace mimo {
namespace embed {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kEmbedThreads = 256;
constexpr int kWaveM = 128, kWaveN = 128;       // one wave's quarter of the tile
constexpr int kBlocksM = kWaveM / 32, kBlocksN = kWaveN / 32;
constexpr int kGroups = kBM / 8 / (kEmbedThreads / 64);  // 1 KB LDS groups per wave per operand

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void *lds_void_ptr;
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Swizzle key of LDS row r: the same logical chunk of rows r .. r + 7 lands
// in 8 distinct 16-byte positions, and that of rows r .. r + 15 in 16
// distinct (row parity, position) pairs, so a 16-byte read by 8 or by 16
// lanes of consecutive rows touches every bank at most once.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
// LDS offset (in bf16) of logical 16-byte chunk v of row r.
__device__ __forceinline__ int lds_at(int r, int v) { return r * kBK + ((v ^ swz(r)) << 3); }

// s_waitcnt immediates (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8; a field at its maximum does not wait).
constexpr int kWaitAll = 0;                 // every counter at zero
constexpr int kWaitVmemButA = 0x0F78;       // vmcnt(8): one stage of A loads may stay in flight
constexpr int kWaitLdsVmemButA = 0x0078;    // lgkmcnt(0) and vmcnt(8)
constexpr int kWaitLdsVmem = 0x0070;        // lgkmcnt(0) and vmcnt(0)

// Output columns one lane writes per 16-byte store, and the lanes per
// staged row.
template <typename OutT>
struct EpilogueShape {
    static constexpr int kOutPerChunk = 16 / int(sizeof(OutT));  // 4 fp32 or 8 bf16
    static constexpr int kLanesPerRow = kWaveN / kOutPerChunk;   // 32 or 16
    static constexpr int kRowsPerPass = 64 / kLanesPerRow;       // 2 or 4
};

// The bias of the output columns this lane stores (the same for every row
// it stores), or zeros.
template <typename OutT>
__device__ __forceinline__ void load_lane_bias(const float *bias, int col0, int lane,
                                               f32x4 (&bv)[EpilogueShape<OutT>::kOutPerChunk / 4]) {
    constexpr int kOut = EpilogueShape<OutT>::kOutPerChunk;
    const int chunk = lane % EpilogueShape<OutT>::kLanesPerRow;
#pragma unroll
    for (int k = 0; k < kOut / 4; ++k)
        bv[k] = bias ? *reinterpret_cast<const f32x4 *>(bias + col0 + chunk * kOut + 4 * k) : f32x4{};
}

// One 16-byte store of converted outputs.
__device__ __forceinline__ u32x4 pack_out(const f32x4 (&v)[1], float *) {
    return __builtin_bit_cast(u32x4, v[0]);
}
__device__ __forceinline__ u32x4 pack_out(const f32x4 (&v)[2], uint16_t *) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    const bf16x8 h = {__bf16(v[0].x), __bf16(v[0].y), __bf16(v[0].z), __bf16(v[0].w),
                      __bf16(v[1].x), __bf16(v[1].y), __bf16(v[1].z), __bf16(v[1].w)};  // nearest even
    return __builtin_bit_cast(u32x4, h);
}

// A wave's 128 x 128 block to memory.  Per 32-row block row, the fp32
// accumulators are staged in the wave's 16 KB LDS region (rows of 512
// bytes, 16-byte chunks XOR-swizzled by the row so that the 32 rows a
// staging store covers fall in distinct chunks); then each lane reads whole
// row segments back, adds the bias of its columns (bv), converts and
// writes 16 bytes, non-temporal.  With W as the MFMA's first operand, value
// q of block (i, j) is row (lane % 32) of A block i and column 8 * (q / 4) +
// 4 * (lane / 32) + q % 4 of W block j.
template <typename OutT>
__device__ __forceinline__ void write_block(const f32x16 (&acc)[kBlocksM][kBlocksN], uint8_t *region,
                                            const f32x4 (&bv)[EpilogueShape<OutT>::kOutPerChunk / 4],
                                            OutT *out, int64_t row0, int col0, int64_t n_rows, int embed_dim,
                                            int lane) {
    typedef EpilogueShape<OutT> S;
    constexpr int kRowBytes = kWaveN * 4;  // fp32 staging
    constexpr int kChunks = kRowBytes / 16;
    static_assert(32 * kRowBytes == 16384, "a wave stages 16 KB");
    const bool full = row0 + kWaveM <= n_rows;
    const int chunk = lane % S::kLanesPerRow;
#pragma unroll
    for (int i = 0; i < kBlocksM; ++i) {
        const int r = lane & 31;
#pragma unroll
        for (int j = 0; j < kBlocksN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c = j * 8 + 2 * g + (lane >> 5);  // 16-byte chunk of 4 columns
                const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                 acc[i][j][4 * g + 3]};
                *reinterpret_cast<f32x4 *>(region + r * kRowBytes + ((c ^ r) % kChunks) * 16) = v;
            }
#pragma unroll
        for (int p = 0; p < 32 / S::kRowsPerPass; ++p) {
            const int rr = p * S::kRowsPerPass + lane / S::kLanesPerRow;
            f32x4 v[S::kOutPerChunk / 4];
#pragma unroll
            for (int k = 0; k < S::kOutPerChunk / 4; ++k) {
                const int c = chunk * (S::kOutPerChunk / 4) + k;
                v[k] = *reinterpret_cast<const f32x4 *>(region + rr * kRowBytes + ((c ^ rr) % kChunks) * 16) + bv[k];
            }
            const int64_t row = row0 + i * 32 + rr;
            if (full || row < n_rows)
                __builtin_nontemporal_store(pack_out(v, static_cast<OutT *>(nullptr)),
                                            reinterpret_cast<u32x4 *>(out + row * embed_dim + col0 +
                                                                      chunk * S::kOutPerChunk));
        }
    }
}

}  // namespace embed
}  // namespace mimo
