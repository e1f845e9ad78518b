// patch_embed.hip -- the patch embedding that consumes the pixel path's rows,
// as a bf16 matrix-core GEMM for AMD Instinct MI355X (gfx950, CDNA4).
//
// What is computed (NeMo Automodel "mimo_v2_flash.vision",
// MiMoVisionPatchEmbed): a Conv3d whose kernel and stride are both
// (T, P, P) = (2, 16, 16) over rows that are exactly one kernel window each,
// i.e. out[r][e] = bias[e] + sum_k rows[r][k] * W[e][k] with the weight
// [E][3][2][16][16] flattened in the rows' (c, tt, py, px) order.
//
// Folded form.  A still image's two temporal slots hold the same values, so
// sum_tt W[e][c][tt][p] * x[c][tt][p] = (W[e][c][0][p] + W[e][c][1][p]) *
// x[c][0][p]: with W' = bf16(W0 + W1) the GEMM runs over K = 768 (the tt = 0
// half of each channel) instead of 1536, half the matrix-core work, exact up
// to that one bf16 rounding of W'.
//
// Kernel.  C = A * W^T with both operands K-contiguous (bf16), fp32
// accumulation on v_mfma_f32_32x32x16_bf16.  A workgroup (4 wave64s) owns a
// 128 x 128 tile of C; each wave a 64 x 64 quarter as 2 x 2 MFMA blocks.  K
// advances 64 at a time through double-buffered LDS (rows padded by 16 bytes
// against bank conflicts): while the waves multiply one stage, the next
// stage's global loads are in flight in registers.  Tiles are ordered N
// fastest and assigned to XCDs in contiguous runs, so one XCD's L2 serves an
// A tile to all of its N tiles, and W (<= 4 MB) stays L2-resident.
#include <hip/hip_runtime.h>

#include <cstring>
#include <string>

#include "device_util.h"
#include "internal.h"
#include "runtime.h"

namespace mimo {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kEmbedThreads = 256;
constexpr int kPitch = kBK + 8;     // LDS row pitch in bf16 (144 bytes)
constexpr int kFoldSeg = 256;       // contiguous K run of one channel in the folded form
constexpr int kFoldStride = 512;    // its stride in the row (the tt = 1 plane is skipped)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct EmbedArgs {
    const uint16_t *rows;  // bf16 [n_rows][1536]
    const uint16_t *w;     // bf16 [E][K]
    const float *bias;     // [E] or null
    void *out;             // OutT [n_rows][E]
    int64_t n_rows;
    int32_t embed_dim;     // E, a multiple of 128
    int32_t k;             // 1536, or 768 folded
    int32_t folded;
    int32_t n_tiles;       // E / 128
};

// Row column of reduction index k0 (a multiple of kBK): the folded form
// reads channel c's tt = 0 plane, K run kFoldSeg, stride kFoldStride.
__device__ __forceinline__ int a_column(int k0, bool folded) {
    return folded ? (k0 / kFoldSeg) * kFoldStride + k0 % kFoldSeg : k0;
}

__device__ __forceinline__ void store_out(float *p, float v) { *p = v; }
__device__ __forceinline__ void store_out(uint16_t *p, float v) {
    *reinterpret_cast<__bf16 *>(p) = __bf16(v);  // round to nearest even
}

template <typename OutT>
__global__ __launch_bounds__(kEmbedThreads) void patch_embed_kernel(EmbedArgs a) {
    __shared__ uint16_t sa[2][kBM * kPitch];
    __shared__ uint16_t sb[2][kBN * kPitch];
    const int64_t tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    const int64_t mt = tile / a.n_tiles;
    const int nt = int(tile - mt * a.n_tiles);
    const int64_t m0 = mt * kBM;
    const int n0 = nt * kBN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // the wave's 64 x 64 quarter
    const bool folded = a.folded != 0;

    // Global -> register loads of one stage: 128 rows x 64 k of A and of W,
    // 16 bytes per load, 4 + 4 per thread.  Rows past n_rows load zeros.
    u32x4 ra[4], rb[4];
    auto load_stage = [&](int k0) {
        const int acol = a_column(k0, folded);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + i * kEmbedThreads;
            const int r = idx >> 3, v = idx & 7;
            const int64_t row = m0 + r;
            if (row < a.n_rows)
                ra[i] = *reinterpret_cast<const u32x4 *>(a.rows + row * kRowLen + acol + v * 8);
            else
                ra[i] = u32x4{0, 0, 0, 0};
            rb[i] = *reinterpret_cast<const u32x4 *>(a.w + int64_t(n0 + r) * a.k + k0 + v * 8);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + i * kEmbedThreads;
            const int r = idx >> 3, v = idx & 7;
            *reinterpret_cast<u32x4 *>(&sa[buf][r * kPitch + v * 8]) = ra[i];
            *reinterpret_cast<u32x4 *>(&sb[buf][r * kPitch + v * 8]) = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

    const int stages = a.k / kBK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    // MFMA operand rows of this lane: A block i covers C rows wm*64 + i*32 +
    // (lane % 32); B block j covers C columns wn*64 + j*32 + (lane % 32); the
    // lane supplies k = 8 * (lane / 32) .. + 7 of each 16-wide k step.
    const int frag_k = 8 * (lane >> 5);
    for (int s = 0; s < stages; ++s) {
        const int buf = s & 1;
        if (s + 1 < stages) load_stage((s + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < kBK; ks += 16) {
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ar = wm * 64 + i * 32 + (lane & 31);
                fa[i] = *reinterpret_cast<const bf16x8 *>(&sa[buf][ar * kPitch + ks + frag_k]);
                const int br = wn * 64 + i * 32 + (lane & 31);
                fb[i] = *reinterpret_cast<const bf16x8 *>(&sb[buf][br * kPitch + ks + frag_k]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (s + 1 < stages) store_stage(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: value q of block (i, j) is C row 8 * (q / 4) + 4 * (lane / 32)
    // + q % 4 of the block, column lane % 32.
    OutT *out = static_cast<OutT *>(a.out);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 64 + j * 32 + (lane & 31);
        const float b = a.bias ? a.bias[col] : 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                if (row < a.n_rows) store_out(out + row * a.embed_dim + col, acc[i][j][q] + b);
            }
    }
}

// W'[e][c][p] = bf16(W[e][c][0][p] + W[e][c][1][p]): the two bf16 values
// are added in float32 and the sum rounded to nearest even once.
__global__ __launch_bounds__(256) void fold_weights_kernel(const uint16_t *w, uint16_t *wf,
                                                           int64_t total) {
    const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t e = i / (3 * kFoldSeg);
    const int64_t rem = i - e * (3 * kFoldSeg);
    const int64_t c = rem / kFoldSeg, p = rem - c * kFoldSeg;
    const int64_t src = e * kRowLen + c * kFoldStride + p;
    const float w0 = float(*reinterpret_cast<const __bf16 *>(w + src));
    const float w1 = float(*reinterpret_cast<const __bf16 *>(w + src + kFoldSeg));
    *reinterpret_cast<__bf16 *>(wf + i) = __bf16(w0 + w1);
}

}  // namespace
}  // namespace mimo

using namespace mimo;

extern "C" {

int mimo_fold_patch_weights(int32_t embed_dim, const void *w, void *w_folded, void *stream) {
    clear_error();
    if (embed_dim < 1 || !w || !w_folded || w == w_folded || !check_ptr_align(w, 16) ||
        !check_ptr_align(w_folded, 16))
        return set_error(MIMO_E_INVALID, "fold_patch_weights: bad embed_dim or pointers");
    const int64_t total = int64_t(embed_dim) * (kRowLen / 2);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid{unsigned((total + 255) / 256), 1, 1}, block{256, 1, 1};
    const hipError_t e = timed_launch(s, [&] {
        hipLaunchKernelGGL(fold_weights_kernel, grid, block, 0, s,
                           static_cast<const uint16_t *>(w), static_cast<uint16_t *>(w_folded), total);
    });
    if (e != hipSuccess) return hip_error(e, "fold_patch_weights: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

int mimo_patch_embed(int64_t n_rows, const void *rows, int32_t embed_dim, const void *w,
                     int32_t folded, const float *bias, int32_t out_dtype, void *out,
                     void *stream) {
    clear_error();
    if (n_rows < 0 || embed_dim < kBN || embed_dim % kBN || embed_dim > 65536)
        return set_error(MIMO_E_INVALID, "patch_embed: embed_dim must be a multiple of 128 in [128, 65536]");
    if (folded != 0 && folded != 1)
        return set_error(MIMO_E_INVALID, "patch_embed: folded must be 0 or 1");
    if (out_dtype != MIMO_F32 && out_dtype != MIMO_BF16)
        return set_error(MIMO_E_INVALID, "patch_embed: out_dtype must be MIMO_F32 or MIMO_BF16");
    if (n_rows == 0) return MIMO_OK;
    if (!rows || !w || !out || !check_ptr_align(rows, 16) || !check_ptr_align(w, 16) ||
        !check_ptr_align(out, 16) || (bias && !check_ptr_align(bias, 4)))
        return set_error(MIMO_E_INVALID, "patch_embed: null or misaligned pointer (rows, w, out: 16 bytes)");
    const int64_t m_tiles = (n_rows + kBM - 1) / kBM;
    const int32_t n_tiles = embed_dim / kBN;
    if (m_tiles * n_tiles > 0x7FFFFFFFll)
        return set_error(MIMO_E_TOO_LARGE, "patch_embed: more than 2^31 - 1 tiles");
    EmbedArgs a;
    a.rows = static_cast<const uint16_t *>(rows);
    a.w = static_cast<const uint16_t *>(w);
    a.bias = bias;
    a.out = out;
    a.n_rows = n_rows;
    a.embed_dim = embed_dim;
    a.k = folded ? kRowLen / 2 : kRowLen;
    a.folded = folded;
    a.n_tiles = n_tiles;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid{unsigned(m_tiles * n_tiles), 1, 1}, block{unsigned(kEmbedThreads), 1, 1};
    const hipError_t e = timed_launch(s, [&] {
        if (out_dtype == MIMO_F32)
            hipLaunchKernelGGL(patch_embed_kernel<float>, grid, block, 0, s, a);
        else
            hipLaunchKernelGGL(patch_embed_kernel<uint16_t>, grid, block, 0, s, a);
    });
    if (e != hipSuccess) return hip_error(e, "patch_embed: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

}  // extern "C"
