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
// accumulation on v_mfma_f32_32x32x16_bf16.  A workgroup (4 wave64s, one
// per SIMD) owns a 256 x 256 tile of C; each wave a 128 x 128 quarter as
// 4 x 4 MFMA blocks (256 accumulators per lane), which keeps the LDS bytes
// per matrix-core flop at (128 + 128) / (128 * 128) of a 16-wide k step.  K
// advances 64 at a time; rows are 128 bytes and their eight 16-byte chunks
// are XOR-swizzled by the row index, so the fragment reads of 16
// consecutive rows hit distinct banks.  Operand tiles go from global memory
// straight into LDS (buffer_load_dwordx4 ... lds, no register staging), A two
// stages ahead of the MFMAs (three LDS buffers) and W one (two buffers):
// the kernel is bound by how fast a CU takes its tiles from L2, so the
// loads go out early, in the first half of each stage and spread between
// the MFMAs.  The tile is written back through LDS so that every store
// covers whole row segments (non-temporal, 16 bytes per lane): the fp32
// accumulators are staged, and each lane adds the bias of its own output
// columns (the same for every row it stores, loaded once) on the way out.
// W is the MFMA's first operand, which gives each lane four consecutive
// output columns to stage.  Tiles are ordered N fastest and assigned to
// XCDs in contiguous runs, so one XCD's L2 serves an A tile to all of its N
// tiles.
#include <hip/hip_runtime.h>

#include <cstring>
#include <string>

#include "device_util.h"
#include "embed_tile.h"
#include "internal.h"
#include "runtime.h"

namespace mimo {
namespace {

using namespace embed;

constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource word 3 (gfx9 family)
constexpr int kFoldSeg = 256;       // contiguous K run of one channel in the folded form
constexpr int kFoldStride = 512;    // its stride in the row (the tt = 1 plane is skipped)

struct EmbedArgs {
    const uint16_t *rows;  // bf16 [n_rows][1536]
    const uint16_t *w;     // bf16 [E][K]
    const float *bias;     // [E] or null
    void *out;             // OutT [n_rows][E]
    int64_t n_rows;
    int32_t embed_dim;     // E, a multiple of 256
    int32_t k;             // 1536, or 768 folded
    int32_t folded;
    int32_t n_tiles;       // E / 256
};

// Row column of reduction index k0 (a multiple of kBK): the folded form
// reads channel c's tt = 0 plane, K run kFoldSeg, stride kFoldStride.
__device__ __forceinline__ int a_column(int k0, bool folded) {
    return folded ? (k0 / kFoldSeg) * kFoldStride + k0 % kFoldSeg : k0;
}

// kFolded: K = 768 over the tt = 0 half of each row, else K = 1536.  K is
// a compile-time constant so that the stage loop unrolls fully: every
// buffer choice and every tail condition is then a constant, and the
// compiler can track each direct load exactly (a loop back edge makes it
// wait for all loads in flight before reading LDS).
template <typename OutT, bool kFolded>
__global__ __launch_bounds__(kEmbedThreads) void patch_embed_kernel(EmbedArgs a) {
    // Three A stages and two W stages (160 KB, all of the CU's LDS) as five
    // distinct arrays: the compiler then sees that the loads filling one
    // stage never alias the reads of another, and does not make those reads
    // wait for the loads in flight.
    __shared__ uint16_t sa0[kBM * kBK], sa1[kBM * kBK], sa2[kBM * kBK];
    __shared__ uint16_t sb0[kBN * kBK], sb1[kBN * kBK];
    const int64_t tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    const int64_t mt = tile / a.n_tiles;
    const int nt = int(tile - mt * a.n_tiles);
    const int64_t m0 = mt * kBM;
    const int n0 = nt * kBN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;  // the wave's quarter
    constexpr bool folded = kFolded;
    constexpr int stages = (kFolded ? kRowLen / 2 : kRowLen) / kBK;  // 12 or 24

    // Global -> LDS loads of one stage: 256 rows x 64 k of A and of W.  Wave
    // w fills LDS row groups [8 kGroups w, 8 kGroups (w + 1)); within a 1 KB
    // group lane l lands at row l / 8, physical chunk l % 8, so it fetches
    // the logical chunk (l % 8) ^ swz(row) of its row.  Rows past n_rows
    // read the last row instead; their results are never stored.  The loads
    // are buffer loads: one resource over the tile's A rows and one over its
    // W rows, a 32-bit byte offset per lane (< 768 KB) and the stage's K
    // offset as the uniform scalar offset.
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.rows + m0 * kRowLen), 0, 0x7FFFFFF0, kBufferWord3);
    const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.w + int64_t(n0) * a.k), 0, 0x7FFFFFF0, kBufferWord3);
    uint32_t a_off[kGroups], w_off[kGroups];
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
        const int r = (wave * kGroups + i) * 8 + (lane >> 3);
        const int v = (lane & 7) ^ swz(r);
        const int64_t row = m0 + r < a.n_rows ? m0 + r : a.n_rows - 1;
        a_off[i] = uint32_t((row - m0) * kRowLen * 2 + v * 16);
        w_off[i] = uint32_t(r * a.k * 2 + v * 16);
    }
    // One group (8 rows x 64 k) of a stage's A or W tile into LDS.
    auto load_a = [&](int grp, int k0, uint16_t *da) {
        const int g = wave * kGroups + grp;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void_ptr)(da + g * 8 * kBK), 16, a_off[grp],
                                                 a_column(k0, folded) * 2, 0, 0);
    };
    auto load_w = [&](int grp, int k0, uint16_t *db) {
        const int g = wave * kGroups + grp;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_void_ptr)(db + g * 8 * kBK), 16, w_off[grp],
                                                 k0 * 2, 0, 0);
    };
    // The barrier between stages.  __syncthreads would add a fence that
    // waits for every load in flight, the A loads two stages ahead included;
    // each thread has already waited for the loads of the next stage
    // (kWaitVmemButA: the A loads of the stage after it are its newest 8
    // vector memory operations), and LDS-DMA data counts as written once
    // vmcnt has passed it.
    auto barrier = [] {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    f32x16 acc[kBlocksM][kBlocksN];
#pragma unroll
    for (int i = 0; i < kBlocksM; ++i)
#pragma unroll
        for (int j = 0; j < kBlocksN; ++j) acc[i][j] = f32x16{};

    // A runs two stages ahead of the MFMAs, W one: stage s reads A buffer
    // s % 3 and W buffer s % 2.
#pragma unroll
    for (int grp = 0; grp < kGroups; ++grp) load_a(grp, 0, sa0);
#pragma unroll
    for (int grp = 0; grp < kGroups; ++grp) load_w(grp, 0, sb0);
#pragma unroll
    for (int grp = 0; grp < kGroups; ++grp) load_a(grp, kBK, sa1);
    __builtin_amdgcn_s_waitcnt(kWaitVmemButA);
    barrier();
    // MFMA operand rows of this lane: A block i covers C rows wm*128 + i*32 +
    // (lane % 32); B block j covers C columns wn*128 + j*32 + (lane % 32);
    // the lane supplies k = 8 * (lane / 32) .. + 7 of each 16-wide k step.
    const int frag_chunk = lane >> 5;
    const int frag_row = lane & 31;
    // Fragments of k step ks from one LDS stage.
    auto read_frags = [&](const uint16_t *ta, const uint16_t *tb, int ks, bf16x8 (&fa)[kBlocksM],
                          bf16x8 (&fb)[kBlocksN]) {
#pragma unroll
        for (int i = 0; i < kBlocksM; ++i)
            fa[i] = *reinterpret_cast<const bf16x8 *>(
                &ta[lds_at(wm * kWaveM + i * 32 + frag_row, 2 * ks + frag_chunk)]);
#pragma unroll
        for (int j = 0; j < kBlocksN; ++j)
            fb[j] = *reinterpret_cast<const bf16x8 *>(
                &tb[lds_at(wn * kWaveN + j * 32 + frag_row, 2 * ks + frag_chunk)]);
    };
    constexpr int kSteps = kBK / 16;
    static_assert(kGroups == 8 && kSteps * kBlocksM == 16, "two loads after each of the first 8 MFMA rows");
    // One stage: multiply this LDS stage (the next k step's fragments are
    // read while this step's MFMAs run).  During the first two k steps, two
    // loads go out after each row of four MFMAs (issued in a burst they would
    // hold the wave at issue): W for stage s + 1, then A for stage s + 2, so
    // the later half of the stage covers their latency.  Before the last k
    // step's MFMAs, whose fragments are already in registers, the wave waits
    // for its own LDS reads and for all but the A loads, meets the others,
    // and reads the next stage's first fragments: the stage change then costs
    // no MFMA idle time.  The loads issued after that barrier overwrite this
    // stage's buffers, which no wave reads any more.  The fragments are
    // double-buffered across stages.
    bf16x8 fa[2][kBlocksM], fb[2][kBlocksN];
    read_frags(sa0, sb0, 0, fa[0], fb[0]);
    auto stage = [&](int s, const uint16_t *ta, const uint16_t *tb, uint16_t *nb, uint16_t *na2,
                     const uint16_t *ta_next, const uint16_t *tb_next) {
        const bool more_w = s + 1 < stages, more_a = s + 2 < stages;
        const int kw = (s + 1) * kBK, ka = (s + 2) * kBK;
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
            if (ks + 1 < kSteps) {
                read_frags(ta, tb, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
            } else if (more_w) {
                // every read of this stage is issued: wait for them and for the
                // next stage's data, meet, and read the next stage's first
                // fragments while this last k step's MFMAs run
                if (more_a)
                    __builtin_amdgcn_s_waitcnt(kWaitLdsVmemButA);
                else
                    __builtin_amdgcn_s_waitcnt(kWaitLdsVmem);
                barrier();
                read_frags(ta_next, tb_next, 0, fa[0], fb[0]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kBlocksM; ++i) {
#pragma unroll
                for (int j = 0; j < kBlocksN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][j], fa[ks & 1][i],
                                                                        acc[i][j], 0, 0, 0);
                const int slot = ks * kBlocksM + i;
                if (slot < 4 && more_w) {
                    load_w(2 * slot, kw, nb);
                    load_w(2 * slot + 1, kw, nb);
                } else if (slot >= 4 && slot < 8 && more_a) {
                    load_a(2 * slot - 8, ka, na2);
                    load_a(2 * slot - 7, ka, na2);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
#pragma unroll
    for (int s = 0; s < stages; ++s) {
        uint16_t *const abuf[3] = {sa0, sa1, sa2};
        uint16_t *const wbuf[2] = {sb0, sb1};
        stage(s, abuf[s % 3], wbuf[s % 2], wbuf[(s + 1) % 2], abuf[(s + 2) % 3], abuf[(s + 1) % 3],
              wbuf[(s + 1) % 2]);
    }
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    barrier();

    // Epilogue through LDS, free now that every wave has passed the last
    // stage's barrier: each wave stages its block in half of one stage array.
    uint8_t *region = reinterpret_cast<uint8_t *>(wave < 2 ? sa0 : sa1) + (wave & 1) * (kBM * kBK);
    const int col0 = n0 + wn * kWaveN;
    f32x4 bv[EpilogueShape<OutT>::kOutPerChunk / 4];
    load_lane_bias<OutT>(a.bias, col0, lane, bv);
    // waited for here, once, so that no store of the epilogue waits on memory
#pragma unroll
    for (int k = 0; k < EpilogueShape<OutT>::kOutPerChunk / 4; ++k) asm volatile("" : "+v"(bv[k]));
    write_block<OutT>(acc, region, bv, static_cast<OutT *>(a.out), m0 + wm * kWaveM, col0, a.n_rows, a.embed_dim,
                      lane);
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
        return set_error(MIMO_E_INVALID, "patch_embed: embed_dim must be a multiple of 256 in [256, 65536]");
    if (folded != 0 && folded != 1)
        return set_error(MIMO_E_INVALID, "patch_embed: folded must be 0 or 1");
    if (out_dtype != MIMO_F32 && out_dtype != MIMO_BF16)
        return set_error(MIMO_E_INVALID, "patch_embed: out_dtype must be MIMO_F32 or MIMO_BF16");
    if (n_rows == 0) return MIMO_OK;
    if (!rows || !w || !out || !check_ptr_align(rows, 16) || !check_ptr_align(w, 16) ||
        !check_ptr_align(out, 16) || (bias && !check_ptr_align(bias, 16)))
        return set_error(MIMO_E_INVALID, "patch_embed: null or misaligned pointer (rows, w, out, bias: 16 bytes)");
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
        if (out_dtype == MIMO_F32) {
            if (folded)
                hipLaunchKernelGGL((patch_embed_kernel<float, true>), grid, block, 0, s, a);
            else
                hipLaunchKernelGGL((patch_embed_kernel<float, false>), grid, block, 0, s, a);
        } else {
            if (folded)
                hipLaunchKernelGGL((patch_embed_kernel<uint16_t, true>), grid, block, 0, s, a);
            else
                hipLaunchKernelGGL((patch_embed_kernel<uint16_t, false>), grid, block, 0, s, a);
        }
    });
    if (e != hipSuccess) return hip_error(e, "patch_embed: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

}  // extern "C"
