// pixel_embed.hip -- the pixel path and its patch embedding in one
// matrix-core kernel for AMD Instinct MI355X (gfx950, CDNA4): still images
// in, embeddings out, with no patch row ever written to memory.
//
// What is computed.  NeMo Automodel "mimo_v2_flash.vision",
// MiMoVisionPatchEmbed: a Conv3d with kernel = stride = (2, 16, 16), i.e.
// out[r][e] = bias[e] + sum_k row_r[k] * W[e][k] over the 1536 values of
// patch row r in (c, tt, py, px) order; the rows are the pixel path of
// NeMo Automodel "mimo_v2_flash.processing" (MimoV2ImageProcessor, class
// docstring): RGBA flattened onto white, the bilinear resize to the
// smart_resize target on 0-255 floats, a = (x - mean255[c]) / std255[c],
// two identical frames.
//
// Algebra used (exact in real numbers).  For a still image the two frames
// are equal, so the weight's two temporal halves can be summed (K = 768,
// W' = W0 + W1).  The standardisation is affine:
//     sum_k a_k W'_k = sum_k x_k (s_c W'_k) - sum_k m_c (s_c W'_k)
// with s_c = 1 / std255[c], m_c = mean255[c].  So with the prepared weight
// Wt = bf16(s_c * W') and bias' = bias - sum_k m_c * Wt_k (both made once by
// mimo_prepare_pixel_embed), the embedding is sum_k x_k Wt_k + bias' on the
// resized 0-255 values x themselves.  For an image whose smart_resize target
// is its own size, x is the source byte, which bf16 holds exactly; for a
// resized image x is the bilinear value in float32 (the pixel path's
// arithmetic) rounded once to bf16.  K runs over the patch's values in the
// source's own (py, px, c) byte order, so that 8 consecutive k are 8
// consecutive source bytes of one pixel row.
//
// Kernel.  The 256 x 256 output tile of embed_tile.h, K in 12 stages of 64.
// The prepared weight goes from global memory straight into LDS
// (buffer_load ... lds), one stage ahead of the matrix cores, as in the
// GEMM over materialised rows.  The pixel operand is produced by the
// workgroup itself: for an image without resample, each thread owns one
// 16-byte chunk position of 8 tile rows; it loads the 8 source bytes of each
// two stages ahead (into registers), converts them to bf16 and writes them
// into the swizzled LDS tile one stage ahead, all between the matrix-core
// instructions of the current stage.  A batch with a resized or RGBA image
// launches a second instance whose producer computes every value with the
// pixel kernel's bilinear arithmetic from global memory: correct for any
// still, but bound by those loads.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>

#include "device_util.h"
#include "embed_tile.h"
#include "internal.h"
#include "runtime.h"
#include "tables.h"

namespace mimo {
namespace {

using namespace embed;

constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource word 3 (gfx9 family)
constexpr int kK = kRowLen / 2;           // 768 values of a still patch: (py, px, c)
constexpr int kStages = kK / kBK;         // 12
constexpr int kRowsPerThread = kBM * (kBK / 8) / kEmbedThreads;  // 8 tile rows per producer thread
// A tile's source bytes are addressed with 32-bit offsets from the first
// image it touches (the host checks every tile against this).
constexpr int64_t kTileSpanLimit = 0x7FFFFFF0ll - 64;

struct PixelEmbedArgs {
    const uint8_t *src;
    int64_t src_end;            // bytes readable from src
    const DevImage *images;
    const int64_t *row_begin;   // [n + 1], rows in merge-block order
    const uint16_t *w;          // bf16 [E][768] in (py, px, c) order
    const float *bias;          // [E]
    void *out;                  // OutT [n_rows][E]
    int64_t n_rows;
    int32_t n;
    int32_t embed_dim;
    int32_t n_tiles;            // E / 256
};

// Largest i in [0, n) with begin[i] <= r (per lane): the image that holds
// row r (images without rows repeat the next one's begin and are skipped).
__device__ __forceinline__ int row_image(const int64_t *begin, int n, int64_t r) {
    int lo = 0, hi = n;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (begin[mid] <= r) lo = mid; else hi = mid;
    }
    return lo;
}

// Where one tile row's patch sits: its image, the patch's first output
// pixel (oy0, ox0).
struct RowPatch {
    int img, oy0, ox0;
};

__device__ __forceinline__ RowPatch row_patch(const PixelEmbedArgs &a, int64_t r, const DevImage &d, int img) {
    const int q = int(r - d.row_offset);  // row within the image (merge-block order)
    const int u = q >> 2;                 // merge unit
    const int br = div_small(u, d.blocks_w, 1.0f / float(d.blocks_w));
    const int bc = u - br * d.blocks_w;
    RowPatch p;
    p.img = img;
    p.oy0 = (br * kMerge + ((q >> 1) & 1)) * kPatch;
    p.ox0 = (bc * kMerge + (q & 1)) * kPatch;
    return p;
}

// bf16 bits of four bytes of u (integers 0..255 are exact in bf16: the
// float's low 16 bits are zero), packed two per dword.
__device__ __forceinline__ void bytes_to_bf16(uint32_t u, uint32_t &lo, uint32_t &hi) {
    const uint32_t f0 = __builtin_bit_cast(uint32_t, float(u & 255u));
    const uint32_t f1 = __builtin_bit_cast(uint32_t, float((u >> 8) & 255u));
    const uint32_t f2 = __builtin_bit_cast(uint32_t, float((u >> 16) & 255u));
    const uint32_t f3 = __builtin_bit_cast(uint32_t, float(u >> 24));
    lo = __builtin_amdgcn_perm(f1, f0, 0x07060302u);
    hi = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
}

// Chunk j (0..95) of a patch: values 8j .. 8j + 7 of its (py, px, c)
// sequence, i.e. patch row py = j / 6, bytes 8 (j % 6) .. + 7 of that row.
__device__ __forceinline__ int chunk_row(int j) { return (j * 43) >> 8; }  // j / 6 for j < 96

// One channel value of the resized image at output pixel (oy, ox): the pixel
// kernel's float32 bilinear arithmetic, RGBA flattened onto white first.
__device__ __forceinline__ float resized_value(const uint8_t *img, const DevImage &d, int oy, int ox, int c) {
    float sy = __builtin_fmaf(d.scale_y, float(oy) + 0.5f, -0.5f);
    sy = sy < 0.0f ? 0.0f : sy;
    int y0 = int(sy);
    y0 = y0 < d.src_h - 1 ? y0 : d.src_h - 1;
    const float ly1 = sy - float(y0), ly0 = 1.0f - ly1;
    float sx = __builtin_fmaf(d.scale_x, float(ox) + 0.5f, -0.5f);
    sx = sx < 0.0f ? 0.0f : sx;
    int x0 = int(sx);
    x0 = x0 < d.src_w - 1 ? x0 : d.src_w - 1;
    const float lx1 = sx - float(x0), lx0 = 1.0f - lx1;
    const int y1 = min(y0 + 1, d.src_h - 1), x1 = min(x0 + 1, d.src_w - 1);
    const int C = d.channels;
    const int64_t rb = int64_t(d.src_w) * C;
    auto at = [&](int y, int x) {
        const uint8_t *p = img + int64_t(y) * rb + int64_t(x) * C;
        uint32_t v = p[c];
        if (C == 4) {
            const uint32_t al = p[3];
            v = 255u - al + (v * al + 127u) / 255u;  // onto white, rounded
        }
        return float(v);
    };
    const float top = __builtin_fmaf(lx0, at(y0, x0), lx1 * at(y0, x1));
    const float bot = __builtin_fmaf(lx0, at(y1, x0), lx1 * at(y1, x1));
    return __builtin_fmaf(ly0, top, ly1 * bot);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {__bf16(lo), __bf16(hi)};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

template <typename OutT, bool kGeneral>
__global__ __launch_bounds__(kEmbedThreads) void pixel_embed_kernel(PixelEmbedArgs a) {
    // Two pixel stages (written one stage ahead by the workgroup) and two
    // weight stages (loaded one stage ahead), each a distinct array.
    __shared__ uint16_t sa0[kBM * kBK], sa1[kBM * kBK];
    __shared__ uint16_t sb0[kBN * kBK], sb1[kBN * kBK];
    const int64_t tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    const int64_t mt = tile / a.n_tiles;
    const int nt = int(tile - mt * a.n_tiles);
    const int64_t m0 = mt * kBM;
    const int n0 = nt * kBN;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- the producer's rows: chunk position jj of tile rows (tid / 8) + 32 i
    const int jj = tid & 7;
    const int row_lo = tid >> 3;
    // the tile's source window starts at the first image it touches
    const int img_first = find_segment(a.row_begin, a.n, m0);
    const uint64_t win_base = reinterpret_cast<uint64_t>(a.src) + uint64_t(a.images[img_first].src_offset);
    const uint64_t win_end = reinterpret_cast<uint64_t>(a.src) + uint64_t(a.src_end);
    const uint64_t win_len = win_end - win_base;
    const __amdgpu_buffer_rsrc_t src_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>(win_base), 0, win_len > 0x7FFFFFF0ull ? 0x7FFFFFF0 : int(win_len), kBufferWord3);
    // per row: byte offset of the patch's first pixel in the window and the
    // image's row pitch (no-resample instance), or the patch (general one)
    uint32_t base[kRowsPerThread], pitch[kRowsPerThread];
    RowPatch patch[kRowsPerThread];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
        const int64_t r = min(m0 + row_lo + 32 * i, a.n_rows - 1);  // rows past the end: any valid row
        const int img = row_image(a.row_begin, a.n, r);
        const DevImage d = a.images[img];
        const RowPatch p = row_patch(a, r, d, img);
        if (kGeneral) {
            patch[i] = p;
        } else {
            pitch[i] = uint32_t(d.src_w) * 3u;
            base[i] = uint32_t(d.src_offset - a.images[img_first].src_offset +
                               (int64_t(p.oy0) * d.src_w + p.ox0) * 3);
        }
    }

    // Source bytes of stage s for the no-resample producer: chunk 8s + jj of
    // each row, 12 dword-aligned bytes that hold its 8.
    u32x3 raw[kRowsPerThread];
    // (pitch < 2^24: the host sends wider images to the general instance, so
    // the product runs on the 24-bit multiplier)
    auto chunk_offset = [&](int s, int i) {
        const int j = 8 * s + jj;
        const int py = chunk_row(j);
        return __umul24(uint32_t(py), pitch[i]) + base[i] + uint32_t(8 * (j - 6 * py));
    };
    auto load_raw = [&](int s, int i) {
        raw[i] = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(
                                                 src_rsrc, int(chunk_offset(s, i) & ~3u), 0, 0));
    };
    // Chunk 8s + jj of row i into the LDS pixel stage `da`, as bf16.
    auto write_chunk = [&](int s, int i, uint16_t *da) {
        const int rr = row_lo + 32 * i;
        u32x4 v;
        if (!kGeneral) {
            const uint32_t sh = chunk_offset(s, i) & 3u;
            const uint32_t u0 = __builtin_amdgcn_alignbyte(raw[i].y, raw[i].x, sh);
            const uint32_t u1 = __builtin_amdgcn_alignbyte(raw[i].z, raw[i].y, sh);
            uint32_t b0, b1, b2, b3;
            bytes_to_bf16(u0, b0, b1);
            bytes_to_bf16(u1, b2, b3);
            v = u32x4{b0, b1, b2, b3};
        } else {
            const DevImage d = a.images[patch[i].img];
            const uint8_t *img = a.src + d.src_offset;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = 8 * (8 * s + jj) + e;
                const int pix = (k * 43691) >> 17;  // k / 3 for k < 768
                const int c = k - 3 * pix;
                x[e] = resized_value(img, d, patch[i].oy0 + (pix >> 4), patch[i].ox0 + (pix & 15), c);
            }
            v = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                      pack_bf16x2(x[6], x[7])};
        }
        *reinterpret_cast<u32x4 *>(&da[lds_at(rr, jj)]) = v;
    };

    // ---- the weight operand: straight to LDS, as in the GEMM over rows
    const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(a.w + int64_t(n0) * kK), 0, 0x7FFFFFF0, kBufferWord3);
    uint32_t w_off[kGroups];
#pragma unroll
    for (int i = 0; i < kGroups; ++i) {
        const int r = (wave * kGroups + i) * 8 + (lane >> 3);
        const int v = (lane & 7) ^ swz(r);
        w_off[i] = uint32_t(r * kK * 2 + v * 16);
    }
    auto load_w = [&](int grp, int k0, uint16_t *db) {
        const int g = wave * kGroups + grp;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, (lds_void_ptr)(db + g * 8 * kBK), 16, w_off[grp],
                                                 k0 * 2, 0, 0);
    };
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

    // Prologue: stage 0's pixels into sa0 and weights into sb0; stage 1's
    // source bytes in flight.
    if (!kGeneral) {
#pragma unroll
        for (int i = 0; i < kRowsPerThread; ++i) load_raw(0, i);
    }
#pragma unroll
    for (int grp = 0; grp < kGroups; ++grp) load_w(grp, 0, sb0);
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) write_chunk(0, i, sa0);
    if (!kGeneral) {
#pragma unroll
        for (int i = 0; i < kRowsPerThread; ++i) load_raw(1, i);
        __builtin_amdgcn_s_waitcnt(kWaitLdsVmemButA);  // the weights; stage 1's bytes may stay in flight
    } else {
        __builtin_amdgcn_s_waitcnt(kWaitLdsVmem);
    }
    barrier();

    const int frag_chunk = lane >> 5;
    const int frag_row = lane & 31;
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
    static_assert(kGroups == 8 && kSteps * kBlocksM == 16 && kRowsPerThread == 8,
                  "two weight loads, pixel chunks and source loads after each of 12 MFMA rows");
    bf16x8 fa[2][kBlocksM], fb[2][kBlocksN];
    read_frags(sa0, sb0, 0, fa[0], fb[0]);
    // Stage s, between its 16 rows of four MFMAs: after rows 0-3 two weight
    // loads each (stage s + 1); within rows 4-11 one pixel chunk each,
    // written into the other pixel buffer (stage s + 1, from the bytes
    // loaded during stage s - 1) and interleaved with the row's MFMAs; in
    // rows 8-11 also two source loads each (stage s + 2).
    // Before the last k step's MFMAs the wave waits for its LDS traffic and
    // for the weights of stage s + 1, meets the others, and reads stage
    // s + 1's first fragments.
    auto stage = [&](int s, const uint16_t *ta, const uint16_t *tb, uint16_t *na, uint16_t *nb) {
        const bool more = s + 1 < kStages, more2 = s + 2 < kStages;
        const int kw = (s + 1) * kBK;
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
            if (ks + 1 < kSteps) {
                read_frags(ta, tb, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
            } else if (more) {
                if (more2 && !kGeneral)
                    __builtin_amdgcn_s_waitcnt(kWaitLdsVmemButA);
                else
                    __builtin_amdgcn_s_waitcnt(kWaitLdsVmem);
                barrier();
                read_frags(na, nb, 0, fa[0], fb[0]);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < kBlocksM; ++i) {
#pragma unroll
                for (int j = 0; j < kBlocksN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][j], fa[ks & 1][i],
                                                                        acc[i][j], 0, 0, 0);
                const int slot = ks * kBlocksM + i;
                if (more) {
                    if (slot < 4) {
                        load_w(2 * slot, kw, nb);
                        load_w(2 * slot + 1, kw, nb);
                    } else if (slot < 12) {
                        // one pixel chunk per row of MFMAs, its ALU work
                        // interleaved with them: a few VALU instructions
                        // after each MFMA, while the matrix core is busy
                        write_chunk(s + 1, slot - 4, na);
                        if (slot >= 8 && more2 && !kGeneral) {
                            // the source bytes of stage s + 2, for chunks
                            // already written this stage
                            load_raw(s + 2, 2 * slot - 16);
                            load_raw(s + 2, 2 * slot - 15);
                        }
                        if (!kGeneral) {
#pragma unroll
                            for (int m = 0; m < kBlocksN; ++m) {
                                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // up to 5 VALU
                            }
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // the no-resample instance runs its stages fully unrolled (every buffer
    // choice a constant, every load tracked exactly); the resampling one is
    // too large to unroll and loops
    constexpr int kStageUnroll = kGeneral ? 1 : kStages;
#pragma unroll kStageUnroll
    for (int s = 0; s < kStages; ++s) {
        const bool even = s % 2 == 0;
        stage(s, even ? sa0 : sa1, even ? sb0 : sb1, even ? sa1 : sa0, even ? sb1 : sb0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    barrier();

    uint8_t *region = reinterpret_cast<uint8_t *>(wave < 2 ? sa0 : sa1) + (wave & 1) * (kBM * kBK);
    const int col0 = n0 + wn * kWaveN;
    f32x4 bv[EpilogueShape<OutT>::kOutPerChunk / 4];
    load_lane_bias<OutT>(a.bias, col0, lane, bv);
#pragma unroll
    for (int k = 0; k < EpilogueShape<OutT>::kOutPerChunk / 4; ++k) asm volatile("" : "+v"(bv[k]));
    write_block<OutT>(acc, region, bv, static_cast<OutT *>(a.out), m0 + wm * kWaveM, col0, a.n_rows,
                      a.embed_dim, lane);
}

// Wt[e][(py*16 + px)*3 + c] = bf16(s_c * (W[e][c][0][py][px] + W[e][c][1][py][px]))
// (the sum and the product in float32, one rounding to bf16), and
// bias'[e] = bias[e] - sum_k m_c * Wt[e][k] (float64, rounded once).  One
// workgroup per output channel e; the float64 sum is reduced in a fixed
// order, so it is the same on every call.
__global__ __launch_bounds__(256) void prepare_pixel_embed_kernel(const uint16_t *w, const float *bias,
                                                                  float m0, float m1, float m2, float s0,
                                                                  float s1, float s2, uint16_t *wt,
                                                                  float *bias_out) {
    __shared__ double part[256];
    const int64_t e = blockIdx.x;
    const int t = threadIdx.x;
    const float mean[3] = {m0, m1, m2}, inv[3] = {s0, s1, s2};
    double acc = 0.0;
    for (int k = t; k < kK; k += 256) {
        const int pix = k / 3, c = k - 3 * pix;
        const int64_t src = e * kRowLen + c * (kTemporal * kPlane) + pix;
        const float w0 = float(*reinterpret_cast<const __bf16 *>(w + src));
        const float w1 = float(*reinterpret_cast<const __bf16 *>(w + src + kPlane));
        const __bf16 v = __bf16((w0 + w1) * inv[c]);
        *reinterpret_cast<__bf16 *>(wt + e * kK + k) = v;
        acc += double(mean[c]) * double(float(v));
    }
    part[t] = acc;
    __syncthreads();
    for (int step = 128; step > 0; step >>= 1) {
        if (t < step) part[t] += part[t + step];
        __syncthreads();
    }
    if (t == 0) bias_out[e] = float((bias ? double(bias[e]) : 0.0) - part[0]);
}

}  // namespace
}  // namespace mimo

using namespace mimo;

extern "C" {

int mimo_prepare_pixel_embed(int32_t embed_dim, const void *w, const float *bias, const float *mean255,
                             const float *std255, void *w_pixels, float *bias_pixels, void *stream) {
    clear_error();
    if (embed_dim < 1 || !w || !w_pixels || !bias_pixels || !mean255 || !std255 || w == w_pixels ||
        !check_ptr_align(w, 16) || !check_ptr_align(w_pixels, 16) || !check_ptr_align(bias_pixels, 4) ||
        (bias && !check_ptr_align(bias, 4)))
        return set_error(MIMO_E_INVALID, "prepare_pixel_embed: bad embed_dim or pointers");
    float inv[3];
    for (int c = 0; c < 3; ++c) {
        if (!(std255[c] > 0.0f) || !std::isfinite(std255[c]) || !std::isfinite(mean255[c]))
            return set_error(MIMO_E_INVALID, "prepare_pixel_embed: std255 must be > 0 and finite");
        inv[c] = float(1.0 / double(std255[c]));  // the pixel kernel's reciprocal
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = timed_launch(s, [&] {
        hipLaunchKernelGGL(prepare_pixel_embed_kernel, dim3(unsigned(embed_dim)), dim3(256), 0, s,
                           static_cast<const uint16_t *>(w), bias, mean255[0], mean255[1], mean255[2],
                           inv[0], inv[1], inv[2], static_cast<uint16_t *>(w_pixels), bias_pixels);
    });
    if (e != hipSuccess) return hip_error(e, "prepare_pixel_embed: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

int mimo_pixel_embed(int32_t n, const mimo_image_desc *desc, const uint8_t *src, int64_t src_capacity,
                     int32_t embed_dim, const void *w_pixels, const float *bias_pixels, int32_t out_dtype,
                     void *out, int64_t capacity_rows, void *workspace, size_t workspace_bytes,
                     void *stream) {
    clear_error();
    if (n < 0 || (n > 0 && !desc))
        return set_error(MIMO_E_INVALID, "pixel_embed: bad n or null pointer");
    if (embed_dim < kBN || embed_dim % kBN || embed_dim > 65536)
        return set_error(MIMO_E_INVALID, "pixel_embed: embed_dim must be a multiple of 256 in [256, 65536]");
    if (out_dtype != MIMO_F32 && out_dtype != MIMO_BF16)
        return set_error(MIMO_E_INVALID, "pixel_embed: out_dtype must be MIMO_F32 or MIMO_BF16");
    if (n == 0) return MIMO_OK;
    if (!src || !check_ptr_align(src, 4) || !w_pixels || !check_ptr_align(w_pixels, 16) || !bias_pixels ||
        !check_ptr_align(bias_pixels, 16) || !out || !check_ptr_align(out, 16))
        return set_error(MIMO_E_INVALID, "pixel_embed: null or misaligned pointer (src 4, w_pixels, "
                                         "bias_pixels and out 16 bytes)");
    if (!workspace || !check_ptr_align(workspace, 16))
        return set_error(MIMO_E_INVALID, "pixel_embed: workspace must be non-null and 16-byte aligned");
    if (workspace_bytes < ws_total_bytes(n))
        return set_error(MIMO_E_CAPACITY, "pixel_embed: workspace smaller than mimo_workspace_bytes(n)");
    bool general = false;
    int64_t src_needed = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mimo_image_desc &d = desc[i];
        if (d.status != MIMO_OK || d.rows == 0) continue;
        if (d.frames != 1)
            return set_error(MIMO_E_UNSUPPORTED, "pixel_embed: item " + std::to_string(i) +
                                                     " is a clip; the folded embedding needs still images");
        // the no-resample producer handles RGB images of row pitch < 2^24 bytes
        general = general || d.channels != 3 || d.src_h != d.dst_h || d.src_w != d.dst_w ||
                  int64_t(d.src_w) * 3 >= (int64_t(1) << 24);
        src_needed = std::max<int64_t>(src_needed, d.src_offset + int64_t(d.src_h) * d.src_w * d.channels);
    }
    if (src_capacity < ((src_needed + 15) & ~int64_t(15)))
        return set_error(MIMO_E_CAPACITY, "pixel_embed: src_capacity below the packed size rounded up to 16");
    BuiltTables t;
    int st = build_tables(n, desc, Tiling(), t);
    if (st != MIMO_OK) return st;
    if (t.total_rows > capacity_rows)
        return set_error(MIMO_E_CAPACITY, "pixel_embed: capacity_rows below the plan's total rows");
    if (t.total_rows == 0) return MIMO_OK;
    const int64_t m_tiles = (t.total_rows + kBM - 1) / kBM;
    const int32_t n_tiles = embed_dim / kBN;
    if (m_tiles * n_tiles > 0x7FFFFFFFll)
        return set_error(MIMO_E_TOO_LARGE, "pixel_embed: more than 2^31 - 1 tiles");
    // every tile's source bytes lie within 2^31 bytes of its first image's
    // (the kernel addresses them with 32-bit offsets from there)
    const int64_t *row_begin = reinterpret_cast<const int64_t *>(t.bytes.data() + ws_images_bytes(n) +
                                                                 ws_prefix_bytes(n));
    auto image_of_row = [&](int64_t r) {  // largest i < n with row_begin[i] <= r
        return int32_t(std::upper_bound(row_begin, row_begin + n, r) - row_begin) - 1;
    };
    for (int64_t m = 0; m < m_tiles; ++m) {
        const int32_t first = image_of_row(m * kBM);
        const int32_t last = image_of_row(std::min((m + 1) * kBM, t.total_rows) - 1);
        const int64_t span = desc[last].src_offset +
                             int64_t(desc[last].src_h) * desc[last].src_w * desc[last].channels -
                             desc[first].src_offset;
        if (span > kTileSpanLimit)
            return set_error(MIMO_E_TOO_LARGE, "pixel_embed: a tile's images span more than 2^31 source bytes");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = upload_table(t.bytes.data(), t.bytes.size(), workspace, s);
    if (e != hipSuccess) return hip_error(e, "pixel_embed: table upload");
    const uint8_t *ws = static_cast<const uint8_t *>(workspace);
    PixelEmbedArgs a;
    a.src = src;
    a.src_end = src_capacity;
    a.images = reinterpret_cast<const DevImage *>(ws);
    a.row_begin = reinterpret_cast<const int64_t *>(ws + ws_images_bytes(n) + ws_prefix_bytes(n));
    a.w = static_cast<const uint16_t *>(w_pixels);
    a.bias = bias_pixels;
    a.out = out;
    a.n_rows = t.total_rows;
    a.n = n;
    a.embed_dim = embed_dim;
    a.n_tiles = n_tiles;
    const dim3 grid{unsigned(m_tiles * n_tiles), 1, 1}, block{unsigned(kEmbedThreads), 1, 1};
    e = timed_launch(s, [&] {
        if (out_dtype == MIMO_F32) {
            if (general)
                hipLaunchKernelGGL((pixel_embed_kernel<float, true>), grid, block, 0, s, a);
            else
                hipLaunchKernelGGL((pixel_embed_kernel<float, false>), grid, block, 0, s, a);
        } else {
            if (general)
                hipLaunchKernelGGL((pixel_embed_kernel<uint16_t, true>), grid, block, 0, s, a);
            else
                hipLaunchKernelGGL((pixel_embed_kernel<uint16_t, false>), grid, block, 0, s, a);
        }
    });
    if (e != hipSuccess) return hip_error(e, "pixel_embed: kernel launch");
    g_dispatches.fetch_add(1);
    return MIMO_OK;
}

}  // extern "C"
