// hf_resize.hip -- the stock-HF contrast path for AMD Instinct MI355X
// (gfx950): the pixels the stock Qwen2-VL processor would give, so a caller
// can measure or reproduce the shift the MiMo path avoids.
//
// What is computed (NeMo Automodel "mimo_v2_flash.processing", module
// docstring, on the stock processor): alpha dropped (RGB bytes kept), a PIL
// antialiased bicubic resize that returns bytes, a 0-1 rescale and a
// float32 normalisation, then the same rows as the MiMo path (two identical
// frames, (c, tt, py, px), merge-block or column order).
//
// Resize arithmetic, as PIL's 8-bit resampler does it: for each resampled
// axis, output i takes inputs [first, first + count) weighted by Keys' cubic
// (a = -0.5) widened by max(n_in / n_out, 1) and normalised; weights are
// rounded to 22 fractional bits; a pass sums bytes x weights in int32 and
// rounds back to a byte, (acc + 2^21) >> 22 clamped to [0, 255].  The
// horizontal pass runs first (only if the width changes), then the vertical
// one (only if the height changes).  The host computes the taps (float64,
// like PIL) and a 256-entry table per channel of the rescale and
// normalisation (float32(float64(v) / 255) then (x - mean) / std in
// float32); so the kernel is integer up to that lookup and its results are
// bit-exact.
//
// Kernel: one workgroup (256 threads) per merge unit, 32 x 32 output
// pixels.  A unit that neither axis resizes reads its source pixels straight
// into an output block.  Otherwise it works in groups of output rows, sized
// so that the band of source rows their vertical taps read fits LDS; per
// group, the source block its taps touch is staged into LDS (in row chunks
// that fit), the horizontal pass turns it into the band, and the vertical
// pass reads the band and writes the group's output values.
//
// Sums of taps, four at a time.  A pass's input is held as signed bytes
// x' = x - 128 and each output's weights as three planes of signed base-256
// digits, w = a + 256 b + 65536 c with a, b, c in [-128, 127].  Then
//     sum x w = sum x' a + 256 sum x' b + 65536 sum x' c + 128 sum w,
// and each partial sum over four consecutive taps is one v_dot4_i32_i8 (four
// exact 8 x 8-bit products added to an int32).  The host folds 128 sum w and
// the rounding term into one constant per output.  It is all int32
// arithmetic, exact modulo 2^32 like PIL's own int32 sum, so the bytes are
// PIL's.  For that, consecutive taps must be consecutive bytes: the source
// block is staged as three channel planes, and the horizontal pass writes
// the band transposed (one LDS column per output column and channel, source
// rows consecutive), so the vertical pass finds its taps consecutive too.
// A window may start at any byte: it is read as aligned dwords and
// realigned with v_alignbyte.  An axis that is not resized (when the other
// one is) runs the same code with one tap of weight 1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <map>
#include <string>
#include <thread>
#include <tuple>
#include <utility>
#include <vector>

#include "device_util.h"
#include "internal.h"
#include "runtime.h"

namespace mimo {
namespace {

constexpr int kHfThreads = 256;
constexpr int kWeightBits = 22;              // fractional bits of the resampler's weights
constexpr int kMaxBandRows = 256;            // most source rows one group's vertical taps read
constexpr int kMaxStageBytes = 48 * 1024;    // LDS for one staged row chunk (three planes)
constexpr int kMaxStagePitch = kMaxStageBytes / 12;  // bytes per staged plane row (>= 4 rows a chunk)
constexpr int kRegDwords = 3;                // windows of up to 12 taps keep their tile's records in LDS
constexpr int kRegRecord = 4 * kRegDwords;   // (the record of such a window: 12 dwords at most)
constexpr int kRecBytes = 2 * kUnitPx * kRegRecord * 4;  // a tile's column and row records
constexpr int kStageBatch = 4;                // staging loads a thread issues before using them
constexpr int kLutBytes = 3 * 256 * 4;
constexpr int kBlockBytes = kUnitPx * kUnitPx * 4;  // the direct path's unit block (RGB per dword)
constexpr int64_t kParallelTapWork = 1 << 18;  // weights (outputs x taps) worth several host threads
constexpr int kBufferWord3 = 0x00020000;     // raw buffer resource word 3 (gfx9 family)
// Launches of the matrix-core instance so far (mimo_hf_matrix_dispatch_count).
std::atomic<int64_t> g_hf_matrix_dispatches{0};
// Zero dwords after the last table: a record's digit planes are read three
// dwords at a time, which may run up to two dwords past the last record.
constexpr size_t kTapsTail = 4;

// Per-item record of the contrast kernel (64 bytes).
struct HfItem {
    int64_t src_offset;   // bytes into the packed sources
    int64_t row_offset;   // first output row
    int64_t x_tab;        // int32 offset of the column table, or -1 when neither axis is resized
    int64_t y_tab;        // int32 offset of the row table, or -1 likewise
    int32_t src_h, src_w;
    int32_t channels;     // 3 or 4 (alpha ignored)
    int32_t blocks_h, blocks_w;
    int32_t ndx, ndy;     // dwords (four taps each) of an output column's / row's window
    int32_t group;        // output rows per vertical group (divides 32)
};
static_assert(sizeof(HfItem) == 64, "HfItem must stay 64 bytes");

// Per-tile record of the matrix-core instance (64 bytes), written by
// hf_tiles_kernel: all a tile needs before its first source load, so the
// tile reads one record instead of walking tile -> item -> tap tables.
struct HfTile {
    int64_t stage_off;   // bytes into the sources of the tile's first staged pixel (row ylo, column xlo)
    int64_t row_m;       // the unit's first row in merge-block order
    int64_t row_c;       // ... and in column order
    int32_t x_tab, y_tab;  // table offsets (x_tab < 0: no resize; stage_off is then the unit's first pixel)
    int32_t xlo, ylo;    // the tile's first staged source column and row
    int32_t row_bytes;
    int16_t ox0, oy0;    // the unit's first output column and row (the instance takes sides below 2^15)
    int16_t dst_w, dst_h;
    int16_t nrows, channels;
    int16_t ndx, ndy;
    int16_t pad[2];
};
constexpr int kMfMaxSide = 32767;  // output sides the matrix-core instance takes (HfTile's 16-bit fields)
static_assert(sizeof(HfTile) == 64, "HfTile must stay 64 bytes");

// An axis table is first[n_out] (each output's first input) followed by one
// record of rec_dwords(nd) int32 per output: the constant 2^21 + 128 sum w,
// then the digit planes a[nd], b[nd], c[nd], tap t in byte t % 4 of dword
// t / 4, zero past the output's own taps; padded to whole 16-byte vectors.
__host__ __device__ constexpr int rec_dwords(int nd) { return (1 + 3 * nd + 3) & ~3; }

struct HfArgs {
    const uint8_t *src;
    int64_t src_end;            // bytes readable from src
    const HfItem *items;
    const int64_t *tile_begin;  // [n + 1]
    const float *lut;           // [3][256]
    const int32_t *taps;
    void *rows;                 // merge-block order, nullable
    void *rows_col;             // column order, nullable
    int32_t n;
    // dynamic LDS, sized for the batch: [lut][band][stage]; the direct path
    // uses the bytes after the lut for its block
    int32_t band_bytes, stage_bytes;
    HfTile *tiles;              // matrix-core instance: one record per tile
    int64_t n_tiles;
    int32_t taps_bytes;         // the tables' exact size (the matrix-core instance reads them through a resource)
};

// workspace: [HfItem x n][int64 tile_begin x (n+1)][float lut x 768][int32 taps]
size_t hf_items_bytes(int32_t n) { return align256(sizeof(HfItem) * size_t(n)); }
size_t hf_prefix_bytes(int32_t n) { return align256(sizeof(int64_t) * (size_t(n) + 1)); }

// Dwords per staged source row and per band column: whole dwords with one
// spare for the realigning read, the band's count made odd so that the
// horizontal pass's writes of 32 columns fall into distinct LDS banks.
__host__ __device__ __forceinline__ int stage_pitch(int span) { return ((span + 3) >> 2) + 1; }
__host__ __device__ __forceinline__ int band_pitch(int rows) { return (((rows + 3) >> 2) + 1) | 1; }

// A raw buffer resource over [base & ~3, src_end), cut to `limit` bytes:
// reads past its end return zero.  `lead` is base's offset inside it.
struct SrcWindow {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t lead;
};

__device__ __forceinline__ SrcWindow src_window(const HfArgs &a, uint64_t base, uint64_t limit = ~uint64_t(0)) {
    const uint64_t start = base & ~uint64_t(3);
    const uint64_t end = reinterpret_cast<uint64_t>(a.src) + uint64_t(a.src_end);
    uint64_t avail = end > start ? end - start : 0;
    avail = avail < limit ? avail : limit;
    SrcWindow w;
    w.rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(start), 0,
                                               avail > 0x7FFFFFF0ull ? 0x7FFFFFF0 : int(avail),
                                               kBufferWord3);
    w.lead = uint32_t(base - start);
    return w;
}

// The 12 (RGB) or 16 (RGBA) bytes of the four consecutive pixels at byte
// offset `off` of the window (any alignment), in u[0..3].
__device__ __forceinline__ void load_quad_bytes(const SrcWindow &w, uint32_t off, int channels, uint32_t (&u)[4]) {
    const uint32_t al = off & ~3u, sh = off & 3u;
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(w.rsrc, int(al), 0, 0));
    uint32_t v4 = 0;
    if (channels == 4) v4 = __builtin_amdgcn_raw_buffer_load_b32(w.rsrc, int(al) + 16, 0, 0);
    u[0] = __builtin_amdgcn_alignbyte(v.y, v.x, sh);
    u[1] = __builtin_amdgcn_alignbyte(v.z, v.y, sh);
    u[2] = __builtin_amdgcn_alignbyte(v.w, v.z, sh);
    u[3] = __builtin_amdgcn_alignbyte(v4, v.w, sh);
}

// RGB bytes of four pixels, one pixel per dword (the direct path's block).
__device__ __forceinline__ u32x4 quad_pixels(const uint32_t (&u)[4], int channels) {
    if (channels == 3)  // R0 G0 B0 R1 | G1 B1 R2 G2 | B2 R3 G3 B3
        return u32x4{u[0] & 0x00FFFFFFu, __builtin_amdgcn_perm(u[1], u[0], 0x0C050403u),
                     __builtin_amdgcn_perm(u[2], u[1], 0x0C040302u), u[2] >> 8};
    return u32x4{u[0] & 0x00FFFFFFu, u[1] & 0x00FFFFFFu, u[2] & 0x00FFFFFFu, u[3] & 0x00FFFFFFu};
}

// Four pixels' bytes split into the three channel planes (one channel's
// four bytes per dword), as signed bytes x - 128.  (v_perm_b32 byte
// selectors: 0-3 pick a byte of the second operand, 4-7 of the first,
// 12 gives zero.)
__device__ __forceinline__ void quad_planes(const uint32_t (&u)[4], int channels, uint32_t (&p)[3]) {
    if (channels == 3) {
        // R: u0.b0 u0.b3 u1.b2 u2.b1   G: u0.b1 u1.b0 u1.b3 u2.b2   B: u0.b2 u1.b1 u2.b0 u2.b3
        p[0] = __builtin_amdgcn_perm(u[2], __builtin_amdgcn_perm(u[1], u[0], 0x0C060300u), 0x05020100u);
        p[1] = __builtin_amdgcn_perm(u[2], __builtin_amdgcn_perm(u[1], u[0], 0x0C070401u), 0x06020100u);
        p[2] = __builtin_amdgcn_perm(u[2], __builtin_amdgcn_perm(u[1], u[0], 0x0C0C0502u), 0x07040100u);
    } else {
        const uint32_t rb0 = __builtin_amdgcn_perm(u[1], u[0], 0x06040200u);  // R0 B0 R1 B1
        const uint32_t rb1 = __builtin_amdgcn_perm(u[3], u[2], 0x06040200u);  // R2 B2 R3 B3
        const uint32_t ga0 = __builtin_amdgcn_perm(u[1], u[0], 0x07050301u);  // G0 A0 G1 A1
        const uint32_t ga1 = __builtin_amdgcn_perm(u[3], u[2], 0x07050301u);  // G2 A2 G3 A3
        p[0] = __builtin_amdgcn_perm(rb1, rb0, 0x06040200u);
        p[1] = __builtin_amdgcn_perm(ga1, ga0, 0x06040200u);
        p[2] = __builtin_amdgcn_perm(rb1, rb0, 0x07050301u);
    }
#pragma unroll
    for (int c = 0; c < 3; ++c) p[c] ^= 0x80808080u;
}

// A window's record (rec_dwords(nd) <= kRegRecord dwords) copied to LDS.
__device__ __forceinline__ void copy_record(const int32_t *rec, int nd, uint32_t *dst) {
    const int vecs = rec_dwords(nd) >> 2;
#pragma unroll
    for (int v = 0; v < kRegDwords; ++v)
        if (v < vecs) reinterpret_cast<u32x4 *>(dst)[v] = *reinterpret_cast<const u32x4 *>(rec + 4 * v);
}

// sum over four taps of x * w (signed bytes) plus acc: v_dot4_i32_i8.
__device__ __forceinline__ int32_t dot4(uint32_t x, uint32_t w, int32_t acc) {
    return __builtin_amdgcn_sdot4(int32_t(x), int32_t(w), acc, false);
}

// Two sums s0, s1 shifted right by kWeightBits and saturated to a byte
// (unsigned, or signed for the _i8 form), in bytes 0 and 1 of the result;
// the upper half of the result register is left undefined.  In the
// dot-product instance the inputs come straight from v_dot4 instructions,
// whose results a VALU instruction may read only three wait states later;
// the compiler keeps that distance for its own instructions but cannot see
// into this one, hence the s_nop.
__device__ __forceinline__ uint32_t shift_pack_u8(int32_t s0, int32_t s1) {
    uint32_t d;
    asm("s_nop 2\n\tv_ashr_pk_u8_i32 %0, %1, %2, 22" : "=v"(d) : "v"(s0), "v"(s1));
    return d;
}
__device__ __forceinline__ uint32_t shift_pack_i8(int32_t s0, int32_t s1) {
    uint32_t d;
    asm("s_nop 2\n\tv_ashr_pk_i8_i32 %0, %1, %2, 22" : "=v"(d) : "v"(s0), "v"(s1));
    return d;
}
static_assert(kWeightBits == 22, "the shift in the packing instructions");

// Four bytes from two packed pairs: bytes 0, 1 of lo, then bytes 0, 1 of hi.
__device__ __forceinline__ uint32_t join_pairs(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Four window sums at once.  Both passes read four windows that start at the
// same offset in four neighbouring LDS lines (four band rows in the
// horizontal pass, four output columns in the vertical one), and both store
// those lines interleaved by dwords: at p, 16-byte group q holds dword q of
// each of the four.  So one 16-byte read gives dword q of all four windows.
// Each window starts `sh` bytes into its dword 0 and is realigned with
// v_alignbyte.  The three digit sums are chained, the higher one shifted
// into the next one's addend: s = ((sum c << 8) + sum b) << 8) + sum a + K,
// which saves setting up two of the three accumulators.
template <int ND>
__device__ __forceinline__ void quad_sums(const uint8_t *p, uint32_t sh, const uint32_t *r,
                                          int32_t (&s)[4]) {
    u32x4 g[ND + 1];
#pragma unroll
    for (int q = 0; q <= ND; ++q) g[q] = *reinterpret_cast<const u32x4 *>(p + 16 * q);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t x[ND];
#pragma unroll
        for (int q = 0; q < ND; ++q) x[q] = __builtin_amdgcn_alignbyte(g[q + 1][j], g[q][j], sh);
        int32_t sc = 0;
#pragma unroll
        for (int q = 0; q < ND; ++q) sc = dot4(x[q], r[1 + 2 * ND + q], sc);
        int32_t sb = int32_t(uint32_t(sc) << 8);
#pragma unroll
        for (int q = 0; q < ND; ++q) sb = dot4(x[q], r[1 + ND + q], sb);
        int32_t sa = int32_t((uint32_t(sb) << 8) + r[0]);
#pragma unroll
        for (int q = 0; q < ND; ++q) sa = dot4(x[q], r[1 + q], sa);
        s[j] = sa;
    }
}

// The same for windows of any length, the record read from memory.
__device__ __forceinline__ void quad_sums_any(const uint8_t *p, uint32_t sh, const int32_t *rec, int nd,
                                              int32_t (&s)[4]) {
    int32_t sa[4], sb[4], sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sa[j] = sb[j] = sc[j] = 0;
    u32x4 lo = *reinterpret_cast<const u32x4 *>(p);
    for (int q = 0; q < nd; ++q) {
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(p + 16 * (q + 1));
        const uint32_t wa = uint32_t(rec[1 + q]), wb = uint32_t(rec[1 + nd + q]), wc = uint32_t(rec[1 + 2 * nd + q]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t x = __builtin_amdgcn_alignbyte(hi[j], lo[j], sh);
            sa[j] = dot4(x, wa, sa[j]);
            sb[j] = dot4(x, wb, sb[j]);
            sc[j] = dot4(x, wc, sc[j]);
        }
        lo = hi;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        s[j] = int32_t(uint32_t(rec[0]) + uint32_t(sa[j]) + ((uint32_t(sb[j]) + (uint32_t(sc[j]) << 8)) << 8));
}

template <int ND>
__device__ __forceinline__ void window_sums(const uint8_t *p, uint32_t sh, const uint32_t *r,
                                            const int32_t *rec, int nd, int32_t (&s)[4]) {
    if (ND)
        quad_sums<ND ? ND : 1>(p, sh, r, s);
    else
        quad_sums_any(p, sh, rec, nd, s);
}

// Horizontal pass of the thread's output column over band row groups
// rq = tid / 32, + 8, ...: per channel, the window sums of four band rows,
// saturated to signed bytes (the column records' constants carry the -128
// that makes them the PIL bytes less 128, the vertical pass's input form),
// as one dword.
template <int ND>
__device__ __forceinline__ void h_pass(const uint8_t *stage, int sgroup, uint8_t *bcol, int bgroup, int groups,
                                       int x0, const uint32_t *r, const int32_t *rec, int nd,
                                       int tid) {
    for (int rq = tid >> 5; rq < groups; rq += kHfThreads / kUnitPx) {
        const uint8_t *src = stage + rq * 3 * sgroup + (x0 >> 2) * 16;
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            int32_t sum[4];
            window_sums<ND>(src + c * sgroup, uint32_t(x0) & 3u, r, rec, nd, sum);
            *reinterpret_cast<uint32_t *>(bcol + c * 8 * bgroup + rq * 16) =
                join_pairs(shift_pack_i8(sum[0], sum[1]), shift_pack_i8(sum[2], sum[3]));
        }
    }
}

// Vertical pass: items (row, patch column, channel, quad) of the group, the
// row fixed per thread; four output columns of one channel per item, the
// bytes through the rescale-and-normalise table, handed to put.
template <int ND, typename Put>
__device__ __forceinline__ void v_pass(const uint8_t *band, int bgroup, int y0, const float *lut,
                                       const uint32_t *r, const int32_t *rec, int nd, int n_items,
                                       int gsh, int tid, Put &&put) {
    for (int idx = tid; idx < n_items; idx += kHfThreads) {
        const int qd = idx & 3;
        const int mc = idx >> (2 + gsh);
        const int mw = mc >= 3 ? 1 : 0;
        const int c = mc - 3 * mw;
        int32_t sum[4];
        window_sums<ND>(band + (c * 8 + mw * 4 + qd) * bgroup + (y0 >> 2) * 16, uint32_t(y0) & 3u, r, rec, nd, sum);
        const uint32_t bytes = join_pairs(shift_pack_u8(sum[0], sum[1]), shift_pack_u8(sum[2], sum[3]));
        const float *lut_c = lut + c * 256;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = lut_c[(bytes >> (8 * j)) & 255u];
        put(mw, c, qd, v);
    }
}

// Four output values (4 pixels of one patch row, one channel) into both
// temporal slots of a row.
template <typename OutT>
__device__ __forceinline__ void store_pair(OutT *row_ptr, const float (&v)[4]);

template <>
__device__ __forceinline__ void store_pair<float>(float *p, const float (&v)[4]) {
    const f32x4 q = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(q, reinterpret_cast<f32x4 *>(p));
    __builtin_nontemporal_store(q, reinterpret_cast<f32x4 *>(p + kPlane));
}

template <>
__device__ __forceinline__ void store_pair<uint16_t>(uint16_t *p, const float (&v)[4]) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 a = {__bf16(v[0]), __bf16(v[1])}, b = {__bf16(v[2]), __bf16(v[3])};
    const u32x2 q = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
    __builtin_nontemporal_store(q, reinterpret_cast<u32x2 *>(p));
    __builtin_nontemporal_store(q, reinterpret_cast<u32x2 *>(p + kPlane));
}

// ---- the matrix-core instance -------------------------------------------
//
// Both passes of one tile are integer matrix products with banded weight
// matrices: band[r][x] = sum_k stage[r][k] Wx[k][x] (r a band row, k a staged
// source column, x an output column), then out[y][x] = sum_r Wy[y][r]
// band[r][x].  When every tile of a batch reads at most 64 source columns
// and 64 band rows with windows of at most 12 taps (downscales up to about
// 1.8x, and upscales), each 16 x 16 block of either product is one
// v_mfma_i32_16x16x64_i8 per weight digit plane: exact int32 sums of
// signed-byte products, joined by shift-adds (digit_product below).  A
// tile's banded matrices are built in LDS (zero but for
// each output's own taps) as 64-byte lines, which the matrix cores read as
// 16-byte fragments: lane l reads line l % 16, bytes 16 (l / 16) .. + 15,
// and holds result rows 4 (l / 16) .. + 3 of column l % 16.
constexpr int kMfmaSpan = 64;  // the K of one instruction: staged columns, band rows
constexpr int kMfMaxNd = 3;    // window dwords (12 taps) the instance takes
// LDS (20 KB: eight workgroups fit a CU): two buffers of one staged
// channel plane each (the horizontal pass takes the channels in turn, the
// other planes wait in registers), the band, and Wx; the vertical pass's
// table then takes the first buffer and Wy takes Wx's place.  The records'
// constants stay in registers.
constexpr int kMfPlane = kMfmaSpan * 64;                 // [64 rows][64 bytes]
constexpr int kMfStage0 = 0;
constexpr int kMfStage1 = kMfStage0 + kMfPlane;
constexpr int kMfBand = kMfStage1 + kMfPlane;            // [channel][32 columns][64 rows]
constexpr int kMfWx = kMfBand + 3 * kUnitPx * 64;        // [digit plane][32 output columns][64]
constexpr int kMfLdsBytes = kMfWx + 3 * kUnitPx * 64;
constexpr int kMfLut = kMfStage0;                        // float [3][256], after the horizontal pass
constexpr int kMfWy = kMfWx;                             // [digit plane][32 output rows][64], likewise
static_assert(kLutBytes <= kMfPlane && kMfLdsBytes == 20 * 1024, "the vertical pass's tables fit");

typedef int32_t i32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4v lds_frag(const uint8_t *p) {
    return __builtin_bit_cast(i32x4v, *reinterpret_cast<const u32x4 *>(p));
}

// A x B for B = (c << 16) + (b << 8) + a (signed digit planes), plus K per
// column of the result (lane l's column l % 16): the products of planes c
// and b are independent, (A Bb << 8) + K seeds the product of plane a, and
// (A Bc << 16) joins last, so each value takes two shift-adds.  The sums
// wrap modulo 2^32, which is harmless, since the true sum fits an int32.
__device__ __forceinline__ i32x4v digit_product(i32x4v a, i32x4v bc, i32x4v bb, i32x4v ba, int32_t k) {
    const i32x4v zero = {0, 0, 0, 0};
    const i32x4v pc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bc, zero, 0, 0, 0);
    const i32x4v pb = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bb, zero, 0, 0, 0);
    i32x4v seed;
#pragma unroll
    for (int i = 0; i < 4; ++i) seed[i] = int32_t((uint32_t(pb[i]) << 8) + uint32_t(k));
    const i32x4v pa = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, ba, seed, 0, 0, 0);
    i32x4v r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = int32_t((uint32_t(pc[i]) << 16) + uint32_t(pa[i]));
    return r;
}

// Every 64-byte line the matrix cores read (staged rows, weight lines, band
// lines) keeps its four 16-byte chunks XOR-swizzled by bits 2-3 of the
// line's index: a fragment read's 16 lanes, which read one chunk of 16
// consecutive lines, then fall into distinct banks (unswizzled, lines 4
// apart share banks), and every 16-byte read stays aligned.
__device__ __forceinline__ int swizzled_dword(int line, int dw) {
    return (((dw >> 2) ^ ((line >> 2) & 3)) << 2) | (dw & 3);
}

// Line i of a banded weight matrix (64 bytes): the digits dg placed at byte
// o, zero elsewhere.  The line is zeroed first, 16 bytes at a time, each
// group of 4 lines in its own chunk order (lines are 64 bytes apart, so
// lanes writing the same chunk of lines 4 apart would share banks); then
// four dwords take the digits shifted by s = o % 4 bytes,
// each the byte-aligned join of two neighbouring digit dwords.  The
// alignment instruction reads its shift (4 - s) modulo 4: at s = 0 the join
// of dwords q and q - 1 is dword q - 1, so the writes start one dword
// earlier, at ceil(o / 4) - 1, and no case needs a select.  No write needs a
// condition either: the digits end by byte 63 (o + 4 nd is at most the
// tile's span of 64), so a dword index past the line carries zeros only,
// and it wraps to a dword before the digits, which is zero as well.
__device__ __forceinline__ void write_line(uint8_t *line, int i, const uint32_t (&dg)[kMfMaxNd], int o) {
    const int key16 = ((i >> 2) & 3) << 4;  // the group's chunk order, in bytes
#pragma unroll
    for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4 *>(line + ((16 * k) ^ key16)) = u32x4{0u, 0u, 0u, 0u};
    const int first = ((o + 3) >> 2) - 1;
    const uint32_t shift = uint32_t(-o) & 3u;  // (4 - s) modulo 4
    const int key = ((i >> 2) & 3) << 2;       // the line's chunk swizzle, as a dword index
    uint32_t *w = reinterpret_cast<uint32_t *>(line);
    uint32_t prev = 0;
#pragma unroll
    for (int q = 0; q <= kMfMaxNd; ++q) {
        const uint32_t cur = q < kMfMaxNd ? dg[q] : 0u;
        w[((first + q) & (kMfmaSpan / 4 - 1)) ^ key] = __builtin_amdgcn_alignbyte(cur, prev, shift);
        prev = cur;
    }
}

template <typename OutT>
__device__ __forceinline__ void resize_mfma(const HfArgs &a, const HfTile &td, int tid, uint8_t *lds8) {
    const int ndx = td.ndx, ndy = td.ndy;
    const int oy0 = td.oy0, ox0 = td.ox0;
    const int xlo = td.xlo, ylo = td.ylo;
    const int nrows = td.nrows;  // <= 64 (the host checked), so are the columns
    const int C = td.channels;
    const uint32_t row_bytes = uint32_t(td.row_bytes);
    // the tables through a buffer resource (32-bit offsets)
    const __amdgpu_buffer_rsrc_t tabs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(a.taps), 0, a.taps_bytes, kBufferWord3);
    auto tab = [&](uint32_t dword) { return int32_t(__builtin_amdgcn_raw_buffer_load_b32(tabs, int(4 * dword), 0, 0)); };
    const uint32_t xrec = uint32_t(td.x_tab + td.dst_w), yrec = uint32_t(td.y_tab + td.dst_h);  // first records
    const uint32_t rdx = uint32_t(rec_dwords(ndx)), rdy = uint32_t(rec_dwords(ndy));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 15, lkb = (lane >> 4) * 16;  // the lane's fragment line and bytes

    // Everything the tile reads from memory, first: the source block (64
    // columns x 64 rows, 4 quads per thread), Wx's and Wy's lines (one per
    // thread: digit plane, output), the records' constants of the lane's
    // result columns, and the table.  The block's resource ends with row
    // nrows - 1's reads (a row's reads span 64 C + 8 bytes at most), so
    // later rows read zero without a memory access.
    const uint64_t stage_base = reinterpret_cast<uint64_t>(a.src) + uint64_t(td.stage_off);
    const SrcWindow win = src_window(a, stage_base,
                                     (stage_base & 3u) + uint64_t(nrows - 1) * row_bytes + uint64_t(64 * C + 8));
    static_assert(kMfmaSpan * kMfmaSpan / 4 == kStageBatch * kHfThreads, "one staging batch per tile");
    uint32_t u[kStageBatch][4];
#pragma unroll
    for (int k = 0; k < kStageBatch; ++k) {
        const uint32_t idx = uint32_t(tid + k * kHfThreads);
        load_quad_bytes(win, win.lead + __umul24(idx >> 4, row_bytes) + (idx & 15u) * uint32_t(4 * C), C, u[k]);
    }
    // waves 0-1 build Wx's lines, waves 2-3 Wy's: thread t of the pair,
    // t < 96, line t (digit plane t / 32, output t % 32); the pair's other
    // threads load what line 95 loads, so that every load is unconditional
    const bool xaxis = wave < 2;
    const int pt = tid & 127;
    const bool writer = pt < 3 * kUnitPx;
    const int lt = min(pt, 3 * kUnitPx - 1);
    const int lp = lt >> 5, li = lt & (kUnitPx - 1);
    const int nd = xaxis ? ndx : ndy;  // >= 1
    // digit plane lp of the line's record, read three dwords at a time (past
    // its nd dwords: the next record or the tables' zero tail, masked)
    const uint32_t dbase = (xaxis ? xrec + __umul24(uint32_t(ox0 + li), rdx) : yrec + __umul24(uint32_t(oy0 + li), rdy)) +
                           1 + lp * nd;
    uint32_t dg[kMfMaxNd];
#pragma unroll
    for (int q = 0; q < kMfMaxNd; ++q) {
        const uint32_t v = uint32_t(tab(dbase + q));
        dg[q] = q < nd ? v : 0u;
    }
    const int lo = tab(xaxis ? uint32_t(td.x_tab + ox0 + li) : uint32_t(td.y_tab + oy0 + li)) - (xaxis ? xlo : ylo);
    // the records' constants of the lane's result column: a wave's
    // horizontal blocks (wave, wave + 4) all lie in column block wave % 2,
    // its vertical ones (wave + 4 j) in row block (wave / 2) % 2
    static_assert(kHfThreads / 64 == 4, "block assignment");
    const int32_t kx = tab(xrec + __umul24(uint32_t(ox0 + 16 * (wave & 1) + lrow), rdx));
    const int32_t ky = tab(yrec + __umul24(uint32_t(oy0 + 16 * ((wave >> 1) & 1) + lrow), rdy));
    float lut_v[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) lut_v[i] = a.lut[tid + i * kHfThreads];
    if (xaxis && writer) write_line(lds8 + kMfWx + (lp * kUnitPx + li) * 64, li, dg, lo);

    // the block as channel planes of signed bytes, all 64 rows: columns
    // past the tile's span, and rows past nrows (zero, or in a source
    // narrower than a row's reads, the bytes that follow), meet only zero
    // weights; plane 0 now
    uint32_t pl[kStageBatch][3];
#pragma unroll
    for (int k = 0; k < kStageBatch; ++k) quad_planes(u[k], C, pl[k]);
    uint32_t waddr[kStageBatch];  // row idx / 16, dword idx % 16, swizzled
#pragma unroll
    for (int k = 0; k < kStageBatch; ++k) {
        const int idx = tid + k * kHfThreads;
        waddr[k] = uint32_t(4 * ((idx & ~15) | swizzled_dword(idx >> 4, idx & 15)));
    }
    auto write_plane = [&](int c, int buf) {
#pragma unroll
        for (int k = 0; k < kStageBatch; ++k) *reinterpret_cast<uint32_t *>(lds8 + buf + waddr[k]) = pl[k][c];
    };
    write_plane(0, kMfStage0);
    __syncthreads();

    // the lane's chunk of its line, swizzled (lines of a 16-line block share
    // their index's bits 2-3 with lrow)
    const int swz = (lrow >> 2) & 3;
    const int lks = 16 * ((lkb >> 4) ^ swz);
    // horizontal pass, one channel at a time: blocks (16 band rows, 16
    // output columns), two per wave so that their matrix-core products
    // overlap: wave w takes column block w % 2 and row blocks w / 2 and
    // w / 2 + 2 (the second only where the band reaches it; otherwise the
    // first is computed twice and stored once).  The lane's LDS addresses
    // are the same in every channel but for the buffer and the band's
    // channel offset, so they are formed once.
    const int rblocks = (nrows + 15) >> 4;  // 1 .. 4
    const int cb = wave & 1, rb0 = wave >> 1;
    const bool one = rb0 < rblocks, two = rb0 + 2 < rblocks;
    const uint32_t a0 = uint32_t((rb0 * 16 + lrow) * 64 + lks);
    const uint32_t a1 = two ? a0 + 2 * 16 * 64 : a0;
    const uint8_t *wl = lds8 + kMfWx + (cb * 16 + lrow) * 64 + lks;
    // rows 4 (lane / 16) .. + 3 of column cb * 16 + lrow, as signed bytes
    const uint32_t st_line = uint32_t(kMfBand + (cb * 16 + lrow) * 64 + lkb / 4);
    const uint32_t s0 = st_line + 16 * (rb0 ^ swz), s1 = st_line + 16 * ((rb0 + 2) ^ swz);
    auto h_block = [&](int buf, uint32_t aoff) {
        return digit_product(lds_frag(lds8 + buf + aoff), lds_frag(wl + 2 * kUnitPx * 64), lds_frag(wl + kUnitPx * 64),
                             lds_frag(wl), kx);
    };
    auto h_store = [&](int c, uint32_t soff, const i32x4v &acc) {
        *reinterpret_cast<uint32_t *>(lds8 + c * kUnitPx * 64 + soff) =
            join_pairs(shift_pack_i8(acc[0], acc[1]), shift_pack_i8(acc[2], acc[3]));
    };
    auto h_pass_channel = [&](int c, int buf) {
        if (one) {
            const i32x4v acc = h_block(buf, a0);
            const i32x4v acc2 = h_block(buf, a1);
            h_store(c, s0, acc);
            if (two) h_store(c, s1, acc2);
        }
    };
    h_pass_channel(0, kMfStage0);
    write_plane(1, kMfStage1);
    __syncthreads();
    h_pass_channel(1, kMfStage1);
    write_plane(2, kMfStage0);
    __syncthreads();
    h_pass_channel(2, kMfStage0);
    __syncthreads();

    // the vertical pass's table and Wy, where the first buffer and Wx were
#pragma unroll
    for (int i = 0; i < 3; ++i) reinterpret_cast<float *>(lds8 + kMfLut)[tid + i * kHfThreads] = lut_v[i];
    if (!xaxis && writer) write_line(lds8 + kMfWy + (lp * kUnitPx + li) * 64, li, dg, lo);
    __syncthreads();

    // vertical pass, transposed: out^T[x][y] = sum_r band^T[x][r] Wy^T[r][y],
    // blocks (channel, 16 output columns, 16 output rows), three per wave;
    // lane l holds output columns 4 (l / 16) .. + 3 of row l % 16: four
    // pixels of a patch row
    const float *lut = reinterpret_cast<const float *>(lds8 + kMfLut);
    const int lane_off = lrow * kPatch + lkb / 4;  // py * 16 + px of the lane's first value
    OutT *out_m = a.rows ? static_cast<OutT *>(a.rows) + td.row_m * kRowLen + lane_off : nullptr;
    OutT *out_c = a.rows_col ? static_cast<OutT *>(a.rows_col) + td.row_c * kRowLen + lane_off : nullptr;
    static_assert(3 * 2 * 2 == 3 * (kHfThreads / 64), "three vertical blocks per wave");
    i32x4v vacc[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int blk = wave + j * (kHfThreads / 64);
        const int xb = blk & 1, yb = (blk >> 1) & 1, c = blk >> 2;
        const i32x4v av = lds_frag(lds8 + kMfBand + (c * kUnitPx + xb * 16 + lrow) * 64 + lks);
        const uint8_t *wl = lds8 + kMfWy + (yb * 16 + lrow) * 64 + lks;
        vacc[j] = digit_product(av, lds_frag(wl + 2 * kUnitPx * 64), lds_frag(wl + kUnitPx * 64), lds_frag(wl),
                                ky);
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int blk = wave + j * (kHfThreads / 64);
        const int xb = blk & 1, yb = (blk >> 1) & 1, c = blk >> 2;
        const uint32_t bytes = join_pairs(shift_pack_u8(vacc[j][0], vacc[j][1]), shift_pack_u8(vacc[j][2], vacc[j][3]));
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = lut[c * 256 + ((bytes >> (8 * q)) & 255u)];
        // unit row yb * 2 + xb (patch row yb, column xb), channel c
        const int off = (yb * kMerge + xb) * kRowLen + c * (kTemporal * kPlane);
        if (out_m) store_pair<OutT>(out_m + off, v);
        if (out_c) store_pair<OutT>(out_c + off, v);
    }
}

// A unit that neither axis resizes, from its tile record: its 32 x 32
// source pixels into an LDS block (after the table), then through the table
// to the outputs.
template <typename OutT>
__device__ __forceinline__ void direct_unit(const HfArgs &a, const HfTile &td, int tid, uint32_t *lds) {
    float *lut = reinterpret_cast<float *>(lds);
    uint32_t *block = lds + kLutBytes / 4;
    for (int i = tid; i < 3 * 256; i += kHfThreads) lut[i] = a.lut[i];
    const int C = td.channels;
    const uint32_t row_bytes = uint32_t(td.row_bytes);
    const SrcWindow win = src_window(a, reinterpret_cast<uint64_t>(a.src) + uint64_t(td.stage_off));
    for (int idx = tid; idx < kUnitPx * kUnitPx / 4; idx += kHfThreads) {
        const int r = idx >> 3, q = idx & 7;
        uint32_t u[4];
        load_quad_bytes(win, win.lead + __umul24(uint32_t(r), row_bytes) + uint32_t(4 * q * C), C, u);
        *reinterpret_cast<u32x4 *>(&block[r * kUnitPx + 4 * q]) = quad_pixels(u, C);
    }
    __syncthreads();
    // items (row, patch column, channel, quad), the row fixed per thread
    const int yl = (tid >> 2) & (kUnitPx - 1);
    const int py_off = (yl & (kPatch - 1)) * kPatch;
    const int64_t mh2 = (yl >> 4) * kMerge;
    OutT *out_m = a.rows ? static_cast<OutT *>(a.rows) + (td.row_m + mh2) * kRowLen + py_off : nullptr;
    OutT *out_c = a.rows_col ? static_cast<OutT *>(a.rows_col) + (td.row_c + mh2) * kRowLen + py_off : nullptr;
    for (int idx = tid; idx < kUnitPx * 2 * 3 * 4; idx += kHfThreads) {
        const int qd = idx & 3;
        const int mc = idx >> 7;
        const int mw = mc >= 3 ? 1 : 0;
        const int c = mc - 3 * mw;
        const uint32_t *px = &block[yl * kUnitPx + mw * kPatch + qd * 4];
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = lut[c * 256 + ((px[j] >> (8 * c)) & 255u)];
        const int off = mw * kRowLen + c * (kTemporal * kPlane) + qd * 4;
        if (out_m) store_pair<OutT>(out_m + off, v);
        if (out_c) store_pair<OutT>(out_c + off, v);
    }
}

// One thread per tile of a matrix-core batch (every item one tile per
// unit): its record, from the item and the tap tables.
__global__ __launch_bounds__(256) void hf_tiles_kernel(HfArgs a) {
    const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (t >= a.n_tiles) return;
    int lo = 0, hi = a.n;  // the item: largest i with tile_begin[i] <= t
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.tile_begin[mid] <= t) lo = mid; else hi = mid;
    }
    const HfItem d = a.items[lo];
    const int unit = int(t - a.tile_begin[lo]);
    const int br = unit / d.blocks_w, bc = unit - br * d.blocks_w;
    HfTile r;
    r.ox0 = int16_t(bc * kUnitPx);
    r.oy0 = int16_t(br * kUnitPx);
    r.dst_w = int16_t(d.blocks_w * kUnitPx);
    r.dst_h = int16_t(d.blocks_h * kUnitPx);
    r.row_m = d.row_offset + int64_t(br * d.blocks_w + bc) * kRowsPerUnit;
    r.row_c = d.row_offset + int64_t(bc * d.blocks_h + br) * kRowsPerUnit;
    r.row_bytes = d.src_w * d.channels;
    r.channels = int16_t(d.channels);
    r.x_tab = int32_t(d.x_tab);
    r.y_tab = int32_t(d.y_tab);
    r.ndx = int16_t(d.ndx);
    r.ndy = int16_t(d.ndy);
    r.pad[0] = r.pad[1] = 0;
    if (d.x_tab >= 0) {
        const int32_t *xt = a.taps + d.x_tab;
        const int32_t *yt = a.taps + d.y_tab;
        r.xlo = xt[bc * kUnitPx];
        r.ylo = yt[br * kUnitPx];
        r.nrows = int16_t(yt[br * kUnitPx + kUnitPx - 1] - r.ylo + 4 * d.ndy);
    } else {
        r.xlo = bc * kUnitPx;
        r.ylo = br * kUnitPx;
        r.nrows = kUnitPx;
    }
    r.stage_off = d.src_offset + int64_t(r.ylo) * r.row_bytes + int64_t(r.xlo) * d.channels;
    a.tiles[t] = r;
}

// The dot-product instance runs six waves per SIMD: a 6000x4000 batch's
// tile takes about 26 KB of LDS there, so six workgroups fill a CU, and the
// register budget that leaves (80) holds it without spilling.  The
// matrix-core instance's tile takes 20 KB, so it runs eight (64 registers).
template <typename OutT, bool kMfma>
__global__ __launch_bounds__(kHfThreads) __attribute__((amdgpu_waves_per_eu(kMfma ? 8 : 6))) void hf_preprocess_kernel(HfArgs a) {
    extern __shared__ uint32_t lds[];
    float *lut = reinterpret_cast<float *>(lds);  // [3][256]
    uint32_t *recs = lds + kLutBytes / 4;  // [column records x 32][row records x 32], kRegRecord dwords each
    uint8_t *region = reinterpret_cast<uint8_t *>(lds) + kLutBytes + kRecBytes;
    const int64_t tile = xcd_contiguous_tile(blockIdx.x, gridDim.x);
    if (kMfma) {
        const HfTile td = a.tiles[tile];
        if (td.x_tab < 0)
            direct_unit<OutT>(a, td, threadIdx.x, lds);
        else
            resize_mfma<OutT>(a, td, threadIdx.x, reinterpret_cast<uint8_t *>(lds));
        return;
    }
    const int img = find_segment(a.tile_begin, a.n, tile);
    const HfItem d = a.items[img];
    // An item lists one tile per (merge unit, group of G output rows); G is
    // a power of two, 32 (one tile per unit) unless the vertical taps of 32
    // rows do not fit the band.
    const int G = d.group;
    const int gsh = __builtin_ctz(unsigned(G));
    const int local = int(tile - a.tile_begin[img]);
    const int unit = local >> (5 - gsh);
    const int g0 = (local & ((kUnitPx >> gsh) - 1)) << gsh;  // the group's first row in the unit
    const int br = div_small(unit, d.blocks_w, 1.0f / float(d.blocks_w));
    const int bc = unit - br * d.blocks_w;
    const int oy0 = br * kUnitPx, ox0 = bc * kUnitPx;
    const int tid = threadIdx.x;
    const uint8_t *img_src = a.src + d.src_offset;
    const int C = d.channels;
    const uint32_t row_bytes = uint32_t(d.src_w) * uint32_t(C);  // < 2^23 (the host checked)

    // The thread's output row of the group in the vertical pass (and in the
    // direct path's stores): the same for each of its work items.
    const int yl = (tid >> 2) & (G - 1);
    // Output values (yl, mw, c, qd): 4 pixels of one patch row and channel,
    // into both temporal slots of the unit's row, in the orders asked for.
    // The thread's pixel row y of the unit fixes its rows' base pointers.
    const int y_unit = g0 + yl;
    const int64_t row_m = d.row_offset + int64_t(br * d.blocks_w + bc) * kRowsPerUnit + (y_unit >> 4) * kMerge;
    const int64_t row_c = d.row_offset + int64_t(bc * d.blocks_h + br) * kRowsPerUnit + (y_unit >> 4) * kMerge;
    const int py_off = (y_unit & (kPatch - 1)) * kPatch;
    OutT *out_m = a.rows ? static_cast<OutT *>(a.rows) + row_m * kRowLen + py_off : nullptr;
    OutT *out_c = a.rows_col ? static_cast<OutT *>(a.rows_col) + row_c * kRowLen + py_off : nullptr;
    auto put = [&](int mw, int c, int qd, const float (&v)[4]) {
        const int off = mw * kRowLen + c * (kTemporal * kPlane) + qd * 4;
        if (out_m) store_pair<OutT>(out_m + off, v);
        if (out_c) store_pair<OutT>(out_c + off, v);
    };
    const int n_items = G * 2 * 3 * 4;  // (row, patch column, channel, quad); a wavefront: 16 rows x 4 quads

    if (d.x_tab < 0) {
        // no resize: the unit's 32 x 32 source pixels go to the block
        for (int i = tid; i < 3 * 256; i += kHfThreads) lut[i] = a.lut[i];
        uint32_t *block = reinterpret_cast<uint32_t *>(region);
        const SrcWindow win = src_window(a, reinterpret_cast<uint64_t>(img_src) +
                                                uint64_t(int64_t(oy0) * row_bytes + int64_t(ox0) * C));
        for (int idx = tid; idx < kUnitPx * kUnitPx / 4; idx += kHfThreads) {
            const int r = idx >> 3, q = idx & 7;
            uint32_t u[4];
            load_quad_bytes(win, win.lead + __umul24(uint32_t(r), row_bytes) + uint32_t(4 * q * C), C, u);
            *reinterpret_cast<u32x4 *>(&block[r * kUnitPx + 4 * q]) = quad_pixels(u, C);
        }
        __syncthreads();
        for (int idx = tid; idx < n_items; idx += kHfThreads) {
            const int qd = idx & 3;
            const int mc = idx >> (2 + gsh);
            const int mw = mc >= 3 ? 1 : 0;
            const int c = mc - 3 * mw;
            const uint32_t *px = &block[(g0 + yl) * kUnitPx + mw * kPatch + qd * 4];
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = lut[c * 256 + ((px[j] >> (8 * c)) & 255u)];
            put(mw, c, qd, v);
        }
        return;
    }

    const int dst_w = d.blocks_w * kUnitPx, dst_h = d.blocks_h * kUnitPx;
    const int32_t *xt = a.taps + d.x_tab;  // first[dst_w], then the records
    const int32_t *yt = a.taps + d.y_tab;
    const int ndx = d.ndx, ndy = d.ndy;
    const int hx = tid & 31;  // the thread's output column in the horizontal pass
    const int oy_a = oy0 + g0;
    const int32_t *xrec = xt + dst_w + int64_t(ox0 + hx) * rec_dwords(ndx);
    const int32_t *yrec = yt + dst_h + int64_t(oy_a + yl) * rec_dwords(ndy);
    // the tile's records (windows of up to 12 taps) into LDS: 32 columns, G rows
    const uint32_t *xr = recs + hx * kRegRecord;
    const uint32_t *yr = recs + (kUnitPx + yl) * kRegRecord;
    if (tid < kUnitPx) {
        if (ndx <= kRegDwords) copy_record(xt + dst_w + int64_t(ox0 + tid) * rec_dwords(ndx), ndx, recs + tid * kRegRecord);
    } else if (tid < kUnitPx + G) {
        const int i = tid - kUnitPx;
        if (ndy <= kRegDwords)
            copy_record(yt + dst_h + int64_t(oy_a + i) * rec_dwords(ndy), ndy, recs + (kUnitPx + i) * kRegRecord);
    }
    for (int i = tid; i < 3 * 256; i += kHfThreads) lut[i] = a.lut[i];
    // the tile's source block: columns [xlo, xlo + xspan), rows [ylo, ylo + nrows)
    // (4 nd inputs past each axis's last first input; bytes past an output's
    // own taps have zero weight, and reads past the sources return zero)
    const int xlo = xt[ox0];
    const int xspan = xt[ox0 + kUnitPx - 1] - xlo + 4 * ndx;
    const int x0 = xt[ox0 + hx] - xlo;
    const int ylo = yt[oy_a];
    const int nrows = yt[oy_a + G - 1] - ylo + 4 * ndy;  // <= kMaxBandRows (the host sized G)
    const int y0 = yt[oy_a + yl] - ylo;
    // LDS lines interleaved by dwords in groups of four (see quad_sums):
    // the staged planes as [row / 4][channel][dword of the row][row % 4],
    // the band as [channel][column / 4][dword of the column][column % 4]
    const int sgroup = 16 * stage_pitch(xspan);  // bytes per (row group, channel)
    const int bgroup = 16 * band_pitch(nrows);   // bytes per (channel, column group)
    const int quads = (xspan + 3) >> 2;
    // staged rows per chunk: a multiple of 4, at least 4 (the host checked)
    const int chunk = min((nrows + 3) & ~3, (a.stage_bytes / (12 * stage_pitch(xspan))) & ~3);
    uint8_t *band = region;
    uint8_t *stage = region + a.band_bytes;
    // staging work items (row, quad) with the quads of a row padded to 2^lq
    const int lq = quads > 1 ? 32 - __builtin_clz(unsigned(quads - 1)) : 0;
    for (int r0 = 0; r0 < nrows; r0 += chunk) {
        const int nr = min(chunk, nrows - r0);
        const SrcWindow win = src_window(a, reinterpret_cast<uint64_t>(img_src) +
                                                uint64_t(int64_t(ylo + r0) * row_bytes + int64_t(xlo) * C));
        const int total = nr << lq;
        for (int base = tid; base < total; base += kStageBatch * kHfThreads) {
            // all of a batch's loads first (reads outside the window return
            // zero, so an item past the end may load too), then their planes
            uint32_t u[kStageBatch][4];
#pragma unroll
            for (int k = 0; k < kStageBatch; ++k) {
                const int idx = base + k * kHfThreads;
                const uint32_t r = uint32_t(idx >> lq), q = uint32_t(idx & ((1 << lq) - 1));
                load_quad_bytes(win, win.lead + __umul24(r, row_bytes) + q * uint32_t(4 * C), C, u[k]);
            }
#pragma unroll
            for (int k = 0; k < kStageBatch; ++k) {
                const int idx = base + k * kHfThreads;
                const int r = idx >> lq, q = idx & ((1 << lq) - 1);
                if (idx < total && q < quads) {
                    uint32_t pl[3];
                    quad_planes(u[k], C, pl);
                    uint8_t *dst = stage + (r >> 2) * 3 * sgroup + q * 16 + (r & 3) * 4;
#pragma unroll
                    for (int c = 0; c < 3; ++c) *reinterpret_cast<uint32_t *>(dst + c * sgroup) = pl[c];
                }
            }
        }
        __syncthreads();
        // horizontal pass: band rows r0 + 4 rq .. + 3 of the thread's column
        // (rows past nr hold bytes of no weight: their source rows lie past
        // every window)
        uint8_t *bcol = band + (hx >> 2) * bgroup + (r0 >> 2) * 16 + (hx & 3) * 4;
        const int groups = (nr + 3) >> 2;
        switch (ndx) {
        case 1: h_pass<1>(stage, sgroup, bcol, bgroup, groups, x0, xr, xrec, ndx, tid); break;
        case 2: h_pass<2>(stage, sgroup, bcol, bgroup, groups, x0, xr, xrec, ndx, tid); break;
        case 3: h_pass<3>(stage, sgroup, bcol, bgroup, groups, x0, xr, xrec, ndx, tid); break;
        default: h_pass<0>(stage, sgroup, bcol, bgroup, groups, x0, xr, xrec, ndx, tid); break;
        }
        __syncthreads();
    }
    switch (ndy) {
    case 1: v_pass<1>(band, bgroup, y0, lut, yr, yrec, ndy, n_items, gsh, tid, put); break;
    case 2: v_pass<2>(band, bgroup, y0, lut, yr, yrec, ndy, n_items, gsh, tid, put); break;
    case 3: v_pass<3>(band, bgroup, y0, lut, yr, yrec, ndy, n_items, gsh, tid, put); break;
    default: v_pass<0>(band, bgroup, y0, lut, yr, yrec, ndy, n_items, gsh, tid, put); break;
    }
}

// ----------------------------------------------------------------- host side

// Keys' cubic convolution kernel, a = -0.5.
double keys_bicubic(double x) {
    const double a = -0.5;
    x = std::fabs(x);
    if (x < 1.0) return ((a + 2.0) * x - (a + 3.0)) * x * x + 1.0;
    if (x < 2.0) return (((x - 5.0) * x + 8.0) * x - 4.0) * a;
    return 0.0;
}

int axis_taps_per_output(int64_t n_in, int64_t n_out) {
    const double scale = double(n_in) / double(n_out);
    const double support = 2.0 * (scale < 1.0 ? 1.0 : scale);
    return int(std::ceil(support)) * 2 + 1;
}

// PIL's window of output i on an axis of n_in inputs: [lo, hi).
struct AxisMap {
    int64_t n_in, n_out;
    double scale, widen, support;
    AxisMap(int64_t in, int64_t out) : n_in(in), n_out(out) {
        scale = double(n_in) / double(n_out);
        widen = scale < 1.0 ? 1.0 : scale;
        support = 2.0 * widen;
    }
    void window(int64_t i, int64_t &lo, int64_t &hi, double &centre) const {
        centre = (double(i) + 0.5) * scale;
        lo = int64_t(centre - support + 0.5);
        if (lo < 0) lo = 0;
        hi = int64_t(centre + support + 0.5);
        if (hi > n_in) hi = n_in;
    }
};

// Every output of an axis gets the same k taps, the most any output of the
// axis has: its window [first, first + k) is moved left where it would run
// past the last input (its own taps then sit further right in the window),
// and the weights it does not use are zero.  The kernel then runs one window
// length for every output of an axis and never reads outside the image; the
// sums are those of the outputs' own taps, since the extra terms are zero.

// k of an axis (at least 1, at most n_in).
int axis_tap_count(int64_t n_in, int64_t n_out) {
    const AxisMap m(n_in, n_out);
    int64_t k = 1;
    for (int64_t i = 0; i < n_out; ++i) {
        int64_t lo, hi;
        double centre;
        m.window(i, lo, hi, centre);
        k = std::max(k, hi - lo);
    }
    return int(k);
}

int axis_dwords(int k) { return (k + 3) / 4; }
size_t axis_table_entries(int64_t n_out, int nd) { return size_t(n_out) * (1 + rec_dwords(nd)); }

// first[] of an axis table at tab (the cheap part: what the host's band and
// staging sizes need).  An axis of equal lengths is the identity: one tap.
void fill_axis_heads(int64_t n_in, int64_t n_out, int k, int32_t *tab) {
    if (n_in == n_out) {
        for (int64_t i = 0; i < n_out; ++i) tab[i] = int32_t(i);
        return;
    }
    const AxisMap m(n_in, n_out);
    for (int64_t i = 0; i < n_out; ++i) {
        int64_t lo, hi;
        double centre;
        m.window(i, lo, hi, centre);
        tab[i] = int32_t(std::min<int64_t>(lo, n_in - k));
    }
}

// One output's record from its k integer weights w (see rec_dwords), its
// constant less `offset`: false if a weight has no three-digit form (|w|
// beyond about 2^23, which normalised bicubic weights never reach).
bool fill_record(const int32_t *w, int k, int nd, int32_t offset, int32_t *rec) {
    int64_t sum = 0;
    uint32_t planes[3][64] = {};
    if (nd > 64) return false;
    for (int t = 0; t < k; ++t) {
        sum += w[t];
        int64_t v = w[t];
        for (int p = 0; p < 3; ++p) {
            const int64_t digit = ((v + 128) & 255) - 128;  // in [-128, 127]
            planes[p][t / 4] |= uint32_t(digit & 255) << (8 * (t % 4));
            v = (v - digit) / 256;
        }
        if (v != 0) return false;
    }
    rec[0] = int32_t((int64_t(1) << (kWeightBits - 1)) + 128 * sum - offset);
    for (int p = 0; p < 3; ++p)
        for (int q = 0; q < nd; ++q) rec[1 + p * nd + q] = int32_t(planes[p][q]);
    return true;
}

// The records of an axis table at tab (zeroed by the caller): the weights
// in float64 as PIL computes them, rounded half away from zero to
// kWeightBits, then split into digits.  A column table's constants are
// 128 << kWeightBits lower: the horizontal pass saturates its sums to signed
// bytes, which then come out as the PIL byte less 128, the vertical pass's
// input form.
bool fill_axis_records(int64_t n_in, int64_t n_out, int k, bool columns, int32_t *tab) {
    const int32_t offset = columns ? int32_t(128) << kWeightBits : 0;
    const int nd = axis_dwords(k);
    int32_t *recs = tab + n_out;
    std::vector<int32_t> wi(size_t(k), 0);
    if (n_in == n_out) {
        const int32_t one = 1 << kWeightBits;
        for (int64_t i = 0; i < n_out; ++i)
            if (!fill_record(&one, 1, nd, offset, recs + i * rec_dwords(nd))) return false;
        return true;
    }
    const AxisMap m(n_in, n_out);
    std::vector<double> w(size_t(k) + 1);
    for (int64_t i = 0; i < n_out; ++i) {
        int64_t lo, hi;
        double centre;
        m.window(i, lo, hi, centre);
        const int64_t cnt = hi - lo;
        double sum = 0.0;
        for (int64_t j = 0; j < cnt; ++j) {
            w[j] = keys_bicubic((double(j + lo) - centre + 0.5) / m.widen);
            sum += w[j];
        }
        std::fill(wi.begin(), wi.end(), 0);
        const int64_t shift = lo - tab[i];
        for (int64_t j = 0; j < cnt; ++j) {
            const double v = sum != 0.0 ? w[j] / sum : w[j];
            const double fixed = v * double(1 << kWeightBits);
            wi[shift + j] = int32_t(v < 0.0 ? fixed - 0.5 : fixed + 0.5);
        }
        if (!fill_record(wi.data(), k, nd, offset, recs + i * rec_dwords(nd))) return false;
    }
    return true;
}

struct HfTables {
    std::vector<uint8_t> head;    // items, tile prefix, lut
    std::vector<int32_t> taps;
    int64_t tiles = 0;
    int64_t rows = 0;
    int32_t band_bytes = 0, stage_bytes = 0;  // dynamic LDS the batch needs (see HfArgs)
    // every resized item's tiles read at most kMfmaSpan source columns and
    // band rows (one group per unit) with windows of at most kMfMaxNd
    // dwords: the matrix-core instance runs the batch
    bool mfma = true;
    size_t lds_bytes() const {
        if (mfma) return size_t(kMfLdsBytes);
        return size_t(kLutBytes) + kRecBytes + std::max<size_t>(kBlockBytes, size_t(band_bytes) + size_t(stage_bytes));
    }
};

// The most source rows one group of g output rows reads (the band the
// kernel forms: 4 nd rows past the group's last first row).
int band_rows(const int32_t *yfirst, int nd, int dst_h, int g) {
    int most = 0;
    for (int y0 = 0; y0 < dst_h; y0 += g) most = std::max(most, yfirst[y0 + g - 1] + 4 * nd - yfirst[y0]);
    return most;
}

// Output rows per vertical group so that the band of source rows one group
// needs fits kMaxBandRows: the largest of 32, 16, ..., 1 that fits everywhere.
int choose_group(const int32_t *yfirst, int nd, int dst_h) {
    for (int g = kUnitPx; g >= 1; g >>= 1)
        if (band_rows(yfirst, nd, dst_h, g) <= kMaxBandRows) return g;
    return 0;
}

int build_hf_tables(int32_t n, const mimo_image_desc *desc, const float *mean01,
                    const float *std01, HfTables &out) {
    out.head.assign(hf_items_bytes(n) + hf_prefix_bytes(n) + align256(kLutBytes), 0);
    HfItem *items = reinterpret_cast<HfItem *>(out.head.data());
    int64_t *tile_begin = reinterpret_cast<int64_t *>(out.head.data() + hf_items_bytes(n));
    float *lut = reinterpret_cast<float *>(out.head.data() + hf_items_bytes(n) + hf_prefix_bytes(n));
    // rescale as float32(float64(v) * (1 / 255)), then (x - mean) / std in float32
    const double rescale = 1.0 / 255.0;
    for (int c = 0; c < 3; ++c)
        for (int v = 0; v < 256; ++v) {
            const float x = float(double(v) * rescale);
            lut[c * 256 + v] = (x - mean01[c]) / std01[c];
        }
    int64_t tiles = 0, rows = 0;
    // One tap table per (input length, output length, axis) in the batch:
    // items of the same size share it (built and uploaded once).  Its first
    // entries are filled here; the records, the costly part, after the
    // loop, several tables at a time.
    std::map<std::tuple<int32_t, int32_t, bool>, std::pair<int64_t, int32_t>> tables;
    auto axis_table = [&](int32_t n_in, int32_t n_out, bool columns, int64_t &tab, int32_t &nd) {
        const auto key = std::make_tuple(n_in, n_out, columns);
        const auto it = tables.find(key);
        if (it == tables.end()) {
            const int k = n_in == n_out ? 1 : axis_tap_count(n_in, n_out);
            const int64_t at = int64_t(out.taps.size());
            out.taps.resize(out.taps.size() + axis_table_entries(n_out, axis_dwords(k)), 0);
            fill_axis_heads(n_in, n_out, k, out.taps.data() + at);
            tables.emplace(key, std::make_pair(at, k));
            tab = at;
            nd = axis_dwords(k);
        } else {
            tab = it->second.first;
            nd = axis_dwords(it->second.second);
        }
    };
    for (int32_t i = 0; i < n; ++i) {
        const mimo_image_desc &s = desc[i];
        HfItem d;
        std::memset(&d, 0, sizeof(d));
        d.x_tab = d.y_tab = -1;
        tile_begin[i] = tiles;
        d.src_offset = s.src_offset;
        d.row_offset = rows;
        d.blocks_w = 1;
        d.group = kUnitPx;
        if (s.status != MIMO_OK || s.rows == 0) {
            items[i] = d;
            continue;
        }
        if (s.src_h < 1 || s.src_w < 1 || (s.channels != 3 && s.channels != 4) || s.frames != 1 ||
            s.dst_h < kUnitPx || s.dst_w < kUnitPx || s.dst_h % kUnitPx || s.dst_w % kUnitPx ||
            s.grid_t != 1 || s.grid_h * kPatch != s.dst_h || s.grid_w * kPatch != s.dst_w ||
            s.rows != int64_t(s.grid_h) * s.grid_w || s.row_offset != rows || s.src_offset < 0)
            return set_error(MIMO_E_INVALID, "preprocess_hf: descriptor " + std::to_string(i) +
                                                 " is not a still-image plan of the 16/2/2 kernels");
        // the staging window addresses a band of source rows (and a few past
        // it) with 32-bit offsets
        if (s.src_h > kMaxSide || s.src_w > kMaxSide || s.dst_h > kMaxSide || s.dst_w > kMaxSide ||
            int64_t(s.src_w) * s.channels * (kMaxBandRows + 2) >= 0x7FFFFFF0ll)
            return set_error(MIMO_E_TOO_LARGE, "preprocess_hf: descriptor " + std::to_string(i) + ": side too large");
        d.src_h = s.src_h;
        d.src_w = s.src_w;
        d.channels = s.channels;
        d.blocks_h = s.dst_h / kUnitPx;
        d.blocks_w = s.dst_w / kUnitPx;
        out.mfma = out.mfma && s.dst_w <= kMfMaxSide && s.dst_h <= kMfMaxSide;
        if (s.dst_w != s.src_w || s.dst_h != s.src_h) {
            // both axes get a table (an axis that keeps its length: one tap of weight 1)
            axis_table(s.src_w, s.dst_w, true, d.x_tab, d.ndx);
            axis_table(s.src_h, s.dst_h, false, d.y_tab, d.ndy);
            const int32_t *xfirst = out.taps.data() + d.x_tab;
            const int32_t *yfirst = out.taps.data() + d.y_tab;
            d.group = choose_group(yfirst, d.ndy, s.dst_h);
            if (d.group == 0)
                return set_error(MIMO_E_UNSUPPORTED, "preprocess_hf: descriptor " + std::to_string(i) +
                                                         ": vertical downscale beyond the kernel's band");
            // the widest source block one tile's 32 output columns read
            int spitch = 0, xspan = 0;  // bytes per staged row and channel; source columns
            for (int32_t x0 = 0; x0 < s.dst_w; x0 += kUnitPx) {
                const int span = xfirst[x0 + kUnitPx - 1] + 4 * d.ndx - xfirst[x0];
                xspan = std::max(xspan, span);
                spitch = std::max(spitch, 4 * stage_pitch(span));
            }
            if (spitch > kMaxStagePitch)
                return set_error(MIMO_E_UNSUPPORTED, "preprocess_hf: descriptor " + std::to_string(i) +
                                                         ": horizontal downscale beyond the kernel's staging");
            const int nrows = band_rows(yfirst, d.ndy, s.dst_h, d.group);
            out.mfma = out.mfma && d.group == kUnitPx && xspan <= kMfmaSpan && nrows <= kMfmaSpan &&
                       d.ndx <= kMfMaxNd && d.ndy <= kMfMaxNd;
            out.band_bytes = std::max(out.band_bytes, 3 * kUnitPx * 4 * band_pitch(nrows));
            // a chunk of staged rows: all of them when that fits, else whole
            // quarters of kMaxStageBytes' worth (at least 4 rows)
            const int chunk = std::min((nrows + 3) & ~3, (kMaxStageBytes / (3 * spitch)) & ~3);
            out.stage_bytes = std::max(out.stage_bytes, 3 * chunk * spitch);
        }
        items[i] = d;
        tiles += int64_t(d.blocks_h) * d.blocks_w * (kUnitPx / d.group);
        rows += s.rows;
    }
    tile_begin[n] = tiles;
    out.tiles = tiles;
    out.rows = rows;
    if (out.taps.size() > size_t(0x7FFFFFFF))
        return set_error(MIMO_E_TOO_LARGE, "preprocess_hf: tap tables above 2^31 entries");
    // the records: tables are independent, so large batches of them are
    // shared out over up to 16 host threads
    struct Job {
        int32_t n_in, n_out, k;
        bool columns;
        int64_t tab;
    };
    std::vector<Job> jobs;
    int64_t work = 0;
    for (const auto &t : tables) {
        jobs.push_back({std::get<0>(t.first), std::get<1>(t.first), t.second.second, std::get<2>(t.first),
                        t.second.first});
        work += int64_t(std::get<1>(t.first)) * t.second.second;
    }
    std::atomic<bool> ok{true};
    auto run = [&](size_t from, size_t step) {
        for (size_t j = from; j < jobs.size(); j += step)
            if (!fill_axis_records(jobs[j].n_in, jobs[j].n_out, jobs[j].k, jobs[j].columns,
                                   out.taps.data() + jobs[j].tab))
                ok.store(false);
    };
    const size_t threads =
        std::min<size_t>({size_t(16), jobs.size(), size_t(std::max(1u, std::thread::hardware_concurrency()))});
    if (threads < 2 || work < kParallelTapWork) {
        run(0, 1);
    } else {
        std::vector<std::thread> pool;
        for (size_t t = 1; t < threads; ++t) pool.emplace_back(run, t, threads);
        run(0, threads);
        for (auto &th : pool) th.join();
    }
    if (!ok.load()) return set_error(MIMO_E_UNSUPPORTED, "preprocess_hf: a resampling weight out of range");
    out.taps.resize(out.taps.size() + kTapsTail, 0);
    return MIMO_OK;
}

// Room for one HfTile per merge unit (the matrix-core instance's tiles).
size_t hf_tiles_bytes(int32_t n, const mimo_image_desc *desc) {
    size_t units = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mimo_image_desc &s = desc[i];
        if (s.status != MIMO_OK || s.rows == 0 || s.dst_w < 1 || s.dst_h < 1) continue;
        units += size_t(s.dst_h / kUnitPx) * size_t(s.dst_w / kUnitPx);
    }
    return align256(units * sizeof(HfTile));
}

}  // namespace
}  // namespace mimo

using namespace mimo;

extern "C" {

int64_t mimo_hf_matrix_dispatch_count(void) { return g_hf_matrix_dispatches.load(); }

size_t mimo_hf_workspace_bytes(int32_t n, const mimo_image_desc *desc) {
    if (n < 0 || (n > 0 && !desc)) return 0;
    size_t entries = 0;
    for (int32_t i = 0; i < n; ++i) {
        const mimo_image_desc &s = desc[i];
        if (s.status != MIMO_OK || s.rows == 0 || s.dst_w < 1 || s.dst_h < 1) continue;
        if (s.dst_w == s.src_w && s.dst_h == s.src_h) continue;
        // at most: each axis its own table, k bounded by the support
        const int kx = s.dst_w != s.src_w ? axis_taps_per_output(s.src_w, s.dst_w) : 1;
        const int ky = s.dst_h != s.src_h ? axis_taps_per_output(s.src_h, s.dst_h) : 1;
        entries += axis_table_entries(s.dst_w, axis_dwords(kx)) + axis_table_entries(s.dst_h, axis_dwords(ky));
    }
    return hf_items_bytes(n) + hf_prefix_bytes(n) + align256(kLutBytes) +
           align256((entries + kTapsTail) * sizeof(int32_t)) + hf_tiles_bytes(n, desc);
}

int mimo_preprocess_hf_batch(int32_t n, const mimo_image_desc *desc, const uint8_t *src,
                             int64_t src_capacity, const float *mean01, const float *std01,
                             int32_t out_dtype, void *rows, void *rows_col, int64_t capacity_rows,
                             void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    if (n < 0 || (n > 0 && !desc) || !mean01 || !std01)
        return set_error(MIMO_E_INVALID, "preprocess_hf: bad n or null pointer");
    if (out_dtype != MIMO_F32 && out_dtype != MIMO_BF16)
        return set_error(MIMO_E_INVALID, "preprocess_hf: out_dtype must be MIMO_F32 or MIMO_BF16");
    if (!rows && !rows_col)
        return set_error(MIMO_E_INVALID, "preprocess_hf: both outputs are null");
    if ((rows && !check_ptr_align(rows, 16)) || (rows_col && !check_ptr_align(rows_col, 16)))
        return set_error(MIMO_E_INVALID, "preprocess_hf: outputs must be 16-byte aligned");
    for (int c = 0; c < 3; ++c)
        if (!(std01[c] > 0.0f) || !std::isfinite(std01[c]) || !std::isfinite(mean01[c]))
            return set_error(MIMO_E_INVALID, "preprocess_hf: std01 must be > 0 and finite");
    if (n == 0) return MIMO_OK;
    if (!src) return set_error(MIMO_E_INVALID, "preprocess_hf: null src");
    if (!workspace || !check_ptr_align(workspace, 16))
        return set_error(MIMO_E_INVALID, "preprocess_hf: workspace must be non-null and 16-byte aligned");
    HfTables t;
    int st = build_hf_tables(n, desc, mean01, std01, t);
    if (st != MIMO_OK) return st;
    const size_t taps_bytes = align256(std::max<size_t>(t.taps.size(), 1) * sizeof(int32_t));
    const size_t need = t.head.size() + taps_bytes + (t.mfma ? align256(size_t(t.tiles) * sizeof(HfTile)) : 0);
    if (workspace_bytes < need)
        return set_error(MIMO_E_CAPACITY, "preprocess_hf: workspace smaller than mimo_hf_workspace_bytes(n, desc)");
    int64_t src_needed = 0;
    for (int32_t i = 0; i < n; ++i)
        if (desc[i].status == MIMO_OK && desc[i].rows > 0)
            src_needed = std::max<int64_t>(src_needed, desc[i].src_offset + int64_t(desc[i].src_h) *
                                                                                 desc[i].src_w * desc[i].channels);
    if (src_capacity < src_needed)
        return set_error(MIMO_E_CAPACITY, "preprocess_hf: src_capacity below the packed size");
    if (t.rows > capacity_rows)
        return set_error(MIMO_E_CAPACITY, "preprocess_hf: capacity_rows below the plan's total rows");
    if (t.tiles == 0) return MIMO_OK;
    if (t.tiles > 0x7FFFFFFFll)
        return set_error(MIMO_E_TOO_LARGE, "preprocess_hf: more than 2^31 - 1 tiles");
    if (t.taps.size() > size_t(0x7FFFFFF0 / sizeof(int32_t)))
        return set_error(MIMO_E_TOO_LARGE, "preprocess_hf: resampling tables beyond 2 GiB");

    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    hipError_t e = upload_table(t.head.data(), t.head.size(), ws, s);
    if (e == hipSuccess && !t.taps.empty())
        e = upload_table(t.taps.data(), t.taps.size() * sizeof(int32_t), ws + t.head.size(), s);
    if (e != hipSuccess) return hip_error(e, "preprocess_hf: table upload");
    HfArgs a;
    a.src = src;
    a.src_end = src_capacity;
    a.items = reinterpret_cast<const HfItem *>(ws);
    a.tile_begin = reinterpret_cast<const int64_t *>(ws + hf_items_bytes(n));
    a.lut = reinterpret_cast<const float *>(ws + hf_items_bytes(n) + hf_prefix_bytes(n));
    a.taps = reinterpret_cast<const int32_t *>(ws + t.head.size());
    a.rows = rows;
    a.rows_col = rows_col;
    a.n = n;
    a.band_bytes = t.band_bytes;
    a.stage_bytes = t.stage_bytes;
    a.tiles = t.mfma ? reinterpret_cast<HfTile *>(ws + t.head.size() + taps_bytes) : nullptr;
    a.n_tiles = t.tiles;
    a.taps_bytes = int32_t(t.taps.size() * sizeof(int32_t));
    const size_t lds = t.lds_bytes();
    const bool f32 = out_dtype == MIMO_F32;
    const void *kernel =
        t.mfma ? (f32 ? reinterpret_cast<const void *>(hf_preprocess_kernel<float, true>)
                      : reinterpret_cast<const void *>(hf_preprocess_kernel<uint16_t, true>))
               : (f32 ? reinterpret_cast<const void *>(hf_preprocess_kernel<float, false>)
                      : reinterpret_cast<const void *>(hf_preprocess_kernel<uint16_t, false>));
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return hip_error(e, "preprocess_hf: LDS size");
    const dim3 grid{unsigned(t.tiles), 1, 1};
    const dim3 block{unsigned(kHfThreads), 1, 1};
    const dim3 tgrid{unsigned((t.tiles + 255) / 256), 1, 1};
    e = timed_launch(s, [&] {
        if (t.mfma) hipLaunchKernelGGL(hf_tiles_kernel, tgrid, dim3(256), 0, s, a);
        if (t.mfma && f32)
            hipLaunchKernelGGL((hf_preprocess_kernel<float, true>), grid, block, lds, s, a);
        else if (t.mfma)
            hipLaunchKernelGGL((hf_preprocess_kernel<uint16_t, true>), grid, block, lds, s, a);
        else if (f32)
            hipLaunchKernelGGL((hf_preprocess_kernel<float, false>), grid, block, lds, s, a);
        else
            hipLaunchKernelGGL((hf_preprocess_kernel<uint16_t, false>), grid, block, lds, s, a);
    });
    if (e != hipSuccess) return hip_error(e, "preprocess_hf: kernel launch");
    g_dispatches.fetch_add(1);
    if (t.mfma) g_hf_matrix_dispatches.fetch_add(1);
    return MIMO_OK;
}

}  // extern "C"
