// C ABI of libmi_resize.so: argument checks, kernel selection, launch.
// The contract (layout, ownership, errors, limits) is in include/mi_resize.h.
#include "mi_resize.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "resize_kernels.hpp"

namespace {

using namespace mirsz;

constexpr int kMaxDim = 65535;
constexpr long long kMaxOutPixels = 1LL << 40;
// Workgroups a launch aims for: 8 per CU on 256 CUs keeps every SIMD busy
// with several waves while each lane still amortises its column taps over a
// band of rows.
constexpr long long kTargetBlocks = 2048;
// Cap for grid-stride kernels, keeping every launch far below the 2^32
// work-items a grid dimension can hold.
constexpr long long kMaxStrideBlocks = 65536;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Kernel family override for testing: MI_RESIZE_PATH=rowseg skips the
// scale-specific fast paths, MI_RESIZE_PATH=direct uses only the
// direct-gather kernels.  Unset (or anything else): automatic choice.
enum class Path { Auto, RowSeg, Direct, Tile };

Path path_override()
{
    const char *v = getenv("MI_RESIZE_PATH");
    if (!v) return Path::Auto;
    if (strcmp(v, "rowseg") == 0) return Path::RowSeg;
    if (strcmp(v, "direct") == 0) return Path::Direct;
    if (strcmp(v, "tile") == 0) return Path::Tile;
    return Path::Auto;
}

// dC: channels of dst (C unless the output stage changes them); dst_es:
// bytes per dst element (that of the dtype unless the output stage changes
// the element type, as the normalising stage does)
int check_args(const void *src, const void *dst, int batch, int H, int W, int C, int dtype,
               int dH, int dW, int dC = 0, size_t dst_es = 0)
{
    if (dC == 0) dC = C;
    if (!src || !dst) return MI_RESIZE_ERR_NULL;
    if (dtype != MI_RESIZE_U8 && dtype != MI_RESIZE_F32) return MI_RESIZE_ERR_DTYPE;
    if (C != 1 && C != 3 && C != 4) return MI_RESIZE_ERR_CHANNELS;
    if (batch < 1 || H < 1 || W < 1 || dH < 1 || dW < 1) return MI_RESIZE_ERR_SHAPE;
    if (H > kMaxDim || W > kMaxDim || dH > kMaxDim || dW > kMaxDim) return MI_RESIZE_ERR_SHAPE;
    if ((long long)batch * dH * dW > kMaxOutPixels) return MI_RESIZE_ERR_SHAPE;
    if ((long long)batch * H * W > kMaxOutPixels) return MI_RESIZE_ERR_SHAPE;
    const size_t es = dtype == MI_RESIZE_U8 ? 1 : 4;
    if (dst_es == 0) dst_es = es;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    const uintptr_t s1 = s0 + (size_t)batch * H * W * C * es;
    const uintptr_t d1 = d0 + (size_t)batch * dH * dW * dC * dst_es;
    if (s0 < d1 && d0 < s1) return MI_RESIZE_ERR_OVERLAP;
    if ((es == 4 && !aligned(src, 4)) || (dst_es == 4 && !aligned(dst, 4)))
        return MI_RESIZE_ERR_ALIGN;
    return MI_RESIZE_OK;
}

struct Grid {
    unsigned blocks;
    int rows_per_block;
    BandGrid bg;
};

// m and s of FastDiv for a divisor d in [1, 2^31]
FastDiv fast_div_for(long long d)
{
    unsigned s = 0;
    while ((1LL << s) < d) ++s;
    const unsigned long long m = ((1ULL << (31 + s)) + (unsigned long long)d - 1) / (unsigned long long)d;
    return FastDiv{(unsigned)m, s};
}

// Row-band grid shared by the generic kernels (about kTargetBlocks
// workgroups, so every workgroup index stays far below 2^31).
Grid band_grid(long long rows_total, int dW, int dH)
{
    Grid g;
    g.bg.col_blocks = (dW + kBlock - 1) / kBlock;
    long long per_row = g.bg.col_blocks;
    long long rpb = (rows_total * per_row + kTargetBlocks - 1) / kTargetBlocks;
    if (rpb < 1) rpb = 1;
    g.rows_per_block = (int)rpb;
    g.blocks = (unsigned)(((rows_total + rpb - 1) / rpb) * per_row);
    g.bg.by_cols = fast_div_for(g.bg.col_blocks);
    g.bg.by_dst_h = fast_div_for(dH);
    return g;
}

// Launch `kernel` through hipLaunchKernel, which returns this launch's own
// status (an earlier error elsewhere on the thread cannot leak into it).  The
// arguments are converted to the kernel's exact parameter types before their
// addresses are handed over.
template <typename T> struct same { using type = T; };

template <typename... P>
int launch(void (*kernel)(P...), dim3 grid, dim3 block, unsigned lds_bytes, hipStream_t st,
           typename same<P>::type... args)
{
    void *argv[] = {(void *)&args..., nullptr};
    const hipError_t e = hipLaunchKernel((const void *)kernel, grid, block, argv, lds_bytes, st);
    return e == hipSuccess ? MI_RESIZE_OK : MI_RESIZE_ERR_HIP;
}

// Float RGB (12-byte pixels) on the direct kernels goes out through LDS as
// whole-line 16-byte stores where output rows are 16-byte aligned (1080p ->
// 2x on the direct kernels: linear 45.3 -> 28.5 us, nearest 32.3 -> 23.0).
constexpr bool kDirectStageRgb = true;

template <typename T, int C, int OUT = kOutSame, bool ROI = false>
int launch_linear_generic(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                          hipStream_t st, const Affine &aff = Affine{},
                          const int32_t *rois = nullptr)
{
    const long long rows = (long long)batch * dH;
    const Grid g = band_grid(rows, dW, dH);
    const bool pix4 = OUT == kOutSame && C == 4 && aligned(src, 4 * sizeof(T)) &&
                      aligned(dst, 4 * sizeof(T));
    auto go = [&](auto kernel) {
        return launch(kernel, dim3(g.blocks), dim3(kBlock), 0, st, (const T *)src, dst, H, W, dH,
                      dW, rows, g.rows_per_block, g.bg, aff, rois);
    };
    if (pix4) return go(linear_generic<T, C, C == 4 && OUT == kOutSame, OUT, ROI>);
    if constexpr (sizeof(T) == 4 && C == 3 && OUT == kOutSame && !ROI) {
        // float RGB rows that start on 16-byte boundaries: staged stores
        if (kDirectStageRgb && dW % 4 == 0 && aligned(dst, 16))
            return go(linear_generic<T, C, false, OUT, ROI, kBorderClamp, true>);
    }
    return go(linear_generic<T, C, false, OUT, ROI>);
}

constexpr long long kMaxGridY = 65535;
// x extents stay well inside HIP's limit of 2^32 threads per dimension
constexpr long long kMaxGridX = 1LL << 24;
// workgroups of a grid whose kernel renumbers them (xcd_contiguous, div_by)
constexpr long long kMaxGroups = 0x7fffffffLL;

template <int C, bool GREY = false>
int launch_half_u8(const void *src, void *dst, int batch, int dH, int dW, hipStream_t st)
{
    constexpr int seg = kHalfLanes * HalfShape<C>::PX;
    const long long rows = (long long)batch * dH;
    const long long segs = (dW + seg - 1) / seg;
    // one or two segments per row: rows along x (see the kernel)
    if (segs <= 2) {
        const dim3 grid((unsigned)(rows < kMaxGridX ? rows : kMaxGridX), (unsigned)segs);
        return launch(linear_half_u8<C, GREY, true>, grid, dim3(kHalfLanes), 0, st,
                      (const uint8_t *)src, (uint8_t *)dst, dW, rows, DivBy{}, (int)segs,
                      rows);
    }
    // a pass covers at most 65535 rows (the row loop is then exercised by
    // batches of realistic size) and its items stay below 2^31 for the
    // kernel's divide by segs
    long long pass = rows < kMaxGridY ? rows : kMaxGridY;
    if (segs * pass > kMaxGroups) pass = kMaxGroups / segs;
    const long long wgs = (segs * pass + kHalfWaves - 1) / kHalfWaves;
    return launch(linear_half_u8<C, GREY, false>, dim3((unsigned)wgs),
                  dim3(kHalfLanes * kHalfWaves), 0, st, (const uint8_t *)src, (uint8_t *)dst,
                  dW, rows, make_div_by((unsigned)segs), (int)segs, pass);
}

// Exact 2:1 uint8 downscale whose rows split into whole 16-byte chunks and
// whole lanes.
bool half_path_fits(int C, int H, int W, int dH, int dW, const void *src, const void *dst)
{
    if (H != 2 * dH || W != 2 * dW || !aligned(src, 16) || !aligned(dst, 16)) return false;
    const int q = C == 1 ? 16 : (C == 3 ? 8 : 4);
    return dW % q == 0;
}

// LDS bytes one row-segment wave may use (its two slots).  Beyond it the
// segment is too wide (strong downscale) and the direct kernels run instead;
// a workgroup of kSegWaves such waves then takes 64 KiB, and a slot of at
// most 8 KiB is at most 8 16-byte chunks per lane.
constexpr int kSegLdsBudget = 16 * 1024;
// Row bands (one wave each) a row-segment launch aims for: 256 per CU on
// 256 CUs, but at least kSegMinBandRows rows each.  Short bands keep many
// independent waves in flight and balance the tail; a band's set-up (its
// column table and row map) is paid once per band, so single-row bands
// cost more than they gain where the output is narrow.
constexpr long long kSegTargetBands = 65536;
// Multi-byte outputs keep two-row bands: three or four measured slower on
// most shapes (64 x 640x480 -> 112x112 RGB 9.5 -> 10.2 / 10.6 us, float
// 16 x 640x480 -> 224x224 RGBA 17.1 -> 18.6 / 18.5, thumbnail nearest 27.2
// -> 28.4 / 28.7), faster on a few (8 x 1080p -> 720p RGB 23.1 -> 21.8 /
// 21.6, thumbnail linear 47.1 -> 46.7 / 49.3), with no row-segment count
// separating the two.
constexpr long long kSegMinBandRows = 2;
// Where each output pixel is a single byte (grey output, one-channel uint8),
// a row moves little and the per-band set-up weighs more, so bands are
// longer - but only as long as enough of them remain to fill the chip.  By
// row segments (output rows x wave segments per row): below 9000, two-row
// bands; below 30000, three; else four.  Measured (us, one-channel linear;
// bands of 2 / 3 / 4 rows): 4K -> 1000x1900 (4000 segments) 7.3 / 8.8 /
// 8.6; 64 x 640x480 -> 112x112 (7168) 8.0 / 8.6 / 8.5; 32 x 720p ->
// 360x500 (11520) 13.0 / 12.7 / 13.0; 8 x 1080p -> 720p (17280) 16.3 /
// 14.8 / 14.9; 256 x 640x480 -> 224x224 (57344) 36.2 / 32.5 / 30.5.
inline long long seg_min_rows_narrow(long long rows, int dW, int px)
{
    const long long cols = (long long)kSegLanes * px;
    const long long segs = rows * ((dW + cols - 1) / cols);
    return segs < 9000 ? 2 : (segs < 30000 ? 3 : 4);
}
// Normalised float output writes four bytes per channel, and there
// single-row bands (more waves, each with its stores in flight sooner)
// measured faster once the band set-up stopped dividing in fp64: the
// 256 x 480x640 -> 224x224 batch NCHW 63.3 -> 60.7 us, NHWC 63.0 -> 61.4;
// 1080p -> 720p, 4 x 720p -> 1080p and 8 x 224^2 -> 256^2 unchanged.
constexpr long long kSegMinBandRowsNorm = 1;
// A crop-then-resize band first reads its image's region from device memory
// before it can map a row, so its bands are made longer to amortise that
// round trip (random crops of the thumbnail batch: 2 rows 44.9 us, 4 rows
// 40.3 us, 8 rows 43.6 us).
constexpr long long kSegMinBandRowsRoi = 4;
// Enlargements (more output pixels than source pixels) amortise a band's set-up
// and its staged boundary row over more output rows, down to about 5000
// bands, within 3..6 rows (us, two-row bands -> this rule: 720p -> 1080p RGB
// 9.8 -> 9.4; 1080p -> 1620x2880 RGB 16.3 -> 14.7, RGBA 17.4 -> 16.0;
// 8x300x400 -> 1000x1200 RGB 29.3 -> 24.5; 2000^2 -> 3000^2 float 22.1 ->
// 17.5; fewer bands than this left too few waves, more rows were slower).
// Retested once wide enlargements took 8 pixels per lane (half the segments
// per row): 2500 / 5000 / 10000 bands, 1080p -> 2000x3000 RGB 17.3 / 14.9 /
// 15.0 us, 8 x 480x640 -> 720x1000 RGB 17.3 / 14.9 / 15.0, 4K grey ->
// 3000x5000 19.6 / 19.6 / 21.4.
constexpr long long kSegTargetBandsUp = 5000;
constexpr long long kSegMinBandRowsUp = 3;
constexpr long long kSegMaxBandRowsUp = 6;
// Below 2^19 output pixels from at most 2^20 source pixels the launch is
// latency-bound and the direct kernels (no staging round trip, no per-lane
// column table of PX entries, one row per workgroup) finish first:
// 4 x 100x100 RGB -> 150x150 6.0 -> 3.4 us, 1x240x320 grey -> 400x530
// 5.5 -> 3.7, 32 x 128x128 RGBA -> 100x100 6.2 -> 5.4.  Larger outputs
// stay on the row-segment kernel (720x960 from 480x640 RGB 5.8 us there,
// 6.6 direct), and so do downscales of large sources, which its staged rows
// serve better (1080p RGB -> 540x800 6.6 vs 6.8).
constexpr long long kSmallOutPixels = 1LL << 19;
constexpr long long kSmallSrcPixels = 1LL << 20;

bool small_launch(int batch, int H, int W, int dH, int dW)
{
    return (long long)batch * dH * dW < kSmallOutPixels && (long long)batch * H * W < kSmallSrcPixels;
}

// Float RGB / RGBA enlarged along rows of the output (dW > W), linear or
// nearest: every output pixel is 12 or 16 bytes, the output outweighs the
// source, and the direct kernel's whole-line stores and cached gathers beat
// staging (1080p RGBA 2x: linear 29.8 vs 62.3 us, nearest 26.4 vs 41.8;
// RGB 2x: 28.4 vs 70.0, 23.0 vs 87.1).  Single-channel floats and all
// uint8 cases stay on the row-segment kernel.
template <typename T, int C>
bool prefer_direct(int W, int dW)
{
    return sizeof(T) == 4 && C >= 3 && dW > W;
}

struct SegPlan {
    dim3 grid;
    int rows_per_block;
    int seg_cap;
};

// Bytes per LDS slot for the widest segment: the source columns touched by
// kernel-side output columns wx0..wx1 span at most (wx1 - wx0) * W / dW + 3
// columns (taps on both sides plus rounding), plus 15 bytes of misalignment
// and the slack a two-tap read may run past the last staged pixel.
bool plan_rowseg(int px, int pixel_bytes, int W, int dW, long long rows, long long min_rows,
                 bool enlarge, SegPlan &pl)
{
    const long long cols = (long long)kSegLanes * px;
    long long span = ((cols - 1) * W) / dW + 3;
    if (span > W) span = W;
    const long long cap = ((span * pixel_bytes + 15 + kSegReadSlack + 15) / 16) * 16;
    if (2 * cap > kSegLdsBudget) return false;
    pl.seg_cap = (int)cap;
    const long long gx = (dW + cols - 1) / cols;
    long long rpb = (rows * gx + kSegTargetBands - 1) / kSegTargetBands;
    if (enlarge) {
        // about kSegTargetBandsUp bands of kSegMinBandRowsUp..kSegMaxBandRowsUp rows
        long long up = (rows * gx + kSegTargetBandsUp - 1) / kSegTargetBandsUp;
        up = up < kSegMinBandRowsUp ? kSegMinBandRowsUp : (up > kSegMaxBandRowsUp ? kSegMaxBandRowsUp : up);
        if (rpb < up) rpb = up;
    }
    if (rpb < min_rows) rpb = min_rows;
    // but keep at least ~2048 bands (two waves per SIMD) where the rows
    // allow: few rows in long bands leave most of the chip idle while each
    // wave walks its rows (8 x 224x224 -> 256x256 RGB 5.9 -> 4.8 us,
    // 1080p RGB -> 540x800 6.6 -> 6.1; a 4096-band floor lost elsewhere,
    // 4K RGB -> 1440x2560 11.9 -> 14.6)
    const long long par = rows * gx / 2048;
    if (rpb > par) rpb = par < 1 ? 1 : par;
    pl.rows_per_block = (int)rpb;
    const long long bands = (rows + rpb - 1) / rpb;
    pl.grid = dim3((unsigned)gx, (unsigned)((bands + kSegWaves - 1) / kSegWaves));
    return true;
}

template <typename T, int C, bool NEAREST, int OUT = kOutSame, bool ROI = false,
          int B = kBorderClamp, int PXO = 0>
bool try_rowseg_px(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                hipStream_t st, int &rc, const Affine &aff = Affine{},
                const int32_t *rois = nullptr, int nn_map = kNearestHalfPixel)
{
    const long long rows = (long long)batch * dH;
    SegPlan pl;
    // a crop is at most W wide, so the whole-image bound covers every crop
    constexpr int out_px_bytes =
        OUT == kOutGrey ? (int)sizeof(T) : (OUT == kOutSame ? C * (int)sizeof(T) : 4 * C);
    constexpr int PX = PXO ? PXO : SegShape<T, C>::PX;
    const long long min_rows = ROI ? kSegMinBandRowsRoi
                               : (OUT == kOutNormNCHW || OUT == kOutNormNHWC) ? kSegMinBandRowsNorm
                               : (out_px_bytes == 1 ? seg_min_rows_narrow(rows, dW, PX)
                                                    : kSegMinBandRows);
    // the output outweighs the source (pixel counts: rgbaf enlarges its
    // rows but halves its columns and is bandwidth-bound, 154.5 us with
    // five-row bands, 161.4 with six); crops are sized against their own
    // regions, so only whole images count
    const bool enlarge = !ROI && (long long)dH * dW > (long long)H * W;
    if (!plan_rowseg(PX, C * (int)sizeof(T), W, dW, rows, min_rows, enlarge, pl))
        return false;
    // chunks of 16 bytes per lane per staged row, rounded up to 1, 2, 4 or 8;
    // a slot then holds 64 lanes x that many chunks (the kernel writes its
    // clamped spare chunks there instead of branching around them)
    const int need = (pl.seg_cap / 16 + kSegLanes - 1) / kSegLanes;
    const int per_lane = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
    pl.seg_cap = per_lane * kSegLanes * 16;
    // wrap adds 16 bytes in front of each slot and 16 behind it for the
    // one-pixel halo around a staged row
    const int slot_bytes = pl.seg_cap + (B == kBorderWrap ? 32 : 0);
    if (2 * slot_bytes > kSegLdsBudget) return false;
    auto go = [&](auto kernel) {
        constexpr int nstage = seg_nhwc_stage_bytes<T, C, OUT, PX>();
        // at most 4 x (16 KiB of slots + 4 KiB of output staging) = 80 KiB,
        // within the 160 KiB one gfx950 workgroup may use
        static_assert(kSegWaves * (kSegLdsBudget + nstage) <= 160 * 1024, "LDS per workgroup");
        // plus the segment's column table where the kernel builds one in LDS
        constexpr int table_bytes = !ROI && PX >= 4 ? kSegLanes * PX * (sizeof(T) == 1 ? 4 : 8) : 0;
        static_assert(kSegWaves * (kSegLdsBudget + nstage) + table_bytes <= 160 * 1024,
                      "LDS per workgroup with the column table");
        const int lds_bytes = kSegWaves * (2 * slot_bytes +
                                           (nstage > 0 && seg_nhwc_staged(dst, dW, C) ? nstage : 0)) +
                              table_bytes;
        return launch(kernel, pl.grid, dim3(kSegLanes * kSegWaves), lds_bytes, st,
                      (const T *)src, dst,
                      H, W, dH, dW, rows, pl.rows_per_block, pl.seg_cap,
                      (long long)batch * H * W * C, aff, rois, nn_map);
    };
    // Non-temporal staging loads when no source row is used by two output
    // rows (a row step of at least 2 for linear, 1 for nearest): nothing
    // staged is read again, so the loads need not allocate in the caches.
    // Where rows are shared, a neighbouring band re-reads its boundary rows
    // from L2, and crops can upscale, so those keep cached loads.
    const bool stream = NEAREST ? H >= dH : H >= 2 * dH;
    auto pick = [&](auto nt) {
        constexpr bool NT = decltype(nt)::value;
        if (per_lane <= 1) return go(rowseg<T, C, NEAREST, 1, NT, OUT, ROI, B, PXO>);
        if (per_lane <= 2) return go(rowseg<T, C, NEAREST, 2, NT, OUT, ROI, B, PXO>);
        if (per_lane <= 4) return go(rowseg<T, C, NEAREST, 4, NT, OUT, ROI, B, PXO>);
        return go(rowseg<T, C, NEAREST, 8, NT, OUT, ROI, B, PXO>);
    };
    if constexpr (!ROI && B == kBorderClamp) {
        if (stream) {
            rc = pick(std::true_type{});
            return true;
        }
    }
    rc = pick(std::false_type{});
    return true;
}

// Output pixels per lane of a one-channel uint8 row segment (a wave covers
// 64 PX columns): the largest of 16 (nearest only), 8 and 4 whose segments
// are at least 80% filled by the row, else the best-filled one.  More
// pixels per lane spread each lane's set-up over more output, while lanes
// past the row's end idle.  Measured (us, linear / nearest; PX 16, 8, 4):
// 256 x 640x480 -> 224x224 57.7 / 25.7, 38.5 / 23.1, 33.1 / 21.1;
// 4K -> 1440x2560 11.2 / 6.8, 9.7 / 7.2, 10.8 / 8.3; 32 x 720p -> 360x500
// 19.1 / 9.8, 13.1 / 9.0, 16.7 / 11.5; 8K -> 1000x700 12.8 / 7.5,
// 9.4 / 6.6, 7.9 / 6.2; 8 x 1080p -> 720p 16.7 / 9.3, 15.0 / 9.9,
// 18.2 / 12.6 (the one miss: nearest takes 8 there).
inline int seg_px_u8_c1(int dW, bool nearest)
{
    int best = 4;
    long long best_num = 0, best_den = 1;   // best fill so far, as a fraction
    for (int px = nearest ? 16 : 8; px >= 4; px /= 2) {
        const long long cols = (long long)kSegLanes * px;
        const long long span = ((dW + cols - 1) / cols) * cols;
        if (5LL * dW >= 4LL * span) return px;   // fill >= 80%
        if ((long long)dW * best_den > best_num * span) {
            best = px;
            best_num = dW;
            best_den = span;
        }
    }
    return best;
}

// 8 output pixels per lane instead of 4 for uint8 RGB / RGBA, one-channel
// float and (nearest only) float RGB, plain output only: where the row fills its 512-column
// segments (uint8 to 95%, float to 80%) and shrinks by at most 1.6 (linear)
// or not at all (uint8 nearest), more pixels per lane spread each lane's
// set-up.  Stronger shrinking stages more source per lane and halves the
// waves, which costs more.  Measured (us, PX 4 -> 8): 4K -> 1440x2560 RGB
// linear 13.7 -> 12.0, RGBA 15.1 -> 13.5 (nearest RGB 11.7 -> 11.0 but
// RGBA 9.7 -> 10.3, so not taken); 1080p -> 2000x3000 RGB 17.3 -> 15.4 /
// 13.1 -> 11.8, RGBA 18.8 -> 17.7 / 10.1 -> 9.6; one-channel float 4K ->
// 1440x2560 linear 11.2 -> 10.0, 8 x 1080p -> 720p 18.6 -> 17.8 (nearest
// slower: 9.6 -> 10.5).  Not taken where they lost: 32 x 720p -> 360x500
// RGB (fills 98%, shrinks 2.56) 21.5 -> 23.5, 8 x 1080p -> 720p RGBA
// (fills 83%) 24.1 -> 25.3.
template <typename T, int C>
bool seg_wide_px8(int W, int dW, bool nearest)
{
    const long long span = ((dW + 511) / 512) * 512;
    // Float RGB: nearest only, on rows filled to 80% that shrink by at most
    // 2.1 (4K -> 1000x1900 15.3 -> 12.8 us, 4K -> 1440x2560 22.2 -> 19.8,
    // 8 x 1080p -> 720p 39.7 -> 36.5; 8K -> 2000x3000, shrinking 2.56,
    // 45.7 -> 57.0; linear slower on most shapes: 4K -> 1440x2560 28.9 ->
    // 30.6).
    if constexpr (sizeof(T) == 4 && C == 3)
        return nearest && 5LL * dW >= 4LL * span && 10LL * W <= 21LL * dW;
    const bool filled = sizeof(T) == 1 ? 20LL * dW >= 19LL * span : 5LL * dW >= 4LL * span;
    if (!filled) return false;
    // uint8 nearest: RGB on rows shrinking by at most 1.6 (4K -> 1440x2560
    // 9.49 -> 8.67 us, 4 x 1080p -> 864x1536 11.71 -> 10.20, 2 x 2560x1600
    // -> 2048x1280 11.37 -> 9.80), RGBA only where the row does not shrink
    // (the same three 9.44 -> 10.06, 11.77 -> 12.12, 11.51 -> 11.72)
    if (nearest) return sizeof(T) == 1 && (C == 3 ? 5LL * W <= 8LL * dW : W <= dW);
    return 5LL * W <= 8LL * dW;
}

template <typename T, int C, bool NEAREST, int OUT = kOutSame, bool ROI = false,
          int B = kBorderClamp>
bool try_rowseg(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                hipStream_t st, int &rc, const Affine &aff = Affine{},
                const int32_t *rois = nullptr, int nn_map = kNearestHalfPixel)
{
    if constexpr (sizeof(T) == 1 && C == 1) {
        switch (seg_px_u8_c1(dW, NEAREST)) {
        case 16:
            if constexpr (NEAREST)
                return try_rowseg_px<T, C, NEAREST, OUT, ROI, B, 16>(src, dst, batch, H, W, dH,
                                                                     dW, st, rc, aff, rois, nn_map);
            break;
        case 8:
            return try_rowseg_px<T, C, NEAREST, OUT, ROI, B, 8>(src, dst, batch, H, W, dH, dW, st,
                                                                rc, aff, rois, nn_map);
        default:
            break;
        }
        return try_rowseg_px<T, C, NEAREST, OUT, ROI, B, 4>(src, dst, batch, H, W, dH, dW, st,
                                                            rc, aff, rois, nn_map);
    } else {
        if constexpr (((sizeof(T) == 1 && C >= 3) || (sizeof(T) == 4 && C != 4)) &&
                      OUT == kOutSame && !ROI && B == kBorderClamp) {
            if (seg_wide_px8<T, C>(W, dW, NEAREST))
                return try_rowseg_px<T, C, NEAREST, OUT, ROI, B, 8>(src, dst, batch, H, W, dH, dW,
                                                                    st, rc, aff, rois, nn_map);
        }
        return try_rowseg_px<T, C, NEAREST, OUT, ROI, B>(src, dst, batch, H, W, dH, dW, st, rc,
                                                         aff, rois, nn_map);
    }
}

// Waves per workgroup of the exact 2x kernels (one source row or row gap
// each).  The kernels write four times what they read, and one-wave
// workgroups of such short work are slower to dispatch than to run.
// Measured (us, 1080x1920 grey -> 4K / 8x480x640 RGB -> 2x / 1080x1920
// RGBA -> 2x): linear 1 wave 4.13 / 9.65 / 8.53, 2 waves 3.67 / 8.92 / 8.52,
// 4 waves 3.53 / 8.73 / 8.78; nearest 1 wave 3.14 / 6.90 / 7.47, 2 waves
// 3.05 / 6.64 / 7.54, 4 waves 3.05 / 6.58 / 7.60.
// Retested after the XCD-contiguous / segment-major grids and the
// first-row prologue: linear 2 / 4 / 8 waves, 1080p -> 4K grey 3.70 / 3.60
// / 3.88 us, RGB 6.53 / 6.03 / 6.78; nearest 1 / 2 / 4 waves, 4 x 720p grey
// 4.20 / 3.65 / 3.65, 1080p -> 4K RGB 5.47 / 5.56 / 5.68.
template <int C> constexpr int kUp2RowsLinear = C == 4 ? 2 : 4;
template <int C> constexpr int kUp2RowsNearest = C == 4 ? 1 : 2;

template <int C, bool NEAREST>
int launch_up2_u8(const void *src, void *dst, int batch, int H, int W, hipStream_t st)
{
    const int chunks_per_row = W / (NEAREST ? Up2Shape<C>::S : Up2LinShape<C>::S);
    constexpr int RB = NEAREST ? kUp2RowsNearest<C> : kUp2RowsLinear<C>;
    if constexpr (NEAREST) {
        const long long rows = (long long)batch * H;
        const long long gx = (chunks_per_row + 63) / 64;
        const long long gy = (rows + RB - 1) / RB;
        // segment-major for one segment per row, or two with a short second
        // (see the kernel)
        if (gx == 1 || (gx == 2 && chunks_per_row - 64 <= 32))
            return launch(nearest_up2_u8<C, RB, true>,
                          dim3((unsigned)(gy < kMaxGridX ? gy : kMaxGridX), (unsigned)gx),
                          dim3(64, RB), 0, st, (const uint8_t *)src, (uint8_t *)dst, W, rows,
                          chunks_per_row);
        return launch(nearest_up2_u8<C, RB, false>,
                      dim3((unsigned)gx, (unsigned)(gy < kMaxGridY ? gy : kMaxGridY)),
                      dim3(64, RB), 0, st, (const uint8_t *)src, (uint8_t *)dst, W, rows,
                      chunks_per_row);
    } else {
        // H + 1 gaps per image (H <= 32767 since dH <= 65535); a 1-D grid
        // of gx * gy * gz workgroups (at most 2^24, so blocks x threads stays
        // below 2^32), images beyond gz strided
        const long long gx = (chunks_per_row + 63) / 64, gy = (H + RB) / RB;
        long long gz = batch < kMaxGridY ? batch : kMaxGridY;
        if (gx * gy * gz > kMaxGridX) gz = kMaxGridX / (gx * gy);
        // one image: no image arithmetic in the prologue, whose scalar work
        // all resident waves queue for (1080p grey 3.65 -> 3.49 us)
        auto kernel = batch == 1 ? linear_up2_u8<C, RB, true> : linear_up2_u8<C, RB, false>;
        return launch(kernel, dim3((unsigned)(gx * gy * gz)), dim3(64 * RB), 0, st,
                      (const uint8_t *)src, (uint8_t *)dst, H, W, batch, chunks_per_row,
                      (unsigned)gx, (unsigned)gy, (unsigned)gz, make_div_by((unsigned)gx),
                      make_div_by((unsigned)gy));
    }
}

// Exact 2x uint8 upscale whose rows split into whole, 16-byte aligned lanes.
bool up2_path_fits(int C, int H, int W, int dH, int dW, const void *src, const void *dst)
{
    if (dH != 2 * H || dW != 2 * W || !aligned(src, 16) || !aligned(dst, 16)) return false;
    const int S = C == 4 ? Up2Shape<4>::S : Up2Shape<1>::S;
    return W % S == 0 && ((long long)W * C) % 16 == 0;
}


template <int BPP>
int launch_nearest(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                   int map, hipStream_t st)
{
    const long long rows = (long long)batch * dH;
    const Grid g = band_grid(rows, dW, dH);
    auto go = [&](auto kernel) {
        return launch(kernel, dim3(g.blocks), dim3(kBlock), 0, st, (const uint8_t *)src,
                      (uint8_t *)dst, H, W, dH, dW, rows, g.rows_per_block, g.bg, map);
    };
    if constexpr (BPP % 16 == 0) {
        if (aligned(src, 16) && aligned(dst, 16)) return go(nearest_generic<BPP, 16>);
    }
    if constexpr (BPP % 4 == 0) {
        if constexpr (BPP == 12) {
            // 12-byte pixels (float RGB) in rows that start on 16-byte
            // boundaries: staged stores
            if (kDirectStageRgb && dW % 4 == 0 && aligned(src, 4) && aligned(dst, 16))
                return go(nearest_generic<BPP, 4, true>);
        }
        if (aligned(src, 4) && aligned(dst, 4)) return go(nearest_generic<BPP, 4>);
    }
    return go(nearest_generic<BPP, 1>);
}

// uint8 linear resizes on the tiled kernel (tile_u8): workgroups of TH
// output rows by 64 PX columns of one image, every source byte they need
// staged into LDS (in rounds of up to 8 chunks per thread).  A tile of TH
// rows is taken where its staged rows and column table fit kTileLdsBudget;
// false otherwise (the caller then picks another kernel).
constexpr long long kTileLdsBudget = 64 * 1024;

template <int C, int TH, bool NEAREST, int OUT>
bool launch_tile_u8(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                    hipStream_t st, int &rc, int nn_map, long long lds_cap = kTileLdsBudget)
{
    constexpr int PX = C == 1 ? 8 : 4;
    constexpr int COLS = 64 * PX;
    // source columns of one segment and source rows of one tile, at most
    long long span = (long long)(COLS - 1) * W / dW + 3;
    if (span > W) span = W;
    const long long n16cap = (15 + span * C + 15) >> 4;
    const long long pitch = 16 * (n16cap + 1);
    const long long rows_cap = (long long)(TH - 1) * H / dH + 3;
    const long long lds = (long long)COLS * 4 + rows_cap * pitch + 16;
    if (lds > lds_cap) return false;
    const long long chunks = (rows_cap * n16cap + 255) / 256;   // per thread, at most
    const int tiles_x = (dW + COLS - 1) / COLS, tiles_y = (dH + TH - 1) / TH;
    const long long blocks = (long long)batch * tiles_y * tiles_x;
    if (blocks >= (1LL << 31)) return false;
    TileGeom tg;
    tg.tiles_x = tiles_x;
    tg.tiles_y = tiles_y;
    tg.by_tiles_x = fast_div_for(tiles_x);
    tg.by_tiles_y = fast_div_for(tiles_y);
    tg.by_n16 = fast_div_for(n16cap);
    tg.n16cap = (int)n16cap;
    tg.pitch = (int)pitch;
    const long long src_bytes = (long long)batch * H * W * C;
    auto go = [&](auto kernel) {
        rc = launch(kernel, dim3((unsigned)blocks), dim3(64 * kTileWaves), (unsigned)lds, st,
                    (const uint8_t *)src, (uint8_t *)dst, H, W, dH, dW, src_bytes, tg, nn_map);
        return true;
    };
    // chunks per thread and staging round (more rounds where a tile needs them)
    if (chunks <= 1) return go(tile_u8<C, PX, TH, 1, NEAREST, OUT>);
    if (chunks <= 2) return go(tile_u8<C, PX, TH, 2, NEAREST, OUT>);
    if (chunks <= 4) return go(tile_u8<C, PX, TH, 4, NEAREST, OUT>);
    return go(tile_u8<C, PX, TH, 8, NEAREST, OUT>);
}

// The tile height by the launch's size.  A tile runs one memory round trip
// and then TH / 4 rows per wave, so it pays where there are enough tiles to
// keep the chip busy: 16-row tiles from about 700 of them, 8-row tiles from
// about 512 (with fewer the row-segment kernel's many short bands win).
// Measured against the row-segment kernel (us, tiles of 16 / 8 rows):
// 1080p -> 1620x2880 RGB 12.39 -> 10.28 / 11.08, 3 x 480x640 RGB 9.15 ->
// 7.68 / 8.07, 8 x 224^2 -> 896^2 RGB 15.78 -> 12.72 / 14.48, 1080p ->
// 1620x2880 RGBA 13.59 -> 12.20 / 13.16; 720p -> 1080p RGB 7.92 -> 7.74 /
// 7.25, 1080p -> 1200x1600 RGB 8.52 -> 9.63 / 8.07, 720p -> 900x1200 RGB
// 6.87 -> 7.52 / 6.32, grey 1080p -> 1620x2880 8.84 -> 7.30 / 7.00; below
// the floor 480x640 -> 720x960 RGB 4.77 -> 6.08 / 4.98 and 8 x 224^2 ->
// 256^2 RGB 4.23 -> 6.94 / 5.07.  One-channel tiles (512 columns, twice an
// RGB tile's) pay from fewer of them: grey 1080p -> 1620x2880 6.77 -> 6.43
// us with 16-row tiles at 612 of them, 600x800 -> 900x1200 5.79 -> 5.09
// with 8-row tiles at 339 (RGB 1080p -> 1200x1600 lost at 525 16-row tiles,
// 7.54 -> 9.01).  `forced` (MI_RESIZE_PATH=tile) skips the floor.  Downscales and crop batches stay on the row-segment kernel: a
// tile there stages about twice the rows it writes before any blend, and
// the thumbnail batch went 45.1 -> 61.0 us, its random crops 34.8 -> 44.5,
// 4K -> 1440x2560 RGB 10.2 -> 13.8.
constexpr long long kTileBlocks16 = 700;
constexpr long long kTileBlocks8 = 512;
constexpr long long kTileBlocks16One = 400;   // one channel
constexpr long long kTileBlocks8One = 200;
// and 16-row tiles only while one fits 24 KiB of LDS (six workgroups per
// CU): the float RGBA image 4320x7680 -> 5927x3153, whose 2.4x column
// downscale makes 16-row tiles 33 KiB, runs 150.2 us on them and 147.3 on
// 8-row tiles (1080p -> 1620x2880 RGBA, 10 KiB tiles: 19.7 on 16 rows,
// 22.6 on 8); the uint8 enlargements' 16-row tiles stay within ~20 KiB
constexpr long long kTileLds16 = 24 * 1024;

template <int C, bool NEAREST = false, int OUT = kOutSame>
bool try_tile_u8(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                 hipStream_t st, int &rc, bool forced, int nn_map = kNearestHalfPixel)
{
    constexpr int COLS = 64 * (C == 1 ? 8 : 4);
    const long long per_image = (dW + COLS - 1) / COLS;
    const long long b16 = (long long)batch * ((dH + 15) / 16) * per_image;
    const long long b8 = (long long)batch * ((dH + 7) / 8) * per_image;
    const long long min16 = C == 1 ? kTileBlocks16One : kTileBlocks16;
    const long long min8 = C == 1 ? kTileBlocks8One : kTileBlocks8;
    if (b16 >= min16 && launch_tile_u8<C, 16, NEAREST, OUT>(src, dst, batch, H, W, dH, dW, st, rc,
                                                             nn_map, kTileLds16))
        return true;
    if (b8 >= min8 || forced)
        return launch_tile_u8<C, 8, NEAREST, OUT>(src, dst, batch, H, W, dH, dW, st, rc, nn_map);
    return false;
}

// One- and four-channel float32 linear row enlargements on tile_f32: the
// geometry, budget and tile-height rule of the uint8 tiles, 8 pixels per
// lane for one channel (tiles of 512 columns) and 1 for RGBA (64 columns,
// so a lane's 16-byte result is one contiguous store).  Against the
// row-segment / direct kernels: grey 1080p -> 1620x2880 13.55 -> 9.51 us,
// RGBA 20.94 -> 19.69, the 4320x7680 -> 5927x3153 RGBA image 152.2 ->
// 150.6 (its tiles stage 1.13 x the source, where the row-segment bands
// fetched 1.23 x).  Float RGB stays on the direct kernel.
template <int C, int TH>
bool launch_tile_f32(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                     hipStream_t st, int &rc, long long lds_cap = kTileLdsBudget)
{
    constexpr int PX = C == 1 ? 8 : (C == 3 ? 4 : 1);
    constexpr int COLS = 64 * PX;
    constexpr int PB = 4 * C;
    long long span = (long long)(COLS - 1) * W / dW + 3;
    if (span > W) span = W;
    const long long n16cap = (15 + span * PB + 15) >> 4;
    const long long pitch = 16 * (n16cap + 1);
    const long long rows_cap = (long long)(TH - 1) * H / dH + 3;
    const long long lds = (long long)COLS * 8 + rows_cap * pitch + 16;
    if (lds > lds_cap) return false;
    const long long chunks = (rows_cap * n16cap + 255) / 256;
    const int tiles_x = (dW + COLS - 1) / COLS, tiles_y = (dH + TH - 1) / TH;
    const long long blocks = (long long)batch * tiles_y * tiles_x;
    if (blocks >= (1LL << 31)) return false;
    TileGeom tg;
    tg.tiles_x = tiles_x;
    tg.tiles_y = tiles_y;
    tg.by_tiles_x = fast_div_for(tiles_x);
    tg.by_tiles_y = fast_div_for(tiles_y);
    tg.by_n16 = fast_div_for(n16cap);
    tg.n16cap = (int)n16cap;
    tg.pitch = (int)pitch;
    const long long src_bytes = (long long)batch * H * W * PB;
    auto go = [&](auto kernel) {
        rc = launch(kernel, dim3((unsigned)blocks), dim3(64 * kTileWaves), (unsigned)lds, st,
                    (const float *)src, (float *)dst, H, W, dH, dW, src_bytes, tg);
        return true;
    };
    if (chunks <= 1) return go(tile_f32<C, PX, TH, 1>);
    if (chunks <= 2) return go(tile_f32<C, PX, TH, 2>);
    if (chunks <= 4) return go(tile_f32<C, PX, TH, 4>);
    return go(tile_f32<C, PX, TH, 8>);
}

template <int C>
bool try_tile_f32(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                  hipStream_t st, int &rc, bool forced)
{
    constexpr int COLS = 64 * (C == 1 ? 8 : (C == 3 ? 4 : 1));
    const long long per_image = (dW + COLS - 1) / COLS;
    const long long b16 = (long long)batch * ((dH + 15) / 16) * per_image;
    const long long b8 = (long long)batch * ((dH + 7) / 8) * per_image;
    if (b16 >= kTileBlocks16 &&
        launch_tile_f32<C, 16>(src, dst, batch, H, W, dH, dW, st, rc, kTileLds16))
        return true;
    if (b8 >= kTileBlocks8 || forced)
        return launch_tile_f32<C, 8>(src, dst, batch, H, W, dH, dW, st, rc);
    return false;
}

template <typename T, int C>
int linear_dispatch(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                    hipStream_t st)
{
    const Path path = path_override();
    if constexpr (sizeof(T) == 1) {
        if (path == Path::Auto && half_path_fits(C, H, W, dH, dW, src, dst))
            return launch_half_u8<C>(src, dst, batch, dH, dW, st);
        if (path == Path::Auto && up2_path_fits(C, H, W, dH, dW, src, dst))
            return launch_up2_u8<C, false>(src, dst, batch, H, W, st);
    }
    int rc;
    const bool small = small_launch(batch, H, W, dH, dW);
    // row enlargements: the tiled kernels
    if (path == Path::Tile || (path == Path::Auto && !small && dH >= H)) {
        if constexpr (sizeof(T) == 1) {
            if (try_tile_u8<C>(src, dst, batch, H, W, dH, dW, st, rc, path == Path::Tile))
                return rc;
        } else if constexpr (C == 1 || C == 4) {
            if (try_tile_f32<C>(src, dst, batch, H, W, dH, dW, st, rc, path == Path::Tile))
                return rc;
        }
    }
    if (path == Path::RowSeg || path == Path::Tile ||
        (path == Path::Auto && !small && !prefer_direct<T, C>(W, dW)))
        if (try_rowseg<T, C, false>(src, dst, batch, H, W, dH, dW, st, rc)) return rc;
    return launch_linear_generic<T, C>(src, dst, batch, H, W, dH, dW, st);
}

template <int BPP, typename T, int C>
int nearest_dispatch(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                     int map, hipStream_t st)
{
    const Path path = path_override();
    if constexpr (sizeof(T) == 1) {
        // an exact 2x enlargement replicates pixels under the half-pixel and
        // the floor mapping alike (not under round, which shifts by one)
        if (path == Path::Auto && map != kNearestRound && up2_path_fits(C, H, W, dH, dW, src, dst))
            return launch_up2_u8<C, true>(src, dst, batch, H, W, st);
    }
    int rc;
    const bool small = small_launch(batch, H, W, dH, dW);
    if constexpr (sizeof(T) == 1) {
        // row enlargements: the tiled kernel
        if (path == Path::Tile || (path == Path::Auto && !small && dH >= H))
            if (try_tile_u8<C, true>(src, dst, batch, H, W, dH, dW, st, rc, path == Path::Tile,
                                     map))
                return rc;
    }
    // float RGB / RGBA enlargements: the direct kernel, as for linear
    // (1080p RGBA 2x 26.4 vs 41.8 us, RGB 2x 23.0 vs 87.1 us)
    if (path == Path::RowSeg || path == Path::Tile ||
        (path == Path::Auto && !small && !prefer_direct<T, C>(W, dW)))
        if (try_rowseg<T, C, true>(src, dst, batch, H, W, dH, dW, st, rc, Affine{}, nullptr, map))
            return rc;
    return launch_nearest<BPP>(src, dst, batch, H, W, dH, dW, map, st);
}

template <int C, int OUT>
int normalize_dispatch(const void *src, float *dst, int batch, int H, int W, int dH, int dW,
                       hipStream_t st, const Affine &aff)
{
    const Path path = path_override();
    int rc;
    const bool small = small_launch(batch, H, W, dH, dW);
    if (path == Path::RowSeg || (path == Path::Auto && !small))
        if (try_rowseg<uint8_t, C, false, OUT>(src, dst, batch, H, W, dH, dW, st, rc, aff))
            return rc;
    return launch_linear_generic<uint8_t, C, OUT>(src, dst, batch, H, W, dH, dW, st, aff);
}

template <typename T, int C>
int roi_dispatch(const void *src, void *dst, int batch, int H, int W, const int32_t *rois,
                 int dH, int dW, hipStream_t st)
{
    const Path path = path_override();
    int rc;
    const bool small = small_launch(batch, H, W, dH, dW);
    if (path == Path::RowSeg || (path == Path::Auto && !small))
        if (try_rowseg<T, C, false, kOutSame, true>(src, dst, batch, H, W, dH, dW, st, rc,
                                                     Affine{}, rois))
            return rc;
    return launch_linear_generic<T, C, kOutSame, true>(src, dst, batch, H, W, dH, dW, st,
                                                       Affine{}, rois);
}

template <typename T, int C>
int border_dispatch(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                    int border, hipStream_t st)
{
    const long long rows = (long long)batch * dH;
    const Path path = path_override();
    const bool small = small_launch(batch, H, W, dH, dW);
    if (path == Path::RowSeg ||
        (path == Path::Auto && !small && !prefer_direct<T, C>(W, dW))) {
        int rc;
        if (border == MI_RESIZE_BORDER_MIRROR) {
            if (try_rowseg<T, C, false, kOutSame, false, kBorderMirror>(src, dst, batch, H, W, dH,
                                                                        dW, st, rc))
                return rc;
        } else if (try_rowseg<T, C, false, kOutSame, false, kBorderWrap>(src, dst, batch, H, W, dH,
                                                                         dW, st, rc)) {
            return rc;
        }
    }
    const Grid g = band_grid(rows, dW, dH);
    const bool pix4 = C == 4 && aligned(src, 4 * sizeof(T)) && aligned(dst, 4 * sizeof(T));
    auto go = [&](auto kernel) {
        return launch(kernel, dim3(g.blocks), dim3(kBlock), 0, st, (const T *)src, dst, H, W, dH,
                      dW, rows, g.rows_per_block, g.bg, Affine{},
                      (const int32_t *)nullptr);
    };
    if (border == MI_RESIZE_BORDER_MIRROR) {
        if (pix4) return go(linear_generic<T, C, C == 4, kOutSame, false, kBorderMirror>);
        return go(linear_generic<T, C, false, kOutSame, false, kBorderMirror>);
    }
    if (pix4) return go(linear_generic<T, C, C == 4, kOutSame, false, kBorderWrap>);
    return go(linear_generic<T, C, false, kOutSame, false, kBorderWrap>);
}

template <typename T, int C>
int grey_dispatch(const void *src, void *dst, int batch, int H, int W, int dH, int dW,
                  hipStream_t st)
{
    const long long rows = (long long)batch * dH;
    const Path path = path_override();
    if constexpr (sizeof(T) == 1) {
        if (path == Path::Auto && half_path_fits(C, H, W, dH, dW, src, dst))
            return launch_half_u8<C, true>(src, dst, batch, dH, dW, st);
    }
    const bool small = small_launch(batch, H, W, dH, dW);
    int rc;
    if constexpr (sizeof(T) == 1) {
        // row enlargements: the tiled kernel
        if (path == Path::Tile || (path == Path::Auto && !small && dH >= H))
            if (try_tile_u8<C, false, kOutGrey>(src, dst, batch, H, W, dH, dW, st, rc,
                                                path == Path::Tile))
                return rc;
    }
    if (path == Path::RowSeg || path == Path::Tile || (path == Path::Auto && !small))
        if (try_rowseg<T, C, false, kOutGrey>(src, dst, batch, H, W, dH, dW, st, rc)) return rc;
    const Grid g = band_grid(rows, dW, dH);
    return launch(linear_generic<T, C, false, kOutGrey>, dim3(g.blocks), dim3(kBlock), 0, st,
                  (const T *)src, dst, H, W, dH, dW, rows, g.rows_per_block, g.bg,
                  Affine{}, (const int32_t *)nullptr);
}

}  // namespace

extern "C" {

int resize_abi_version(void) { return MI_RESIZE_ABI_VERSION; }

const char *resize_status_string(int status)
{
    switch (status) {
    case MI_RESIZE_OK: return "ok";
    case MI_RESIZE_ERR_NULL: return "src or dst is a null pointer";
    case MI_RESIZE_ERR_SHAPE:
        return "a size is out of range (need 1 <= H, W, dst_H, dst_W <= 65535, batch >= 1, "
               "batch*H*W and batch*dst_H*dst_W <= 2^40)";
    case MI_RESIZE_ERR_CHANNELS: return "channel count must be 1, 3 or 4";
    case MI_RESIZE_ERR_DTYPE: return "dtype must be MI_RESIZE_U8 (0) or MI_RESIZE_F32 (1)";
    case MI_RESIZE_ERR_OVERLAP: return "src and dst buffers overlap";
    case MI_RESIZE_ERR_HIP: return "the HIP runtime refused the kernel launch";
    case MI_RESIZE_ERR_ALIGN: return "float32 src and dst must be 4-byte aligned";
    case MI_RESIZE_ERR_PARAM:
        return "bad normalisation parameters (mean/std must be non-null, std finite and "
               "non-zero, alpha finite, layout 0 or 1)";
    default: return "unknown status";
    }
}

int resize_linear(const void *src, void *dst, int batch, int H, int W, int C, int dtype,
                  int dst_H, int dst_W, void *stream)
{
    const int rc = check_args(src, dst, batch, H, W, C, dtype, dst_H, dst_W);
    if (rc != MI_RESIZE_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == MI_RESIZE_U8) {
        switch (C) {
        case 1: return linear_dispatch<uint8_t, 1>(src, dst, batch, H, W, dst_H, dst_W, st);
        case 3: return linear_dispatch<uint8_t, 3>(src, dst, batch, H, W, dst_H, dst_W, st);
        default: return linear_dispatch<uint8_t, 4>(src, dst, batch, H, W, dst_H, dst_W, st);
        }
    }
    switch (C) {
    case 1: return linear_dispatch<float, 1>(src, dst, batch, H, W, dst_H, dst_W, st);
    case 3: return linear_dispatch<float, 3>(src, dst, batch, H, W, dst_H, dst_W, st);
    default: return linear_dispatch<float, 4>(src, dst, batch, H, W, dst_H, dst_W, st);
    }
}

int resize_nearest_mapping(const void *src, void *dst, int batch, int H, int W, int C, int dtype,
                           int dst_H, int dst_W, int mapping, void *stream)
{
    const int rc = check_args(src, dst, batch, H, W, C, dtype, dst_H, dst_W);
    if (rc != MI_RESIZE_OK) return rc;
    if (mapping != MI_RESIZE_NEAREST_HALF_PIXEL && mapping != MI_RESIZE_NEAREST_FLOOR &&
        mapping != MI_RESIZE_NEAREST_ROUND)
        return MI_RESIZE_ERR_PARAM;
    hipStream_t st = (hipStream_t)stream;
    const int m = mapping;
    if (dtype == MI_RESIZE_U8) {
        switch (C) {
        case 1: return nearest_dispatch<1, uint8_t, 1>(src, dst, batch, H, W, dst_H, dst_W, m, st);
        case 3: return nearest_dispatch<3, uint8_t, 3>(src, dst, batch, H, W, dst_H, dst_W, m, st);
        default: return nearest_dispatch<4, uint8_t, 4>(src, dst, batch, H, W, dst_H, dst_W, m, st);
        }
    }
    switch (C) {
    case 1: return nearest_dispatch<4, float, 1>(src, dst, batch, H, W, dst_H, dst_W, m, st);
    case 3: return nearest_dispatch<12, float, 3>(src, dst, batch, H, W, dst_H, dst_W, m, st);
    default: return nearest_dispatch<16, float, 4>(src, dst, batch, H, W, dst_H, dst_W, m, st);
    }
}

int resize_linear_grey(const void *src, void *dst, int batch, int H, int W, int C, int dtype,
                       int dst_H, int dst_W, void *stream)
{
    const int rc = check_args(src, dst, batch, H, W, C, dtype, dst_H, dst_W, 1);
    if (rc != MI_RESIZE_OK) return rc;
    if (C != 3 && C != 4) return MI_RESIZE_ERR_CHANNELS;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == MI_RESIZE_U8) {
        if (C == 3) return grey_dispatch<uint8_t, 3>(src, dst, batch, H, W, dst_H, dst_W, st);
        return grey_dispatch<uint8_t, 4>(src, dst, batch, H, W, dst_H, dst_W, st);
    }
    if (C == 3) return grey_dispatch<float, 3>(src, dst, batch, H, W, dst_H, dst_W, st);
    return grey_dispatch<float, 4>(src, dst, batch, H, W, dst_H, dst_W, st);
}

int resize_nearest(const void *src, void *dst, int batch, int H, int W, int C, int dtype,
                   int dst_H, int dst_W, void *stream)
{
    return resize_nearest_mapping(src, dst, batch, H, W, C, dtype, dst_H, dst_W,
                                  MI_RESIZE_NEAREST_HALF_PIXEL, stream);
}

int resize_linear_normalize(const void *src, float *dst, int batch, int H, int W, int C,
                            int dst_H, int dst_W, float alpha, const float *mean,
                            const float *std_dev, int layout, void *stream)
{
    // uint8 source, float32 destination of C channels
    const int rc = check_args(src, dst, batch, H, W, C, MI_RESIZE_U8, dst_H, dst_W, C,
                              sizeof(float));
    if (rc != MI_RESIZE_OK) return rc;
    if (!mean || !std_dev || (layout != 0 && layout != 1) || !isfinite(alpha))
        return MI_RESIZE_ERR_PARAM;
    Affine aff{};
    for (int c = 0; c < C; ++c) {
        const double sd = std_dev[c], mu = mean[c];
        if (!isfinite(sd) || sd == 0.0 || !isfinite(mu)) return MI_RESIZE_ERR_PARAM;
        aff.scale[c] = (float)((double)alpha / sd);
        aff.bias[c] = (float)(-mu / sd);
    }
    hipStream_t st = (hipStream_t)stream;
    if (layout == 0) {
        switch (C) {
        case 1: return normalize_dispatch<1, kOutNormNHWC>(src, dst, batch, H, W, dst_H, dst_W, st, aff);
        case 3: return normalize_dispatch<3, kOutNormNHWC>(src, dst, batch, H, W, dst_H, dst_W, st, aff);
        default: return normalize_dispatch<4, kOutNormNHWC>(src, dst, batch, H, W, dst_H, dst_W, st, aff);
        }
    }
    switch (C) {
    case 1: return normalize_dispatch<1, kOutNormNCHW>(src, dst, batch, H, W, dst_H, dst_W, st, aff);
    case 3: return normalize_dispatch<3, kOutNormNCHW>(src, dst, batch, H, W, dst_H, dst_W, st, aff);
    default: return normalize_dispatch<4, kOutNormNCHW>(src, dst, batch, H, W, dst_H, dst_W, st, aff);
    }
}

int resize_linear_roi(const void *src, void *dst, int batch, int H, int W, int C, int dtype,
                      const int32_t *rois, int dst_H, int dst_W, void *stream)
{
    const int rc = check_args(src, dst, batch, H, W, C, dtype, dst_H, dst_W);
    if (rc != MI_RESIZE_OK) return rc;
    if (!rois) return MI_RESIZE_ERR_NULL;
    if (!aligned(rois, 4)) return MI_RESIZE_ERR_ALIGN;
    hipStream_t st = (hipStream_t)stream;
    if (dtype == MI_RESIZE_U8) {
        switch (C) {
        case 1: return roi_dispatch<uint8_t, 1>(src, dst, batch, H, W, rois, dst_H, dst_W, st);
        case 3: return roi_dispatch<uint8_t, 3>(src, dst, batch, H, W, rois, dst_H, dst_W, st);
        default: return roi_dispatch<uint8_t, 4>(src, dst, batch, H, W, rois, dst_H, dst_W, st);
        }
    }
    switch (C) {
    case 1: return roi_dispatch<float, 1>(src, dst, batch, H, W, rois, dst_H, dst_W, st);
    case 3: return roi_dispatch<float, 3>(src, dst, batch, H, W, rois, dst_H, dst_W, st);
    default: return roi_dispatch<float, 4>(src, dst, batch, H, W, rois, dst_H, dst_W, st);
    }
}

int resize_linear_border(const void *src, void *dst, int batch, int H, int W, int C, int dtype,
                         int dst_H, int dst_W, int border, void *stream)
{
    const int rc = check_args(src, dst, batch, H, W, C, dtype, dst_H, dst_W);
    if (rc != MI_RESIZE_OK) return rc;
    if (border != MI_RESIZE_BORDER_CLAMP && border != MI_RESIZE_BORDER_MIRROR &&
        border != MI_RESIZE_BORDER_WRAP)
        return MI_RESIZE_ERR_PARAM;
    if (border == MI_RESIZE_BORDER_CLAMP)
        return resize_linear(src, dst, batch, H, W, C, dtype, dst_H, dst_W, stream);
    hipStream_t st = (hipStream_t)stream;
    if (dtype == MI_RESIZE_U8) {
        switch (C) {
        case 1: return border_dispatch<uint8_t, 1>(src, dst, batch, H, W, dst_H, dst_W, border, st);
        case 3: return border_dispatch<uint8_t, 3>(src, dst, batch, H, W, dst_H, dst_W, border, st);
        default: return border_dispatch<uint8_t, 4>(src, dst, batch, H, W, dst_H, dst_W, border, st);
        }
    }
    switch (C) {
    case 1: return border_dispatch<float, 1>(src, dst, batch, H, W, dst_H, dst_W, border, st);
    case 3: return border_dispatch<float, 3>(src, dst, batch, H, W, dst_H, dst_W, border, st);
    default: return border_dispatch<float, 4>(src, dst, batch, H, W, dst_H, dst_W, border, st);
    }
}

int resize_copy_bytes(const void *src, void *dst, int64_t nbytes, void *stream)
{
    if (!src || !dst) return MI_RESIZE_ERR_NULL;
    if (nbytes < 0) return MI_RESIZE_ERR_SHAPE;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (nbytes > 0 && s0 < d0 + (uintptr_t)nbytes && d0 < s0 + (uintptr_t)nbytes)
        return MI_RESIZE_ERR_OVERLAP;
    if (nbytes == 0) return MI_RESIZE_OK;
    hipStream_t st = (hipStream_t)stream;
    long long head = 0;
    if (aligned(src, 16) && aligned(dst, 16)) {
        const long long n16 = nbytes / 16;
        if (n16 > 0) {
            // up to 32 MiB one chunk per lane (more waves for a short
            // launch); beyond, enough lanes for about one unrolled pass each
            long long blocks = (n16 + kBlock - 1) / kBlock;
            if (blocks > 8192)
                blocks = (n16 + kBlock * kCopyUnroll - 1) / (kBlock * kCopyUnroll);
            if (blocks > kMaxStrideBlocks) blocks = kMaxStrideBlocks;
            const int rc = launch(copy_16, dim3((unsigned)blocks), dim3(kBlock), 0, st,
                                  (const uint4 *)src, (uint4 *)dst, n16);
            if (rc != MI_RESIZE_OK) return rc;
            head = n16 * 16;
        }
    }
    const long long rest = nbytes - head;
    if (rest > 0) {
        long long blocks = (rest + kBlock - 1) / kBlock;
        if (blocks > kMaxStrideBlocks) blocks = kMaxStrideBlocks;
        return launch(copy_1, dim3((unsigned)blocks), dim3(kBlock), 0, st,
                      (const uint8_t *)src + head, (uint8_t *)dst + head, rest);
    }
    return MI_RESIZE_OK;
}

}  // extern "C"
