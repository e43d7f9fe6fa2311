// gfx950 kernels for linear (bilinear) and nearest-neighbour image resize.
//
// Internal to libmi_resize.so; the C ABI in resize_abi.hip validates the
// arguments and launches these.  What is computed is stated in
// include/mi_resize.h; the passages it follows are "From Prototype to
// Performance: Optimizing OpenCV Resize on Volcanic GPUs" (Imagination blog,
// "Naive resize with linear sampling": pixel centre + 0.5 scaled into the
// input, linear filter) and hnwysp.cn news/129086 (s2.1 nearest, s2.2 the
// four-neighbour bilinear sum, s3.3 / s6.1 clamping, s6.2 fixed point).
//
// Data layout: NHWC, channels interleaved, images back to back.  Output rows
// are numbered globally, g = n * dH + dy, so a batch is one long column of
// rows and the grid never has to know where one image ends.
//
// Every lane owns a fixed set of output columns for the whole band of rows
// its block covers, so the per-column taps and weights (the "x table") are
// computed once per lane and kept in registers across the band; per-row taps
// and weights are uniform across the block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mirsz {

constexpr int kBlock = 256;   // 4 wave64 per workgroup
// The direct kernels' lane-contiguous stores carry the non-temporal hint
// (their output is never read back; float RGBA 1080p -> 2x 51.7 -> 29.9 us).
constexpr bool kDirectNtStores = true;
// four dwords as a native vector (16-byte loads and stores, non-temporal ones)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Orders this wave's LDS accesses before and after it.  A wave's LDS
// operations complete in issue order, so keeping the compiler from moving
// them across this point is all the synchronisation a wave-private slot needs.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Division by a launch-time constant d >= 1 as a multiply and a shift, for
// dividends below 2^31 (the round-up method: shift = 31 + ceil(log2 d),
// magic = floor(2^shift / d) + 1; exact for every such dividend).  Built on
// the host, passed by value.
struct DivBy {
    unsigned long long magic;
    int shift;
};

inline DivBy make_div_by(unsigned d)
{
    int lg = 0;
    while ((1ULL << lg) < d) ++lg;
    return DivBy{(1ULL << (31 + lg)) / d + 1, 31 + lg};
}

__device__ __forceinline__ unsigned div_by(unsigned n, DivBy d)
{
    return (unsigned)((n * d.magic) >> d.shift);
}

// Workgroups reach the 8 XCDs round-robin by linear id.  This renumbers
// workgroup lin of nwg so that each XCD takes one contiguous run of ids
// (XCD k the k-th run): where the work per workgroup repeats with the grid's
// x extent (a short last segment of every row), whole rows then share out
// evenly, and neighbouring rows stay on one XCD.
__device__ __forceinline__ unsigned xcd_contiguous(unsigned lin, unsigned nwg)
{
    const unsigned xcd = lin & 7;
    return xcd * (nwg >> 3) + min(xcd, nwg & 7) + (lin >> 3);
}

// Division by a launch constant d (1 <= d <= 2^31) as a multiply: for
// 0 <= n < 2^31, floor(n / d) = umulhi(2n, m) >> s with s = ceil(log2 d)
// and m = ceil(2^(31+s) / d) < 2^32.  Since m d - 2^(31+s) lies in [0, d),
// n m / 2^(31+s) exceeds n / d by less than n / 2^(31+s) < 2^-s <= 1 / d,
// which never carries it past the next integer.  The host computes m and s.
struct FastDiv {
    unsigned m, s;
};

__device__ __forceinline__ unsigned fast_div(unsigned n, FastDiv f)
{
    return __umulhi(2u * n, f.m) >> f.s;
}

// The direct kernels' 1-D grid: col_blocks workgroups side by side per band
// of rows_per_block output rows (rows numbered across the batch), with the
// divisions that split a workgroup index and a row index.
struct BandGrid {
    int col_blocks;
    FastDiv by_cols;    // d = col_blocks
    FastDiv by_dst_h;   // d = dH
};

// The band and column block of this workgroup, and the image and row of
// output row g.
__device__ __forceinline__ void band_of_block(const BandGrid &bg, long long &rb, int &cb)
{
    const unsigned r = fast_div(blockIdx.x, bg.by_cols);   // grids stay far below 2^31
    rb = r;
    cb = (int)(blockIdx.x - r * (unsigned)bg.col_blocks);
}

__device__ __forceinline__ long long image_of_row(long long g, int dH, const BandGrid &bg)
{
    return g < (1LL << 31) ? (long long)fast_div((unsigned)g, bg.by_dst_h) : g / dH;
}

// --------------------------------------------------------------------------
// Exact floor division for the coordinate maps below: q = floor(num / den)
// and r = num - q den in [0, den), for an integer num with |num / den| below
// 2^17 and den in [1, 2^17).  The caller passes num twice: numf, num rounded
// once to fp32 (an fma of exact small factors, or a correctly rounded
// conversion), and num_lo, its low 32 bits.  The estimate numf x rcp(den)
// carries three roundings of at most 2^-24, 2^-23 (the hardware reciprocal's
// one ulp) and 2^-24 relative, so it lies within 2^17 x 2^-22 = 2^-5 of
// num / den and its floor is q or q +- 1.  The remainder of that guess lies
// in [-den, 2 den), inside 32 bits, so the wrapped 32-bit difference is
// exact and one step in either direction fixes q.  About 8 instructions
// where an fp64 division with its conversions costs ~40; checked against
// integer floor division over the maps' full ranges (2 n_out, n_in up to
// 65535, the biases used here, and reciprocals one ulp off either way).
// --------------------------------------------------------------------------
struct QR { int q, r; };

__device__ __forceinline__ QR floor_divmod(float numf, unsigned num_lo, int den)
{
    int q = (int)floorf(numf * __builtin_amdgcn_rcpf((float)den));
    int r = (int)(num_lo - (unsigned)__mul24(q, den));
    if (r < 0) { q -= 1; r += den; } else if (r >= den) { q += 1; r -= den; }
    return {q, r};
}

// floor_divmod of 2 d n_in + bias: every factor and the bias are below 2^24,
// so one fma rounds the numerator once and 24-bit multiplies give its low
// word (d < 2^16, n_in <= 65535, |bias| < 2^17).
__device__ __forceinline__ QR map_divmod(int d2, int n_in, int bias, int den)
{
    return floor_divmod(__builtin_fmaf((float)d2, (float)n_in, (float)bias),
                        __umul24((unsigned)d2, (unsigned)n_in) + (unsigned)bias, den);
}

// --------------------------------------------------------------------------
// Coordinate map for one axis.  Output index d of an axis of n_out samples
// taken from n_in samples: x = (d + 1/2) n_in / n_out - 1/2 = num / den with
// num = (2d + 1) n_in - n_out, den = 2 n_out.  x0 = floor(x) and the
// remainder r = num - x0 den in [0, den) come out exact from floor_divmod
// (the quotient lies in [-1, n_in)).  Taps are clamped to the edge.
// --------------------------------------------------------------------------
struct Tap {
    int a;      // clamp(x0, 0, n_in - 1)
    int b;      // clamp(x0 + 1, 0, n_in - 1)
    int r;      // remainder, u = r / den
    int den;    // 2 * n_out
};

__device__ __forceinline__ Tap axis_tap(int d, int n_in, int n_out)
{
    const int den = 2 * n_out;
    const QR m = map_divmod(2 * d + 1, n_in, -n_out, den);
    Tap t;
    t.a = m.q < 0 ? 0 : (m.q > n_in - 1 ? n_in - 1 : m.q);
    t.b = m.q + 1 < 0 ? 0 : (m.q + 1 > n_in - 1 ? n_in - 1 : m.q + 1);
    t.r = m.r;
    t.den = den;
    return t;
}

// Border rules for source coordinates beyond the outermost pixel centres
// (hnwysp.cn news/129086 s6.1): clamp to the edge (the default), mirror
// (reflect the coordinate about the outermost pixel centres: x -> -x below 0,
// x -> 2 (n - 1) - x above n - 1) or wrap (periodic image).  The half-pixel
// map keeps every coordinate within (-1/2, n - 1/2), so one reflection or one
// period always brings it inside.  Mirror and wrap act on the exact
// coordinate before the floor, as the definition states; for linear
// interpolation mirror equals reflecting the taps about the edge pixel.
enum : int { kBorderClamp = 0, kBorderMirror = 1, kBorderWrap = 2 };

template <int B>
__device__ __forceinline__ Tap axis_tap_b(int d, int n_in, int n_out)
{
    if constexpr (B == kBorderClamp) {
        return axis_tap(d, n_in, n_out);
    } else {
        long long num = (long long)(2 * d + 1) * n_in - n_out;
        const int den = 2 * n_out;
        Tap t;
        t.den = den;
        if (n_in == 1) {
            t.a = t.b = 0;
            t.r = 0;
            return t;
        }
        const long long last = (long long)(n_in - 1) * den;
        if constexpr (B == kBorderMirror) {
            if (num < 0) num = -num;
            if (num > last) num = 2 * last - num;
        } else {
            if (num < 0) num += (long long)n_in * den;
            if (num >= (long long)n_in * den) num -= (long long)n_in * den;
        }
        // num now lies in [0, n_in den): the quotient in [0, n_in)
        const QR m = floor_divmod((float)num, (unsigned)num, den);
        t.a = m.q;
        t.b = m.q + 1 < n_in ? m.q + 1 : (B == kBorderWrap ? 0 : n_in - 1);
        t.r = m.r;
        return t;
    }
}

// u rounded half up to 11 fractional bits: floor(n / d) with n = 4096 r +
// den < 2^30 and d = 2 den (den <= 131070), in [0, 2048].  The quotient is
// estimated in fp32 - n converts with relative error <= 2^-24, the hardware
// reciprocal is within one ulp, the product rounds once, so the estimate is
// within 2049 x 2^-22 < 1 of n / d - and its truncation corrected by one
// step in either direction from the exact remainder.  About 8 instructions
// instead of a 32-bit integer division's ~35; checked against the division
// for every r < den = 2 n_out, n_out = 1 .. 65535, on the GPU (no
// difference), and the band set-up that runs it PX times per lane got
// faster with it (1080p -> 1620x2880 RGB 14.97 -> 14.50 us).
__device__ __forceinline__ unsigned weight11(const Tap &t)
{
    const unsigned n = (unsigned)t.r * 4096u + (unsigned)t.den, d = 2u * (unsigned)t.den;
    const unsigned q = (unsigned)((float)n * __builtin_amdgcn_rcpf((float)d));
    const int rem = (int)(n - q * d);
    return rem < 0 ? q - 1 : (rem >= (int)d ? q + 1 : q);
}

// u as float: r and den are below 2^24, so both convert exactly and the
// quotient is correctly rounded.
__device__ __forceinline__ float weightf(const Tap &t)
{
    return (float)t.r / (float)t.den;
}

// Nearest source index under one of three mappings, each
// floor((2 d n_in + bias) / (2 n_out)) limited to n_in - 1 and exact by the
// same argument as axis_tap:
//   kNearestHalfPixel  (the default) the half-pixel coordinate rounded half
//                      up, floor((2d + 1) n_in / (2 n_out)): bias n_in;
//   kNearestFloor      the corner-aligned coordinate d n_in / n_out
//                      (hnwysp.cn news/129086 s3.2 maps d / scale with no
//                      half-pixel shift), floored - the legacy nearest of
//                      image libraries: bias 0;
//   kNearestRound      the same coordinate rounded half up, as that kernel's
//                      floor(x + 0.5): bias n_out.
enum : int { kNearestHalfPixel = 0, kNearestFloor = 1, kNearestRound = 2 };

__device__ __forceinline__ int nearest_bias(int map, int n_in, int n_out)
{
    return map == kNearestFloor ? 0 : (map == kNearestRound ? n_out : n_in);
}

__device__ __forceinline__ int nearest_index(int d, int n_in, int n_out, int map)
{
    const int q = map_divmod(2 * d, n_in, nearest_bias(map, n_in, n_out), 2 * n_out).q;
    return q > n_in - 1 ? n_in - 1 : q;
}

// 11-bit fixed-point blend of one channel, exact in 32 bits:
// every partial sum is below 2048 * 2048 * 255 + 2^21 < 2^31.  The weights
// lie in [0, 2048]; masking them to 12 bits (a no-op on their values, and
// hoisted out of the row loop) shows the compiler that every product fits
// the full-rate 24-bit multiply-add, where it otherwise picks quarter-rate
// 32-bit multiplies and 64-bit multiply-adds.
__device__ __forceinline__ unsigned blend_u8(unsigned p00, unsigned p01, unsigned p10,
                                             unsigned p11, unsigned wx1, unsigned wy1)
{
    wx1 &= 0xfffu;
    wy1 &= 0xfffu;
    const unsigned wx0 = (2048u - wx1) & 0xfffu, wy0 = (2048u - wy1) & 0xfffu;
    const unsigned top = __umul24(wx0, p00) + __umul24(wx1, p01);
    const unsigned bot = __umul24(wx0, p10) + __umul24(wx1, p11);
    return (__umul24(wy0, top) + __umul24(wy1, bot) + (1u << 21)) >> 22;
}

// The same blend on tap pairs, for kernels that hold each row's two taps of
// a channel as 16-bit halves of one register (tap a low, tap b high) and
// the column weights as the pair (2048 - u, u): one unsigned 16-bit dot
// product per row gives wx0 p_a + wx1 p_b <= 2048 * 255 exactly, and the
// row sums are combined with the row weights scaled by 4, so that
//   4 (wy0 top + wy1 bot) + 2^23 = 4 (sum + 2^21) < 2^32
// carries the rounded result, floor((sum + 2^21) / 2^22), in bits 24..31:
// a byte permute then packs it with no shift.  Where both taps are one
// column the pair (2048, 0) gives 2048 p_a, as the scalar form does.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// One row's horizontal sum wx0 p_a + wx1 p_b from a tap pair and a weight pair.
__device__ __forceinline__ uint32_t row_sum_u8(uint32_t pair, uint32_t wx)
{
    return __builtin_amdgcn_udot2(__builtin_bit_cast(u16x2_t, pair), __builtin_bit_cast(u16x2_t, wx),
                                  0u, false);
}

// a * b + c on the full-rate 24-bit multiply-add: a and b below 2^24, the
// result modulo 2^32.  Written out because from the plain expression the
// compiler keeps two multiplies and a three-way add, one more instruction
// per sum.
__device__ __forceinline__ uint32_t mad_u24(uint32_t a, uint32_t b, uint32_t c)
{
    uint32_t r;
    asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// The vertical step: the rounded result in bits 24..31.
__device__ __forceinline__ uint32_t col_sum_u8(uint32_t top, uint32_t bot, uint32_t wy0x4,
                                               uint32_t wy1x4)
{
    return mad_u24(wy0x4, top, mad_u24(wy1x4, bot, 1u << 23));
}

__device__ __forceinline__ uint32_t blend_u8_pairs(uint32_t pa, uint32_t pb, uint32_t wx,
                                                   uint32_t wy0x4, uint32_t wy1x4)
{
    return col_sum_u8(row_sum_u8(pa, wx), row_sum_u8(pb, wx), wy0x4, wy1x4);
}

// Column weight pair of blend_u8_pairs: (2048 - u, u), or (2048, 0) where
// tap b is not the next column.
__device__ __forceinline__ uint32_t weight_pair(unsigned u, bool next)
{
    return next ? (2048u - u) | (u << 16) : 2048u;
}

// Byte 3 of each of four words, packed into one word (first word lowest).
__device__ __forceinline__ uint32_t pack_byte3(uint32_t f0, uint32_t f1, uint32_t f2, uint32_t f3)
{
    const uint32_t lo = __builtin_amdgcn_perm(f1, f0, 0x0c0c0703u);
    const uint32_t hi = __builtin_amdgcn_perm(f3, f2, 0x0c0c0703u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

__device__ __forceinline__ float blend_f32(float p00, float p01, float p10, float p11,
                                           float wx, float wy)
{
    const float t = fmaf(wx, p01 - p00, p00);
    const float b = fmaf(wx, p11 - p10, p10);
    return fmaf(wy, b - t, t);
}

// --------------------------------------------------------------------------
// Output stage.  kOutSame stores the resized elements in the source type.
// The normalising stages (uint8 sources) store float32
//     out = v * scale[c] + bias[c]      (one fused multiply-add)
// where v is the exact uint8 resize result, either interleaved like the
// source (NHWC) or as one plane per channel (NCHW).  The host derives
// scale = alpha / std and bias = -mean / std in double precision.
// kOutGrey (RGB or RGBA sources) converts every tap to grey first - the
// pages' preprocessing runs cvtColor's RGB2Gray before resize ("Performance
// Optimization of Object Tracking Algorithms in OpenCV on GPUs" s3.1.1) -
// and stores one channel of the source type.
// --------------------------------------------------------------------------
enum : int { kOutSame = 0, kOutNormNHWC = 1, kOutNormNCHW = 2, kOutGrey = 3 };

// Grey value of one RGB pixel with the ITU-R BT.601 luma weights 0.299,
// 0.587 and 0.114: exact for uint8, rounded half up; two fused
// multiply-adds for float32.
__device__ __forceinline__ unsigned grey_u8(unsigned r, unsigned g, unsigned b)
{
    return (299u * r + 587u * g + 114u * b + 500u) / 1000u;
}

__device__ __forceinline__ float grey_f32(float r, float g, float b)
{
    return fmaf(0.114f, b, fmaf(0.587f, g, 0.299f * r));
}

struct Affine {
    float scale[4];
    float bias[4];
};

// Region of interest of image n: crop {x, y, w, h} from a device array of
// int32 quadruples, clamped into the image (x in [0, W-1], w in [1, W - x],
// likewise y / h), so any values are safe to read through.
struct Crop {
    int x, y, w, h;
};

__device__ __forceinline__ Crop load_crop(const int32_t *rois, long long n, int H, int W)
{
    const int32_t *q = rois + 4 * n;
    Crop c;
    c.x = min(max((int)q[0], 0), W - 1);
    c.y = min(max((int)q[1], 0), H - 1);
    c.w = min(max((int)q[2], 1), W - c.x);
    c.h = min(max((int)q[3], 1), H - c.y);
    return c;
}

// --------------------------------------------------------------------------
// Generic linear resize, any scale, C in {1, 3, 4}.  Grid: 1-D,
// blockIdx = row_block * col_blocks + col_block, split by a multiply
// (BandGrid).  Replacing that division and the one of the first row by dH,
// each a ~20-instruction sequence ahead of the first load, with FastDiv made
// the small launches 5-10 % faster (48x64 -> 72x96 grey 2.04 -> 1.93 us,
// 16 x 64x64 -> 96x96 RGB 3.35 -> 3.03).  A block covers kBlock
// output columns of `rows_per_block` consecutive global rows; one lane per
// output pixel per row.  PIX4: C == 4 and the buffers are aligned so that a
// whole pixel moves as one 4-byte (u8) or 16-byte (f32) access.
// --------------------------------------------------------------------------
//
// Stores: a lane's value or 4- or 16-byte pixel is one lane-contiguous
// store with the non-temporal hint (one-byte values excepted: 64 bytes per
// instruction are part of a line).  STG (float RGB, output rows 16-byte
// aligned): each wave's 64 pixels (768 bytes) go through LDS and out as
// lane-contiguous 16-byte non-temporal stores instead of three strided
// floats per lane; lanes past the row end then compute on the last
// column's taps and store nothing.
template <typename T, int C, bool PIX4, int OUT = kOutSame, bool ROI = false,
          int BORDER = kBorderClamp, bool STG = false>
__global__ __launch_bounds__(kBlock) void linear_generic(
    const T *__restrict__ src, void *__restrict__ dst_v, int H, int W, int dH, int dW,
    long long rows_total, int rows_per_block, BandGrid bg, Affine aff,
    const int32_t *__restrict__ rois)
{
    static_assert(!STG || (sizeof(T) == 4 && C == 3 && OUT == kOutSame && !ROI &&
                           BORDER == kBorderClamp), "staged stores are for float RGB");
    T *const dst = (T *)dst_v;
    float *const dstf = (float *)dst_v;
    auto st = [](auto &ref, auto v) {
        if constexpr (kDirectNtStores && sizeof(v) > 1) __builtin_nontemporal_store(v, &ref);
        else ref = v;
    };
    __shared__ __attribute__((aligned(16))) float stage_all[STG ? kBlock * C : 1];
    long long rb;
    int cb;
    band_of_block(bg, rb, cb);
    const int wave_x0 = cb * kBlock + ((int)threadIdx.x & ~63);   // the wave's first column
    const int x_lane = cb * kBlock + (int)threadIdx.x;
    if (STG ? wave_x0 >= dW : x_lane >= dW) return;
    const int x = STG ? min(x_lane, dW - 1) : x_lane;

    long long g = rb * rows_per_block;
    long long g_end = g + rows_per_block;
    if (g_end > rows_total) g_end = rows_total;
    long long n = image_of_row(g, dH, bg);
    int dy = (int)(g - n * dH);
    const size_t img_elems = (size_t)H * W * C;
    const size_t row_elems = (size_t)W * C;

    // the source region resized: the whole image or image n's crop
    Crop crop{0, 0, W, H};
    if constexpr (ROI) crop = load_crop(rois, n, H, W);
    int xa, xb;
    unsigned wx1 = 0;
    float wxf = 0.f;
    auto column = [&]() {
        const Tap tx = axis_tap_b<BORDER>(x, crop.w, dW);
        xa = (crop.x + tx.a) * C;
        xb = (crop.x + tx.b) * C;
        if constexpr (sizeof(T) == 1) wx1 = weight11(tx);
        else wxf = weightf(tx);
    };
    column();

    for (; g < g_end; ++g) {
        const Tap ty = axis_tap_b<BORDER>(dy, crop.h, dH);
        const T *img = src + (size_t)n * img_elems;
        const T *r0 = img + (size_t)(crop.y + ty.a) * row_elems;
        const T *r1 = img + (size_t)(crop.y + ty.b) * row_elems;
        T *out = dst + ((size_t)g * dW + x) * C;
        if constexpr (sizeof(T) == 1) {
            const unsigned wy1 = weight11(ty);
            if constexpr (PIX4) {
                const uint32_t a = *(const uint32_t *)(r0 + xa);
                const uint32_t b = *(const uint32_t *)(r0 + xb);
                const uint32_t c = *(const uint32_t *)(r1 + xa);
                const uint32_t d = *(const uint32_t *)(r1 + xb);
                uint32_t o = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int s = 8 * k;
                    o |= blend_u8((a >> s) & 255u, (b >> s) & 255u, (c >> s) & 255u,
                                  (d >> s) & 255u, wx1, wy1) << s;
                }
                st(*(uint32_t *)out, o);
            } else if constexpr (OUT == kOutSame) {
#pragma unroll
                for (int k = 0; k < C; ++k) {
                    const uint8_t v = (uint8_t)blend_u8(r0[xa + k], r0[xb + k], r1[xa + k],
                                                        r1[xb + k], wx1, wy1);
                    if constexpr (C == 1) st(out[k], v); else out[k] = v;
                }
            } else if constexpr (OUT == kOutGrey) {
                auto gr = [](const T *p) { return grey_u8(p[0], p[1], p[2]); };
                st(dst[(size_t)g * dW + x],
                   (uint8_t)blend_u8(gr(r0 + xa), gr(r0 + xb), gr(r1 + xa), gr(r1 + xb), wx1, wy1));
            } else {
#pragma unroll
                for (int k = 0; k < C; ++k) {
                    const float v = (float)blend_u8(r0[xa + k], r0[xb + k], r1[xa + k],
                                                    r1[xb + k], wx1, wy1);
                    const float o = fmaf(v, aff.scale[k], aff.bias[k]);
                    if constexpr (OUT == kOutNormNHWC)
                        dstf[((size_t)g * dW + x) * C + k] = o;
                    else
                        st(dstf[(((size_t)n * C + k) * dH + dy) * dW + x], o);
                }
            }
        } else {
            const float wyf = weightf(ty);
            if constexpr (PIX4) {
                const float4 a = *(const float4 *)(r0 + xa);
                const float4 b = *(const float4 *)(r0 + xb);
                const float4 c = *(const float4 *)(r1 + xa);
                const float4 d = *(const float4 *)(r1 + xb);
                float4 o;
                o.x = blend_f32(a.x, b.x, c.x, d.x, wxf, wyf);
                o.y = blend_f32(a.y, b.y, c.y, d.y, wxf, wyf);
                o.z = blend_f32(a.z, b.z, c.z, d.z, wxf, wyf);
                o.w = blend_f32(a.w, b.w, c.w, d.w, wxf, wyf);
                st(*(u32x4_t *)out, __builtin_bit_cast(u32x4_t, o));
            } else if constexpr (OUT == kOutGrey) {
                auto gr = [](const T *p) { return grey_f32(p[0], p[1], p[2]); };
                st(dst[(size_t)g * dW + x],
                   blend_f32(gr(r0 + xa), gr(r0 + xb), gr(r1 + xa), gr(r1 + xb), wxf, wyf));
            } else if constexpr (STG) {
                float *stage = stage_all + (threadIdx.x & ~63) * C;   // this wave's 64 pixels
#pragma unroll
                for (int k = 0; k < C; ++k)
                    stage[(threadIdx.x & 63) * C + k] =
                        blend_f32(r0[xa + k], r0[xb + k], r1[xa + k], r1[xb + k], wxf, wyf);
                wave_sync();
                // the row segment's bytes: a multiple of 48 (dW % 4 == 0)
                const int seg_bytes = min(64, dW - wave_x0) * C * 4;
                const int bb = 16 * (threadIdx.x & 63);
                if (bb < seg_bytes)
                    __builtin_nontemporal_store(
                        *(const u32x4_t *)((const uint8_t *)stage + bb),
                        (u32x4_t *)((uint8_t *)(dst + ((size_t)g * dW + wave_x0) * C) + bb));
                wave_sync();
            } else {
#pragma unroll
                for (int k = 0; k < C; ++k) {
                    const float v = blend_f32(r0[xa + k], r0[xb + k], r1[xa + k], r1[xb + k], wxf, wyf);
                    if constexpr (C == 1) st(out[k], v); else out[k] = v;
                }
            }
        }
        if (++dy == dH) {
            dy = 0;
            ++n;
            if constexpr (ROI) {
                if (g + 1 < g_end) {
                    crop = load_crop(rois, n, H, W);
                    column();
                }
            }
        }
    }
}

// --------------------------------------------------------------------------
// Exact 2:1 downscale of uint8 (H = 2 dH, W = 2 dW).  The half-pixel centre
// of output pixel d lands exactly between source pixels 2d and 2d + 1
// (x = 2d + 1/2), so both 11-bit weights are 1024 on both axes and the
// general formula reduces, bit for bit, to the rounded 2x2 mean
// (a + b + c + d + 2) >> 2.  No tap is ever clamped.
//
// A wave owns a segment of 64 * PX output pixels of one output row
// (PX = 16 for C = 1, 4 for C = 3 and 4).  Each source row of the
// segment (2 PX C bytes per lane) is read with 16-byte non-temporal loads at
// lane-consecutive addresses - every load instruction covers whole cache
// lines, which is what lets the streaming hint help - and staged in LDS; each
// lane then reads its 2 PX C bytes of both rows back, forms PX C means and
// writes them with one contiguous store.  Measured on the 4K RGB frame this
// beats lanes that load their own (strided) bytes directly by about 8 %, and
// matches a plain kernel with the same 4:1 read / write byte mix.
// Needs dW % (C == 1 ? 16 : C == 3 ? 8 : 4) == 0 and 16-byte aligned src /
// dst, so every row and every 16-byte chunk is aligned.  Output row g reads
// source rows 2g and 2g + 1 of the flattened N * H rows, because H = 2 dH.
//
// Two grid layouts.  Rows of one or two segments (small frames in a batch)
// use seg_major: x = output rows (stride gridDim.x), y = segment; a grid
// that is 1 or 2 workgroups wide and thousands tall dispatches markedly
// slower than the same workgroups laid along x (64 x 224x224 RGB: 5.28 ->
// 4.08 us; 16 x 640x480 RGB: 5.82 -> 4.89 us, where the full first
// segments of all rows also go out before the short second ones).  Wider
// rows number their (row, segment) items row-major with the XCD
// renumbering below (4K RGB 6.50 -> 6.40 us, 4K RGBA 8.38 -> 8.21 us,
// 8 x 1080p RGB 11.10 -> 10.89 us, all on a 2-D grid of one-wave
// workgroups, since replaced by the 1-D grid of two-wave workgroups); the
// segment-major order is slower there (4K RGBA 8.71 us).  Eight pixels per lane instead of
// four (RGB, RGBA) measured slower on the 4K frames (RGB 6.52 -> 6.97 us),
// and so did fewer workgroups looping over 2 or 4 rows each (6.39 -> 6.75 /
// 6.90 us): one row per wave keeps the most loads in flight.  Grey output
// with 8 pixels per lane was slower too (4K -> 1080p grey 6.09-6.26 ->
// 6.40-6.43 us), and would need widths that are multiples of 8 for RGBA.
// --------------------------------------------------------------------------
template <int C> struct HalfShape { static constexpr int PX = C == 1 ? 16 : 4; };

constexpr int kHalfLanes = 64;
// Waves per workgroup of the row-major grid, each with its own segment.
// Workgroups of one wave dispatch slowly: an empty launch of 8640 of them
// costs 2.9 us back to back (4.6 us on the earlier 8 x 1080 2-D grid),
// against 2.0 us for 4320 two-wave and 1.54 us for 2160 four-wave
// workgroups.  A single 4K RGB launch does not see it (its dispatch
// overlaps the memory phase: 6.43 us with one or two waves, 6.52 four,
// 6.61 eight), but frames pipelined over three streams do, where the
// dispatcher serves several grids at once: 5.41 us per frame with one
// wave, 5.06-5.12 with two, 5.05-5.08 with four.
constexpr int kHalfWaves = 2;


__device__ __forceinline__ uint4 load_stream(const uint8_t *p)
{
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Writes one wave's output row segment back to device memory.  The segment
// sits in LDS lane-major (lane L's OUT bytes at L * OUT); store k of every
// lane takes bytes [1024 k + 16 L, +16), so each store instruction of the
// wave covers 1 KiB of whole cache lines, which the non-temporal hint needs
// to pay (strided 16-byte pieces of a lane's own chunk would leave partial
// lines).  seg_bytes = active lanes * OUT.
template <int OUT>
__device__ __forceinline__ void store_staged(const uint8_t *lds, uint8_t *out, int seg_bytes,
                                             int lane)
{
    static_assert(OUT % 16 == 0, "whole 16-byte pieces");
#pragma unroll
    for (int k = 0; k < OUT / 16; ++k) {
        const int b = 1024 * k + 16 * lane;
        if (b < seg_bytes)
            __builtin_nontemporal_store(*(const u32x4_t *)(lds + b), (u32x4_t *)(out + b));
    }
}

// GREY (C = 3 or 4): each source pixel is converted to grey first and one
// byte per output pixel is stored; the 2:1 weights make the result the
// rounded mean of the four greys, as the general formula gives.
//
// One-wave workgroups, one output row segment at a time.  A lane's 16-byte
// result (C = 1, 4) is one lane-contiguous non-temporal store; narrower ones
// (RGB: 12 bytes) are stored as dwords with no hint.  Measured on the 4K RGB
// frame: staging the 12-byte results through LDS for whole-line
// non-temporal stores 6.7 -> 8.3 us, two or four waves per workgroup 6.7 ->
// 6.85 us, the non-temporal hint on the 12-byte stores 6.54 -> 6.74 us
// (though 5% faster on a 16 x 480x640 batch); non-temporal 16-byte stores
// for grey 4K -> 1080p 4.01 -> 3.88 us.
//
// Segment-major workgroups are one wave; row-major ones kHalfWaves waves,
// each wave with its own segment and LDS slot (no workgroup barrier).
// Row-major: a 1-D grid over the (row, segment) items of a pass of
// `pass_rows` output rows, wave w of workgroup b taking item
// kHalfWaves b' + w, where b' numbers the workgroups XCD-contiguously; a
// wave then steps by pass_rows rows while rows remain.
template <int C, bool GREY, bool SEG_MAJOR>
__global__ __launch_bounds__(kHalfLanes * kHalfWaves) void linear_half_u8(
    const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int dW, long long rows,
    DivBy by_segs, int segs, long long pass_rows)
{
    static_assert(!GREY || C >= 3, "grey needs RGB(A)");
    constexpr int PX = HalfShape<C>::PX;
    constexpr int SEG = kHalfLanes * PX;          // output pixels per segment
    constexpr int SRC_B = 2 * SEG * C;            // source bytes per row per segment
    constexpr int NL = (SRC_B / 16 + kHalfLanes - 1) / kHalfLanes;   // loads per lane per row
    constexpr int LB = 2 * PX * C;                // source bytes per lane per row
    constexpr int OC = GREY ? 1 : C;              // output channels
    constexpr int OB = PX * OC;                   // output bytes per lane
    constexpr int WAVES = SEG_MAJOR ? 1 : kHalfWaves;
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[WAVES][2 * SRC_B];

    const int lane = (int)threadIdx.x & (kHalfLanes - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kHalfLanes);
    uint8_t *const lds = lds_all[wave];
    int seg;
    long long g, g_step;
    if constexpr (SEG_MAJOR) {
        seg = blockIdx.y;
        g = blockIdx.x;
        g_step = gridDim.x;
    } else {
        // each XCD takes a contiguous run of (row, segment) items
        const unsigned item = xcd_contiguous(blockIdx.x, gridDim.x) * WAVES + wave;
        if (item >= (unsigned long long)pass_rows * segs) return;   // the last workgroup's spare wave
        const unsigned row = div_by(item, by_segs);
        seg = (int)(item - row * (unsigned)segs);
        g = row;
        g_step = pass_rows;
    }
    const int seg_px = min(SEG, dW - seg * SEG);
    const int n16 = seg_px * 2 * C / 16;          // whole: dW meets the divisibility rule
    const size_t src_row = (size_t)2 * dW * C;
    const size_t dst_row = (size_t)dW * OC;
    // One output row.  The grid's row extent never exceeds rows, so every
    // workgroup has a first row, taken before the loop: the loop's
    // pointer-step set-up (35 scalar instructions, which all resident waves
    // queue for on the CU's scalar unit) then comes after that row instead of
    // ahead of its loads, and the first loads issue at the 56th instruction
    // instead of past the 100th (4K RGB 6.39 -> 6.29 us, grey 3.57 -> 3.51,
    // 64 x 224x224 RGB 4.09 -> 3.94).
    auto do_row = [&](long long g) __attribute__((always_inline)) {
        const uint8_t *s0 = src + (size_t)(2 * g) * src_row + (size_t)seg * SRC_B;
        const uint8_t *s1 = s0 + src_row;
        uint4 va[NL], vb[NL];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int k = lane + kHalfLanes * i;
            if (k < n16) {
                va[i] = load_stream(s0 + 16 * k);
                vb[i] = load_stream(s1 + 16 * k);
            }
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int k = lane + kHalfLanes * i;
            if (k < n16) {
                *(uint4 *)(lds + 16 * k) = va[i];
                *(uint4 *)(lds + SRC_B + 16 * k) = vb[i];
            }
        }
        wave_sync();
        uint8_t r[OB];
        if (lane * PX < seg_px) {
            uint8_t a[LB], b[LB];
            __builtin_memcpy(a, lds + LB * lane, LB);
            __builtin_memcpy(b, lds + SRC_B + LB * lane, LB);
            if constexpr (GREY) {
#pragma unroll
                for (int k = 0; k < PX; ++k) {
                    const int p = 2 * k * C;      // first byte of source pixel 2k
                    const unsigned s4 = grey_u8(a[p], a[p + 1], a[p + 2]) +
                                        grey_u8(a[p + C], a[p + C + 1], a[p + C + 2]) +
                                        grey_u8(b[p], b[p + 1], b[p + 2]) +
                                        grey_u8(b[p + C], b[p + C + 1], b[p + C + 2]);
                    r[k] = (uint8_t)((s4 + 2u) >> 2);
                }
            } else {
                // output byte k = (a[p] + a[p + C] + b[p] + b[p + C] + 2) >> 2
                // with p = 2k - k % C, computed for pairs of output bytes,
                // one per 16-bit half: the four taps are picked as byte pairs
                // with v_perm_b32 (two bytes at most 4 apart lie in two
                // consecutive dwords) and added with v_pk_add_u16; the sum s
                // <= 1020 gives 64 s + 128 <= 65408, whose high byte is
                // (s + 2) >> 2.  About 40% fewer VALU ops than byte by byte
                // (4K -> 1080p RGB 6.61-6.80 -> 6.54-6.70 us, grey 3.81 ->
                // 3.59 us).
                typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
                uint32_t aw[LB / 4], bw[LB / 4], ow[OB / 4];
                __builtin_memcpy(aw, a, LB);
                __builtin_memcpy(bw, b, LB);
                auto pick = [&](const uint32_t (&w)[LB / 4], int i, int j) {
                    const int lo = (i < j ? i : j) / 4;
                    const int d = lo < LB / 4 - 2 ? lo : LB / 4 - 2;
                    return __builtin_bit_cast(
                        u16x2, __builtin_amdgcn_perm(w[d + 1], w[d],
                                                     0x0c000c00u | (uint32_t)(i - 4 * d) |
                                                         ((uint32_t)(j - 4 * d) << 16)));
                };
                u16x2 z[OB / 2];
#pragma unroll
                for (int h = 0; h < OB / 2; ++h) {
                    const int k = 2 * h;
                    const int p0 = 2 * k - k % C, p1 = 2 * (k + 1) - (k + 1) % C;
                    const u16x2 sum = pick(aw, p0, p1) + pick(aw, p0 + C, p1 + C) +
                                      pick(bw, p0, p1) + pick(bw, p0 + C, p1 + C);
                    z[h] = sum * (unsigned short)64 + (unsigned short)128;
                }
#pragma unroll
                for (int w = 0; w < OB / 4; ++w)
                    ow[w] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, z[2 * w + 1]),
                                                  __builtin_bit_cast(uint32_t, z[2 * w]),
                                                  0x07050301u);
                __builtin_memcpy(r, ow, OB);
            }
        }
        uint8_t *o = dst + (size_t)g * dst_row + (size_t)seg * SEG * OC + (size_t)lane * OB;
        if (lane * PX < seg_px) {
            if constexpr (OB % 16 == 0) {
#pragma unroll
                for (int k = 0; k < OB / 16; ++k) {
                    u32x4_t q;
                    __builtin_memcpy(&q, r + 16 * k, 16);
                    __builtin_nontemporal_store(q, (u32x4_t *)o + k);
                }
            } else {
#pragma unroll
                for (int k = 0; k < OB / 4; ++k) {
                    uint32_t q;
                    __builtin_memcpy(&q, r + 4 * k, 4);
                    ((uint32_t *)o)[k] = q;
                }
            }
        }
        wave_sync();
    };
    do_row(g);
    for (g += g_step; g < rows; g += g_step) do_row(g);
}

// --------------------------------------------------------------------------
// Exact 2x upscale of uint8 (dH = 2 H, dW = 2 W).  Output column 2k sits at
// source coordinate k - 1/4 and column 2k + 1 at k + 1/4, so the 11-bit
// weights are exactly 512 and 1536 and the general formula reduces, bit for
// bit, to (sum of k_ij p_ij + 8) >> 4 with k_ij in {9, 3, 3, 1}: a
// horizontal 1:3 or 3:1 sum h per source row, then (3 h_a + h_b + 8) >> 4
// down the column.  Edge taps clamp to the first / last pixel.
//
// Rows: a wave takes the gap g (-1 .. H - 1) between source rows g and
// g + 1 (clamped) and writes output rows 2g + 1 (3:1) and 2g + 2 (1:3), of
// which the first gap has only the second and the last only the first, so
// each source row is read by two waves, not three.
//
// Columns: a lane owns S source pixels (chunk m, IN = S C bytes) and writes
// the OUT = 2 IN output bytes [OUT m, OUT m + OUT) of both rows.  It loads
// the chunk as dwords with one dword of neighbours on each side (a copy of
// its own edge pixel where the row ends), so every tap is a constant byte
// position in that window.  Output bytes go in pairs (k, k + 1), one per
// 16-bit half: each output byte is 1 x one tap + 3 x another, so a pair is
// one v_pk_mad_u16 of two byte pairs picked with v_perm_b32 (any two bytes
// at most 4 apart lie in two consecutive dwords).  All sums stay below
// 2^16: h <= 1020 and 48 h_a + 16 h_b + 128 <= 65408, whose high byte is
// (3 h_a + h_b + 8) >> 4, so the rounding shift is a byte selection.
//
// Needs W % S == 0, W C % 16 == 0 and 16-byte aligned buffers.  Workgroup:
// RB waves, one gap each.  Grid: one dimension of gx * gy * gz workgroups,
// numbered XCD-contiguously and split into x = 64-chunk segment across a
// row (gx), y = group of RB gaps of an image (gy), z = image (stride gz).
// A 3-D grid of the same workgroups (x, y, z) dispatched slower: the
// 1080p grey frame 3.66 -> 3.47 us.  Stores are non-temporal (the output
// is not read back); chunks wider than 16 bytes per output row go out
// through LDS so that every store instruction covers whole cache lines.
// --------------------------------------------------------------------------
template <int C> struct Up2Shape { static constexpr int S = C == 4 ? 8 : 16; };
// source pixels per lane of the linear kernel
template <int C> struct Up2LinShape { static constexpr int S = C == 4 ? 4 : 8; };

// Byte position, in a lane's dword window, of the tap that output byte k of
// its chunk weights by 1 (W1) or by 3 (!W1).  Output byte k is channel k % C
// of output pixel q = k / C, which takes source pixel q / 2 with weight 3
// and its left (q even) or right (q odd) neighbour with weight 1; source
// pixel i (-1 .. S) channel c sits at 4 + i C + c.
template <int C, bool W1>
__host__ __device__ constexpr int up2_tap(int k)
{
    const int q = k / C, c = k % C, i = q / 2;
    return 4 + (W1 ? (q % 2 ? i + 1 : i - 1) : i) * C + c;
}

// Selector of __builtin_amdgcn_perm(e[d + 1], e[d], sel) that zero-extends
// window bytes a and b (both in dwords d, d + 1) into the low and high
// 16-bit halves.
__host__ __device__ constexpr uint32_t up2_pair_sel(int a, int b, int d)
{
    return 0x0c000c00u | (uint32_t)(a - 4 * d) | ((uint32_t)(b - 4 * d) << 16);
}

// Output byte pair (k, k + 1) of one row's taps of weight 1 (W1) or 3 from
// the ND-dword window e.  The two dwords start at the lower tap's dword,
// moved back one when that is the window's last.
template <int C, bool W1, int ND>
__device__ __forceinline__ uint32_t up2_pick(const uint32_t (&e)[ND], int k)
{
    // k is a compile-time constant after unrolling, so are d and the selector
    const int a = up2_tap<C, W1>(k), b = up2_tap<C, W1>(k + 1);
    const int lo = (a < b ? a : b) / 4;
    const int d = lo < ND - 2 ? lo : ND - 2;
    return __builtin_amdgcn_perm(e[d + 1], e[d], up2_pair_sel(a, b, d));
}

// One-channel rows on 4-byte dot products.  Output byte q of row 2g + 1
// or 2g + 2 is (9 t + 3 u + 3 v + w + 8) >> 4 over its four taps (the near
// and far column of the near and far row), the same sum as the packed form
// above; scaled by 16, with 128 added, it is below 2^16 and its byte 1 is
// the result.  Source pixels i and i + 1 (window bytes 4 + i, 5 + i) give
// one register (a_i, a_i+1, b_i, b_i+1) - one byte permute, or three where
// the pair straddles a dword - that serves output bytes 2i + 1 (i weighted
// 3, i + 1 weighted 1) and 2i + 2 (the other way round) of both rows: four
// weight vectors, 16 x (vertical x horizontal) weights on those bytes.
// Checked bit for bit against the oracle on the CPU before its first run.
template <int S, int ND>
__device__ __forceinline__ void up2_rows_c1(const uint32_t (&ea)[ND], const uint32_t (&eb)[ND],
                                            uint32_t (&oa)[S / 2], uint32_t (&ob)[S / 2])
{
    static_assert(ND == S / 4 + 2, "window of the lane's bytes and a dword each side");
    constexpr uint32_t kOddA = 0x10303090u, kOddB = 0x30901030u;    // q = 2i + 1
    constexpr uint32_t kEvenA = 0x30109030u, kEvenB = 0x90303010u;  // q = 2i + 2
    uint32_t G[S + 1];   // G[j]: source pixels j - 1 and j (window bytes 3 + j, 4 + j)
#pragma unroll
    for (int j = 0; j <= S; ++j) {
        const int lo = 3 + j, d = lo / 4, o = lo % 4;
        if (o != 3) {
            const uint32_t sel = (uint32_t)o | ((uint32_t)(o + 1) << 8) | ((uint32_t)(4 + o) << 16) |
                                 ((uint32_t)(5 + o) << 24);
            G[j] = __builtin_amdgcn_perm(eb[d], ea[d], sel);
        } else {
            const uint32_t sa = __builtin_amdgcn_alignbyte(ea[d + 1], ea[d], 3);
            const uint32_t sb = __builtin_amdgcn_alignbyte(eb[d + 1], eb[d], 3);
            G[j] = __builtin_amdgcn_perm(sb, sa, 0x05040100u);
        }
    }
    uint32_t ra[2 * S], rb[2 * S];
#pragma unroll
    for (int q = 0; q < 2 * S; ++q) {
        const int j = (q + 1) / 2;
        ra[q] = __builtin_amdgcn_udot4(G[j], q % 2 ? kOddA : kEvenA, 128u, false);
        rb[q] = __builtin_amdgcn_udot4(G[j], q % 2 ? kOddB : kEvenB, 128u, false);
    }
    // byte 1 of four results per output dword
#pragma unroll
    for (int w = 0; w < S / 2; ++w) {
        oa[w] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(ra[4 * w + 3], ra[4 * w + 2], 0x0c0c0501u),
                                      __builtin_amdgcn_perm(ra[4 * w + 1], ra[4 * w], 0x0c0c0501u),
                                      0x05040100u);
        ob[w] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(rb[4 * w + 3], rb[4 * w + 2], 0x0c0c0501u),
                                      __builtin_amdgcn_perm(rb[4 * w + 1], rb[4 * w], 0x0c0c0501u),
                                      0x05040100u);
    }
}

template <int C, int RB, bool ONE = false>
__global__ __launch_bounds__(64 * RB) void linear_up2_u8(
    const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int H, int W,
    int batch, int chunks_per_row, unsigned gx, unsigned gy, unsigned gz, DivBy by_gx,
    DivBy by_gy)
{
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    constexpr int S = Up2LinShape<C>::S;
    constexpr int IN = S * C;              // source bytes of a chunk
    constexpr int OUT = 2 * IN;            // output bytes of a chunk per row
    constexpr int NP = OUT / 2;            // output byte pairs per row
    constexpr int ND = IN / 4 + 2;         // window dwords
    static_assert(IN % 4 == 0 && OUT % 16 == 0 && C <= 4, "chunk shape");
    static_assert(up2_tap<C, true>(0) >= 4 - C && up2_tap<C, true>(OUT - 1) < 4 * ND,
                  "taps inside the window");
    constexpr bool STAGE = OUT > 16;       // wider chunks go out through LDS
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[STAGE ? RB * 2 * 64 * OUT : 16];
    const int lane = (int)threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    // (segment, gap group, image) of this workgroup, XCD-contiguous
    const unsigned wid = xcd_contiguous(blockIdx.x, gridDim.x);
    const unsigned yz = div_by(wid, by_gx);
    const unsigned bx = wid - yz * gx;
    const unsigned bz = ONE || gz == 1 ? 0u : div_by(yz, by_gy);
    const unsigned by = yz - bz * gy;
    const int m = bx * 64 + lane;
    const int g = (int)(by * RB + wave) - 1;   // gap, uniform across the wave
    const bool active = m < chunks_per_row;
    if (g >= H || (!STAGE && !active)) return;
    const size_t row_bytes = (size_t)W * C;
    const int ra = g > 0 ? g : 0, rb = g + 1 < H ? g + 1 : H - 1;
    const bool has_a = g >= 0, has_b = g + 1 < H;    // output rows 2g + 1, 2g + 2
    const bool left = m > 0, right = (m + 1) * S < W;
    // rows of two or more chunks hold IN + 8 bytes around every chunk
    const bool one_load = chunks_per_row >= 2;
    // The lane's source windows of both rows, each a dword window around
    // the lane's IN bytes with the edge pixel moved into a missing
    // neighbour.  Both rows' loads issue before the first wait: loading and
    // shifting each row in turn put the wait for row a's load, behind the
    // uniform branch on the window's shape, before row b's load was issued
    // (two memory round trips per wave).
    // one_load: the whole window in one load per row, [p - 4, p + IN + 4)
    // inside the row, [p, p + IN + 8) at its start and [p - 8, p + IN) at
    // its end, then shifted into place (one 16-byte load per row for C = 1
    // instead of three loads: 1080p grey 3.49 -> 3.42 us).  Otherwise a
    // one-chunk row: its bytes and its own edge dwords.
    auto windows = [&](const uint8_t *row_a, const uint8_t *row_b, uint32_t (&ea)[ND],
                       uint32_t (&eb)[ND]) {
        const uint8_t *pa = row_a + (size_t)m * IN, *pb = row_b + (size_t)m * IN;   // 4-byte aligned
        if (one_load) {
            const int sh = !left ? 0 : (!right ? -8 : -4);
            uint32_t A[ND], B[ND];
            __builtin_memcpy(A, __builtin_assume_aligned(pa + sh, 4), 4 * ND);
            __builtin_memcpy(B, __builtin_assume_aligned(pb + sh, 4), 4 * ND);
#pragma unroll
            for (int k = 0; k < ND; ++k) {
                const uint32_t a_m = A[k > 0 ? k - 1 : 0], a_0 = A[k], a_p = A[k < ND - 1 ? k + 1 : ND - 1];
                const uint32_t b_m = B[k > 0 ? k - 1 : 0], b_0 = B[k], b_p = B[k < ND - 1 ? k + 1 : ND - 1];
                ea[k] = !left ? a_m : (!right ? a_p : a_0);
                eb[k] = !left ? b_m : (!right ? b_p : b_0);
            }
            if (!left) {
                ea[0] = A[0] << (8 * (4 - C));
                eb[0] = B[0] << (8 * (4 - C));
            }
            if (!right) {
                ea[ND - 1] = A[ND - 1] >> (8 * (4 - C));
                eb[ND - 1] = B[ND - 1] >> (8 * (4 - C));
            }
        } else {
            uint32_t A[ND - 2], B[ND - 2];
            __builtin_memcpy(A, __builtin_assume_aligned(pa, IN % 16 == 0 ? 16 : 8), IN);
            __builtin_memcpy(B, __builtin_assume_aligned(pb, IN % 16 == 0 ? 16 : 8), IN);
            // both loads unconditional, so that all of them issue before the first wait
            const uint32_t lwa = *(const uint32_t *)pa, rwa = *(const uint32_t *)(pa + IN - 4);
            const uint32_t lwb = *(const uint32_t *)pb, rwb = *(const uint32_t *)(pb + IN - 4);
            // (element-wise: a memcpy into part of ea sent the windows to scratch)
#pragma unroll
            for (int k = 0; k < ND - 2; ++k) {
                ea[k + 1] = A[k];
                eb[k + 1] = B[k];
            }
            ea[0] = lwa << (8 * (4 - C));
            ea[ND - 1] = rwa >> (8 * (4 - C));
            eb[0] = lwb << (8 * (4 - C));
            eb[ND - 1] = rwb >> (8 * (4 - C));
        }
    };
    // horizontal sums of one source row's window, one u16x2 per output byte pair
    auto hsum = [&](const uint32_t (&e)[ND], u16x2 (&h)[NP]) {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const u16x2 u = __builtin_bit_cast(u16x2, up2_pick<C, true, ND>(e, 2 * j));
            const u16x2 v = __builtin_bit_cast(u16x2, up2_pick<C, false, ND>(e, 2 * j));
            h[j] = v * (unsigned short)3 + u;
        }
    };
    // high bytes of 48 h_x + 16 h_y + 128 for four output bytes
    auto vsum = [](const u16x2 (&hx)[NP], const u16x2 (&hy)[NP], int w) {
        const u16x2 z0 = hx[2 * w] * (unsigned short)48 +
                         (hy[2 * w] * (unsigned short)16 + (unsigned short)128);
        const u16x2 z1 = hx[2 * w + 1] * (unsigned short)48 +
                         (hy[2 * w + 1] * (unsigned short)16 + (unsigned short)128);
        return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, z1),
                                     __builtin_bit_cast(uint32_t, z0), 0x07050301u);
    };
    uint8_t *lds0 = lds_all + wave * 2 * 64 * OUT, *lds1 = lds0 + 64 * OUT;
    const int seg_bytes = min(64, chunks_per_row - (int)bx * 64) * OUT;
    // image n; the first runs ahead of the loop (see nearest_up2_u8)
    auto do_image = [&](int n) __attribute__((always_inline)) {
        const uint8_t *img = src + (size_t)n * H * row_bytes;
        // offset of output row 2g + 2 of image n; row 2g + 1 precedes it and
        // exists only when has_a, so its address is formed only then
        const size_t off_b = ((size_t)n * 2 * H + (size_t)(2 * g + 2)) * (2 * row_bytes) +
                          (size_t)bx * 64 * OUT;
        if (active) {
            uint32_t ea[ND], eb[ND];
            windows(img + (size_t)ra * row_bytes, img + (size_t)rb * row_bytes, ea, eb);
            uint32_t oa[OUT / 4], ob[OUT / 4];
            if constexpr (C == 1) {
                up2_rows_c1<S, ND>(ea, eb, oa, ob);
            } else {
                u16x2 ha[NP], hb[NP];
                hsum(ea, ha);
                hsum(eb, hb);
#pragma unroll
                for (int w = 0; w < OUT / 4; ++w) {
                    oa[w] = vsum(ha, hb, w);      // row 2g + 1: 3 x row g + row g + 1
                    ob[w] = vsum(hb, ha, w);      // row 2g + 2: row g + 3 x row g + 1
                }
            }
#pragma unroll
            for (int k = 0; k < OUT / 16; ++k) {
                const u32x4_t qa = {oa[4 * k], oa[4 * k + 1], oa[4 * k + 2], oa[4 * k + 3]};
                const u32x4_t qb = {ob[4 * k], ob[4 * k + 1], ob[4 * k + 2], ob[4 * k + 3]};
                if constexpr (STAGE) {
                    *(u32x4_t *)(lds0 + lane * OUT + 16 * k) = qa;
                    *(u32x4_t *)(lds1 + lane * OUT + 16 * k) = qb;
                } else {
                    // one 16-byte piece per lane and row: already lane-contiguous
                    if (has_a)
                        __builtin_nontemporal_store(
                            qa, (u32x4_t *)(dst + (off_b - 2 * row_bytes) + lane * OUT));
                    if (has_b) __builtin_nontemporal_store(qb, (u32x4_t *)(dst + off_b + lane * OUT));
                }
            }
        }
        if constexpr (STAGE) {
            wave_sync();
            if (has_a) store_staged<OUT>(lds0, dst + (off_b - 2 * row_bytes), seg_bytes, lane);
            if (has_b) store_staged<OUT>(lds1, dst + off_b, seg_bytes, lane);
            wave_sync();
        }
    };
    // bz < gz <= batch: every workgroup has a first image
    if constexpr (ONE) {
        do_image(0);
    } else {
        do_image((int)bz);
        for (int n = (int)bz + (int)gz; n < batch; n += gz) do_image(n);
    }
}

// --------------------------------------------------------------------------
// Exact 2x nearest upscale of uint8.  For dW = 2 W the rounded half-pixel
// coordinate of output column d is floor((2d + 1) / 4) = d / 2, so the
// output is every source pixel repeated twice in both directions.  A lane
// reads S pixels of source row j and writes them doubled to output rows 2j
// and 2j + 1.  Same shape rules, workgroup and stores as linear_up2_u8.
// Grid: x = 64-chunk segments, y = groups of RB rows of all N H source rows
// (strided past the grid's extent); SEG_MAJOR swaps the two.  The launcher
// takes SEG_MAJOR for rows of one segment (a grid 1 wide and thousands tall
// dispatches slowly: 64 x 112x112 grey 3.34 -> 2.86 us) and for two
// segments whose second is at most half full, which the round-robin spread
// of workgroups over the XCDs would hand to the same four XCDs (4 x 720p
// grey, 64 + 16 chunks: 4.83 -> 3.85 us).  Otherwise the plain order stays:
// with a nearly full second segment (1080p -> 4K RGB, 64 + 56 chunks) both
// the segment-major grid and the XCD-contiguous renumbering the linear
// kernel uses measured slower (5.69 -> 5.93 us).
// --------------------------------------------------------------------------
template <int C, int RB, bool SEG_MAJOR>
__global__ __launch_bounds__(64 * RB) void nearest_up2_u8(
    const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int W, long long rows,
    int chunks_per_row)
{
    constexpr int S = Up2Shape<C>::S;
    constexpr int IN = S * C;
    constexpr int OUT = 2 * S * C;
    // wider chunks go out through LDS; an unstaged chunk is one 16-byte piece
    constexpr bool STAGE = OUT > 16;
    static_assert(OUT % 16 == 0 && (STAGE || OUT == 16), "chunk shape");
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[STAGE ? RB * 64 * OUT : 16];
    const int lane = threadIdx.x;
    // (segment, row group) of this workgroup
    const unsigned bx = SEG_MAJOR ? blockIdx.y : blockIdx.x;
    const unsigned by = SEG_MAJOR ? blockIdx.x : blockIdx.y;
    const long long row_step = (long long)(SEG_MAJOR ? gridDim.x : gridDim.y) * RB;
    const int m = bx * 64 + lane;
    const bool active = m < chunks_per_row;
    if (!STAGE && !active) return;
    const size_t row_bytes = (size_t)W * C;
    uint8_t *lds = lds_all + threadIdx.y * 64 * OUT;
    const int seg_bytes = min(64, chunks_per_row - (int)bx * 64) * OUT;
    // t is uniform across the wave.  The first row runs ahead of the loop,
    // so the loop's pointer-step set-up does not delay its loads (as in the
    // 2:1 kernel).
    auto do_row = [&](long long t) __attribute__((always_inline)) {
        // source row t of the flattened N*H rows feeds output rows 2t, 2t + 1
        uint8_t *d0 = dst + (size_t)(2 * t) * (2 * row_bytes) + (size_t)bx * 64 * OUT;
        if (active) {
            // the chunk starts at m * IN bytes into a row of W C bytes (a
            // multiple of 16): aligned to 16 bytes, or to IN when IN < 16
            const uint8_t *row = src + (size_t)t * row_bytes + (size_t)m * IN;
            uint8_t in[IN], out[OUT];
            __builtin_memcpy(in, __builtin_assume_aligned(row, IN < 16 ? IN : 16), IN);
#pragma unroll
            for (int i = 0; i < S; ++i)
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    out[(2 * i) * C + c] = in[i * C + c];
                    out[(2 * i + 1) * C + c] = in[i * C + c];
                }
#pragma unroll
            for (int k = 0; k < OUT / 16; ++k) {
                u32x4_t q;
                __builtin_memcpy(&q, out + 16 * k, 16);
                if constexpr (STAGE) {
                    *(u32x4_t *)(lds + lane * OUT + 16 * k) = q;
                } else {
                    __builtin_nontemporal_store(q, (u32x4_t *)(d0 + lane * OUT));
                    __builtin_nontemporal_store(q, (u32x4_t *)(d0 + 2 * row_bytes + lane * OUT));
                }
            }
        }
        if constexpr (STAGE) {
            wave_sync();
            store_staged<OUT>(lds, d0, seg_bytes, lane);
            store_staged<OUT>(lds, d0 + 2 * row_bytes, seg_bytes, lane);
            wave_sync();
        }
    };
    long long t = (long long)by * RB + threadIdx.y;
    if (t >= rows) return;
    do_row(t);
    for (t += row_step; t < rows; t += row_step) do_row(t);
}

// --------------------------------------------------------------------------
// Nearest neighbour, any scale, any pixel size.  Same grid as
// linear_generic.  A pixel of BPP bytes moves in units of UNIT bytes
// (16, 4 or 1), chosen by the host from the pixel size and the alignment.
// --------------------------------------------------------------------------
template <int UNIT>
struct CopyUnit;
template <> struct CopyUnit<1>  { using type = uint8_t; };
template <> struct CopyUnit<4>  { using type = uint32_t; };
template <> struct CopyUnit<16> { using type = uint4; };

// Stores: a whole 4- or 16-byte pixel per lane is one lane-contiguous
// non-temporal store; STG (12-byte pixels, output rows 16-byte aligned)
// writes each wave's 64 pixels through LDS as lane-contiguous 16-byte
// non-temporal stores, as the linear direct kernel does for float RGB.
template <int BPP, int UNIT, bool STG = false>
__global__ __launch_bounds__(kBlock) void nearest_generic(
    const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int H, int W, int dH, int dW,
    long long rows_total, int rows_per_block, BandGrid bg, int map)
{
    using U = typename CopyUnit<UNIT>::type;
    constexpr int K = BPP / UNIT;
    static_assert(!STG || (BPP == 12 && UNIT == 4), "staged stores are for 12-byte pixels");
    __shared__ __attribute__((aligned(16))) uint8_t stage_all[STG ? kBlock * BPP : 16];
    long long rb;
    int cb;
    band_of_block(bg, rb, cb);
    const int wave_x0 = cb * kBlock + ((int)threadIdx.x & ~63);   // the wave's first column
    const int x_lane = cb * kBlock + (int)threadIdx.x;
    if (STG ? wave_x0 >= dW : x_lane >= dW) return;
    // lanes past the row end (staged form only) copy the last column, unstored
    const int x = STG ? min(x_lane, dW - 1) : x_lane;
    const size_t sx = (size_t)nearest_index(x, W, dW, map) * BPP;

    long long g = rb * rows_per_block;
    long long g_end = g + rows_per_block;
    if (g_end > rows_total) g_end = rows_total;
    long long n = image_of_row(g, dH, bg);
    int dy = (int)(g - n * dH);
    for (; g < g_end; ++g) {
        const int sy = nearest_index(dy, H, dH, map);
        const U *from = (const U *)(src + (((size_t)n * H + sy) * W) * BPP + sx);
        if constexpr (STG) {
            uint8_t *stage = stage_all + (threadIdx.x & ~63) * BPP;   // this wave's 64 pixels
#pragma unroll
            for (int k = 0; k < K; ++k) ((U *)(stage + (threadIdx.x & 63) * BPP))[k] = from[k];
            wave_sync();
            // the row segment's bytes: a multiple of 48 (dW % 4 == 0)
            const int seg_bytes = min(64, dW - wave_x0) * BPP;
            const int bb = 16 * (threadIdx.x & 63);
            if (bb < seg_bytes)
                __builtin_nontemporal_store(*(const u32x4_t *)(stage + bb),
                                            (u32x4_t *)(dst + ((size_t)g * dW + wave_x0) * BPP + bb));
            wave_sync();
        } else {
            U *to = (U *)(dst + ((size_t)g * dW + x) * BPP);
            if constexpr (K == 1 && UNIT >= 4 && kDirectNtStores) {
                if constexpr (UNIT == 16)
                    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, from[0]), (u32x4_t *)to);
                else
                    __builtin_nontemporal_store(from[0], to);
            } else {
#pragma unroll
                for (int k = 0; k < K; ++k) to[k] = from[k];
            }
        }
        if (++dy == dH) { dy = 0; ++n; }
    }
}

// --------------------------------------------------------------------------
// Row-segment kernel: any scale, linear or nearest, u8 or f32, C in {1,3,4}.
//
// A wave (64 lanes) owns a segment of 64 * PX consecutive output columns
// and a band of `rows_per_block` consecutive output rows; a workgroup packs
// kSegWaves such waves, each on its own band with its own LDS slots, so no
// workgroup-wide barrier is needed.  Each lane owns PX consecutive output
// pixels of the segment and keeps their column taps and weights in
// registers for the whole band.
//
// Per output row the wave stages the source row(s) it needs - only the
// columns [sa, sb] its segment touches - into LDS with 16-byte loads that
// are coalesced across lanes, then every lane gathers its taps from LDS
// (arbitrary, scale-dependent tap positions cost LDS reads instead of
// scattered global accesses), blends, and writes its PX * C elements with
// one or a few vector stores.  Both taps of one source row are adjacent, so
// one unaligned LDS read fetches them together.  Two LDS slots cache the
// last two staged source rows, so consecutive output rows that share a
// source row (every upscale) stage it once.
//
// The staging is pipelined one row deep (see issue_segment), and rows that
// no other output row needs are loaded and the results stored with
// non-temporal hints.
//
// Row taps advance incrementally from row to row: the numerator of the
// source coordinate grows by 2H per output row, so the quotient and
// remainder update with one compare instead of a division.
//
// The host sizes `seg_cap` (bytes per slot) for the widest segment plus
// misalignment and read slack, and uses this kernel only while 2 * seg_cap
// stays within its LDS budget; stronger downscales take the direct kernels.
// --------------------------------------------------------------------------
template <typename T, int C> struct SegShape;   // PX = output pixels per lane
// one-channel uint8: the launcher picks 16, 8 or 4 per output width
template <> struct SegShape<uint8_t, 1> { static constexpr int PX = 16; };
template <> struct SegShape<uint8_t, 3> { static constexpr int PX = 4; };
template <> struct SegShape<uint8_t, 4> { static constexpr int PX = 4; };
template <> struct SegShape<float, 1> { static constexpr int PX = 4; };
template <> struct SegShape<float, 3> { static constexpr int PX = 4; };
template <> struct SegShape<float, 4> { static constexpr int PX = 1; };

constexpr int kSegLanes = 64;
constexpr int kSegReadSlack = 16;  // bytes a two-tap LDS read may run past the segment
// Waves per row-segment workgroup.  Each wave works alone on a band of its
// own, with its own two LDS slots; packing several into one workgroup keeps
// the CU's workgroup slots from capping how many waves it holds.
constexpr int kSegWaves = 4;

__device__ __forceinline__ int seg_lane() { return (int)threadIdx.x & (kSegLanes - 1); }

// One source-row segment to stage: `bytes` bytes from p (uniform across the
// wave) into an LDS slot, as 16-byte chunks from the 16-byte boundary at or
// below p.  `clean` says every chunk lies wholly inside the source buffer
// [lo, hi); the caller decides it from the row (see rowseg), and segments
// that are not clean are staged with every chunk checked.
struct Segment {
    const uint8_t *base;   // 16-byte aligned address of chunk 0
    uint8_t *slot;
    int mis;               // offset of p inside the slot
    int n16;               // chunks to stage
    bool on;               // this row needs staging
    bool clean;
    __device__ void plan(bool want, uint8_t *slot_, const uint8_t *p, int bytes)
    {
        on = want;
        slot = slot_;
        mis = (int)((uintptr_t)p & 15);
        base = p - mis;
        n16 = (mis + bytes + 15) >> 4;
    }
};

// Staging of a segment that touches the start or end of the source buffer:
// chunks wholly inside are copied as 16 bytes, the others byte by byte, so
// nothing outside [lo, hi) is read.  Rare (at most the buffer's first and
// last rows), so its loops stay rolled: it sits behind a wave-uniform branch
// and costs nothing when not taken.
__device__ __forceinline__ void stage_edge_segment(const Segment &S, const uint8_t *lo,
                                                   const uint8_t *hi)
{
#pragma unroll 1
    for (int k = seg_lane(); k < S.n16; k += kSegLanes) {
        const uint8_t *q = S.base + 16 * k;
        if (q >= lo && q + 16 <= hi) {
            *(uint4 *)(S.slot + 16 * k) = *(const uint4 *)q;
        } else {
#pragma unroll 1
            for (int b = 0; b < 16; ++b)
                S.slot[16 * k + b] = (q + b >= lo && q + b < hi) ? q[b] : (uint8_t)0;
        }
    }
}

// Staging is software-pipelined one output row deep: the 16-byte chunks of
// the next row's segments are loaded into registers (issue_segment) before
// the current row is blended and stored, and written to LDS (commit_segment)
// at the top of the next iteration.  The wave therefore has the next row's
// loads in flight while it computes and stores, instead of waiting for
// memory once per row.  A lane handles chunks lane, lane + 64, ... (KMAX of
// them); a lane past the segment re-reads its last chunk and writes into
// the slot's slack (a slot holds 64 KMAX chunks), so the clean case has no
// divergent branches at all.
typedef unsigned int seg_v4u __attribute__((ext_vector_type(4)));

template <int KMAX, bool NT>
__device__ __forceinline__ void issue_segment(const Segment &S, seg_v4u (&v)[KMAX])
{
    if (S.on && S.clean) {
#pragma unroll
        for (int i = 0; i < KMAX; ++i) {
            // (uniform) a round of chunks wholly past the segment loads nothing
            if (kSegLanes * i < S.n16) {
                const int k = min(seg_lane() + kSegLanes * i, S.n16 - 1);
                const seg_v4u *q = (const seg_v4u *)(S.base + 16 * k);
                if constexpr (NT) v[i] = __builtin_nontemporal_load(q);
                else v[i] = *q;
            }
        }
    }
}

template <int KMAX>
__device__ __forceinline__ void commit_segment(const Segment &S, const seg_v4u (&v)[KMAX],
                                               const uint8_t *lo, const uint8_t *hi)
{
    if (S.on) {
        if (S.clean) {
#pragma unroll
            for (int i = 0; i < KMAX; ++i)
                if (kSegLanes * i < S.n16)
                    *(seg_v4u *)(S.slot + 16 * (seg_lane() + kSegLanes * i)) = v[i];
        } else {
            stage_edge_segment(S, lo, hi);
        }
    }
}

// LDS reads of a few bytes at any byte address.  Multi-byte LDS reads that
// are not naturally aligned run far slower than aligned ones (a 2x uint8
// upscale whose tap reads were unaligned dword reads took 36 us, the same
// kernel with byte reads 16.7 us), so these read the aligned dwords around
// the bytes and shift them into place.  They may read up to 3 bytes past
// the last byte asked for (inside a slot's read slack).
__device__ __forceinline__ uint32_t lds_bytes4(const uint8_t *p)
{
    const unsigned sh = (unsigned)(uintptr_t)p & 3u;
    const uint32_t *w = (const uint32_t *)__builtin_assume_aligned(p - sh, 4);
    return __builtin_amdgcn_alignbyte(w[1], w[0], sh);
}

__device__ __forceinline__ void lds_bytes8(const uint8_t *p, uint32_t &lo, uint32_t &hi)
{
    const unsigned sh = (unsigned)(uintptr_t)p & 3u;
    const uint32_t *w = (const uint32_t *)__builtin_assume_aligned(p - sh, 4);
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
    lo = __builtin_amdgcn_alignbyte(w1, w0, sh);
    hi = __builtin_amdgcn_alignbyte(w2, w1, sh);
}

// What one output row needs from the staging step: the segments to stage,
// where tap a of its two source rows sits in LDS, its row weight, and which
// output row it is.
struct RowPlan {
    Segment A, B;
    int la, lb;            // LDS byte offsets of column sa in the two source rows
    unsigned wy1;          // uint8 row weight (11-bit)
    float wyf;             // float row weight
    long long n;           // output image
    int dy;                // output row within the image
    const uint8_t *row_a, *row_b;   // start of the two source rows
};

// Store N elements of one lane: vectorised when the chunk is whole and
// aligned, element by element otherwise (row ends, odd pitches).  The
// stores are non-temporal: a resize writes its result once and never reads
// it back, so it should not displace cached source rows.
template <typename T, int N>
__device__ __forceinline__ void store_chunk(T *out, const T (&v)[N], int valid)
{
    constexpr int BYTES = N * (int)sizeof(T);
    if (valid == N && BYTES % 16 == 0 && ((uintptr_t)out & 15) == 0) {
#pragma unroll
        for (int k = 0; k < BYTES / 16; ++k) {
            u32x4_t q;
            __builtin_memcpy(&q, (const uint8_t *)v + 16 * k, 16);
            __builtin_nontemporal_store(q, (u32x4_t *)out + k);
        }
    } else if (valid == N && BYTES % 4 == 0 && ((uintptr_t)out & 3) == 0) {
#pragma unroll
        for (int k = 0; k < BYTES / 4; ++k) {
            uint32_t q;
            __builtin_memcpy(&q, (const uint8_t *)v + 4 * k, 4);
            __builtin_nontemporal_store(q, (uint32_t *)out + k);
        }
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k)
            if (k < valid) __builtin_nontemporal_store(v[k], out + k);
    }
}

// Half-pixel map of one axis that steps from one output index to the next
// without dividing (rows down a band, columns across a lane's pixels).
struct AxisStepper {
    // all below 2^18: q in [-1, n_in], r < den = 2 n_out <= 131070
    int q, r;              // floor and remainder of num / den for the current row
    int dq, dr;            // 2 n_in = dq * den + dr
    int den;
    __device__ void init(int d, int n_in, int n_out) { init_biased(d, n_in, n_out, n_in - n_out); }
    // numerator 2 d n_in + bias instead of (2d + 1) n_in - n_out (nearest
    // mappings; bias in [0, n_in + n_out])
    __device__ void init_biased(int d, int n_in, int n_out, int bias)
    {
        den = 2 * n_out;
        const QR m = map_divmod(2 * d, n_in, bias, den);
        q = m.q;
        r = m.r;
        const QR s = floor_divmod((float)(2 * n_in), (unsigned)(2 * n_in), den);
        dq = s.q;
        dr = s.r;
    }
    __device__ void next()
    {
        q += dq;
        r += dr;
        if (r >= den) { r -= den; q += 1; }
    }
};

// Taps of one axis under border rule B, from the floor q and remainder r of
// the exact coordinate num / den (an AxisStepper's state), n source pixels.
// Clamp: the edge pixel repeats.  Mirror: the coordinate is first reflected
// about the outermost pixel centres - in integers, so the remainder (and
// with it the weight) is that of the reflected coordinate.  Wrap: the taps
// stay unwrapped, a = q in [-1, n - 1] and b = a + 1 in [0, n]; the caller
// reads column -1 as n - 1 and column n as 0 (shifting a coordinate by a
// whole period leaves its remainder unchanged).
template <int B>
__device__ __forceinline__ void border_taps(int q, int r, int den, int n, int &a, int &b, int &rr)
{
    if constexpr (B == kBorderClamp) {
        a = min(max(q, 0), n - 1);
        b = min(max(q + 1, 0), n - 1);
        rr = r;
    } else if constexpr (B == kBorderMirror) {
        if (n == 1) {
            a = b = 0;
            rr = 0;
            return;
        }
        if (q < 0) {                                    // num < 0: num -> -num
            q = r == 0 ? -q : -q - 1;
            r = r == 0 ? 0 : den - r;
        } else if (q > n - 1 || (q == n - 1 && r > 0)) {  // num > (n - 1) den
            q = 2 * (n - 1) - q - (r > 0 ? 1 : 0);
            r = r > 0 ? den - r : 0;
        }
        a = q;
        b = min(q + 1, n - 1);
        rr = r;
    } else {
        a = q;
        b = q + 1;
        rr = r;
    }
}

constexpr bool kSegStageFloatRgb = true;
// Normalised NHWC output of the row-segment kernel: each lane's PX C floats
// would go out as strided 16-byte pieces, so where output rows start on
// 16-byte boundaries each wave's row segment goes through LDS (64 PX C
// floats per wave, after all waves' slots) and out as lane-contiguous
// 16-byte non-temporal stores.  Compile-time: only this output stage has
// the code and the LDS.
template <typename T, int C, int OUT, int PX = SegShape<T, C>::PX>
__host__ __device__ constexpr int seg_nhwc_stage_bytes()
{
    return OUT == kOutNormNHWC || (kSegStageFloatRgb && OUT == kOutSame && sizeof(T) == 4 && C == 3)
               ? kSegLanes * PX * C * 4
               : 0;
}
__host__ __device__ inline bool seg_nhwc_staged(const void *dst, int dW, int C)
{
    return ((uintptr_t)dst & 15) == 0 && ((size_t)dW * C * 4) % 16 == 0;
}

template <typename T, int C, bool NEAREST, int KMAX, bool NT, int OUT = kOutSame, bool ROI = false,
          int B = kBorderClamp, int PXO = 0>
__global__ __launch_bounds__(kSegLanes * kSegWaves) void rowseg(
    const T *__restrict__ src, void *__restrict__ dst_v, int H, int W, int dH, int dW,
    long long rows_total, int rows_per_block, int seg_cap, long long src_elems, Affine aff,
    const int32_t *__restrict__ rois, int nn_map)
{
    T *const dst = (T *)dst_v;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_all[];
    constexpr int PX = PXO ? PXO : SegShape<T, C>::PX;   // PXO: the launcher's choice
    constexpr int PB = C * (int)sizeof(T);        // bytes per pixel
    static_assert(B == kBorderClamp || (!NEAREST && !ROI && OUT == kOutSame),
                  "mirror / wrap borders are for the plain linear resize");
    static_assert(OUT != kOutGrey || (!NEAREST && C >= 3), "grey needs a linear RGB(A) resize");
    // Wrap stages each row with a one-pixel halo: column -1 (= W - 1) in
    // front of it, column W (= 0) behind it.  PAD bytes in front of the
    // staged chunks hold the first; the slot's slack the second.
    constexpr int PAD = B == kBorderWrap ? 16 : 0;
    const int slot_bytes = seg_cap + 2 * PAD;
    const int lane = seg_lane();
    // wave index, made visibly uniform so that all per-row planning stays scalar
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kSegLanes);
    uint8_t *const lds = lds_all + (size_t)wave * 2 * slot_bytes;   // this wave's two slots
    constexpr int NSTAGE = seg_nhwc_stage_bytes<T, C, OUT, PX>();
    [[maybe_unused]] const bool nstaged = NSTAGE > 0 && seg_nhwc_staged(dst_v, dW, C);
    [[maybe_unused]] uint8_t *const lds_n =
        lds_all + (size_t)kSegWaves * 2 * slot_bytes + (size_t)wave * NSTAGE;
    const int wx0 = blockIdx.x * kSegLanes * PX;  // first output column of the segment
    const int wx1 = min(wx0 + kSegLanes * PX, dW) - 1;
    const int x0 = wx0 + lane * PX;               // this lane's first output column
    const int valid_px = max(0, min(PX, dW - x0));

    // The segment's column table, built once by the workgroup's four waves
    // (whose bands share the segment) into LDS, one packed entry per output
    // column: (tap a's byte offset from column sa) << 13 | (tap b is the
    // next column) << 12 | the 11-bit weight, and for float the weight in a
    // second word.  Where lanes own PX >= 4 columns the build splits over all
    // 256 threads and takes a quarter of the per-lane work: thumb 49.0 ->
    // 47.3 us, 1080p -> 1620x2880 RGB 15.0 -> 14.5, 4K -> 1440x2560 RGB
    // 12.0 -> 11.5, 720p -> 1080p RGB 9.35 -> 8.96.  With one column per lane
    // (float RGBA) one wave builds it while three wait at the barrier
    // (rgbaf 153.2 -> 154.6 us), so each lane keeps its own table in
    // registers there, as crops do (their table changes with the image).
    constexpr bool LDS_TABLE = !ROI && PX >= 4;
    constexpr int TWORDS = sizeof(T) == 1 ? 1 : 2;
    uint32_t *const ctab = (uint32_t *)(lds_all + (size_t)kSegWaves * 2 * slot_bytes +
                                        (nstaged ? (size_t)kSegWaves * NSTAGE : 0));
    if constexpr (LDS_TABLE) {
        int sa0;   // seg_range's first column, for the whole image
        {
            if constexpr (B != kBorderClamp) {
                AxisStepper s0, s1;
                s0.init(wx0, W, dW);
                s1.init(wx1, W, dW);
                int a0, b0, a1, b1, r;
                border_taps<B>(s0.q, s0.r, s0.den, W, a0, b0, r);
                border_taps<B>(s1.q, s1.r, s1.den, W, a1, b1, r);
                sa0 = min(a0, a1);
            } else if constexpr (NEAREST) {
                sa0 = nearest_index(wx0, W, dW, nn_map);
            } else {
                sa0 = axis_tap(wx0, W, dW).a;
            }
        }
        // the columns past dW - 1 repeat the last one, as the lanes' own
        // tables do
        for (int j = threadIdx.x; j < kSegLanes * PX; j += kSegLanes * kSegWaves) {
            AxisStepper xs;
            xs.init_biased(min(wx0 + j, dW - 1), W, dW,
                           NEAREST ? nearest_bias(nn_map, W, dW) : W - dW);
            uint32_t e0, e1 = 0;
            if constexpr (NEAREST) {
                e0 = (uint32_t)((min(xs.q, W - 1) - sa0) * PB) << 13;
            } else {
                int a, b, rr;
                border_taps<B>(xs.q, xs.r, xs.den, W, a, b, rr);
                Tap t;
                t.r = rr;
                t.den = xs.den;
                e0 = ((uint32_t)((a - sa0) * PB) << 13) | ((uint32_t)(b != a) << 12);
                if constexpr (sizeof(T) == 1) e0 |= weight11(t);
                else e1 = __builtin_bit_cast(uint32_t, weightf(t));
            }
            ctab[j * TWORDS] = e0;
            if constexpr (TWORDS == 2) ctab[j * TWORDS + 1] = e1;
        }
        __syncthreads();
    }
    long long g = ((long long)blockIdx.y * kSegWaves + wave) * rows_per_block;
    if (g >= rows_total) return;                  // a band past the last row
    long long g_end = g + rows_per_block;
    if (g_end > rows_total) g_end = rows_total;
    const long long n0 = g / dH;

    // Source columns [sa, sb] of a crop (relative to its left edge) touched
    // by the segment's output columns.
    auto seg_range = [&](const Crop &c, int &sa, int &sb) {
        if constexpr (B != kBorderClamp) {
            // the taps of the first and last columns bound the segment's
            // (mirror reflects at most the outermost columns onto the edge
            // pixels; wrap's range is unwrapped, from -1 to W)
            AxisStepper s0, s1;
            s0.init(wx0, c.w, dW);
            s1.init(wx1, c.w, dW);
            int a0, b0, a1, b1, r;
            border_taps<B>(s0.q, s0.r, s0.den, c.w, a0, b0, r);
            border_taps<B>(s1.q, s1.r, s1.den, c.w, a1, b1, r);
            sa = min(a0, a1);
            sb = max(b0, b1);
        } else if constexpr (NEAREST) {
            sa = nearest_index(wx0, c.w, dW, nn_map);
            sb = nearest_index(wx1, c.w, dW, nn_map);
        } else {
            sa = axis_tap(wx0, c.w, dW).a;
            sb = axis_tap(wx1, c.w, dW).b;
        }
    };

    // This lane's column table: byte offset of tap a from column sa, whether
    // tap b is the next column (it is not only where both taps clamp to the
    // last column), and the weights: for uint8 the pair (2048 - u, u), or
    // (2048, 0) where tap b is tap a, for float u.  Recomputed when a crop changes
    // with the image.  The lane's first column is mapped with one division;
    // the next ones step from it exactly (the numerator grows by 2 n_in per
    // column), and columns past the last output column repeat it.
    int toff[PX];
    bool tnext[PX];
    uint32_t twp[PX];
    float twf[PX];
    auto lane_table = [&](const Crop &c, int sa) {
        AxisStepper xs;
        // nearest steps its own mapping's numerator, whose floor is the index
        xs.init_biased(min(x0, dW - 1), c.w, dW,
                       NEAREST ? nearest_bias(nn_map, c.w, dW) : c.w - dW);
        const int last = c.w - 1;
#pragma unroll
        for (int p = 0; p < PX; ++p) {
            if (p > 0 && x0 + p <= dW - 1) xs.next();
            if constexpr (NEAREST) {
                const int k = xs.q;
                toff[p] = (min(k, last) - sa) * PB;
                tnext[p] = false;
                twp[p] = 0;
                twf[p] = 0.f;
            } else {
                int a, b, rr;
                border_taps<B>(xs.q, xs.r, xs.den, c.w, a, b, rr);
                (void)last;
                toff[p] = (a - sa) * PB;
                tnext[p] = b != a;
                Tap t;
                t.r = rr;
                t.den = xs.den;
                if constexpr (sizeof(T) == 1) twp[p] = weight_pair(weight11(t), b != a);
                else twf[p] = weightf(t);
            }
        }
    };

    // The source region resized: the whole image, or image n's crop.
    Crop crop{0, 0, W, H};
    if constexpr (ROI) crop = load_crop(rois, n0, H, W);

    const uint8_t *lo = (const uint8_t *)src;
    const uint8_t *hi = lo + (size_t)src_elems * sizeof(T);
    const size_t row_bytes = (size_t)W * PB;
    const unsigned row_bytes32 = (unsigned)W * PB;   // below 2^20
    const size_t img_bytes = (size_t)H * row_bytes;
    T *const out_lane = dst + (size_t)x0 * C;

    // Planning state: the next output row to plan, its image's first source
    // row, its crop and segment.
    long long pn = n0;
    const uint8_t *pimg = lo + (size_t)n0 * img_bytes;
    int pdy = (int)(g - n0 * dH);
    int seg_sa;                      // first source column, relative to the crop
    int psa, pbytes;                 // first staged source column (absolute), bytes
    bool halo_l = false, halo_r = false;   // wrap: columns -1 and W are in the segment
    auto set_segment = [&]() {
        int sb;
        seg_range(crop, seg_sa, sb);
        if constexpr (B == kBorderWrap) {
            halo_l = seg_sa < 0;
            halo_r = sb > crop.w - 1;
            const int c0 = max(seg_sa, 0), c1 = min(sb, crop.w - 1);
            psa = c0 + crop.x;
            pbytes = (c1 - c0 + 1) * PB;
        } else {
            psa = seg_sa + crop.x;
            pbytes = (sb - seg_sa + 1) * PB;
        }
    };
    set_segment();
    AxisStepper ys;
    auto row_init = [&](int d) {
        ys.init_biased(d, crop.h, dH, NEAREST ? nearest_bias(nn_map, crop.h, dH) : crop.h - dH);
    };
    row_init(pdy);
    // source row (its first byte) held in each LDS slot, and its offset there
    const uint8_t *held0 = nullptr, *held1 = nullptr;
    int mis0 = 0, mis1 = 0;

    // Whether the 16-byte chunks of a segment of `row` (source rows lie
    // row_bytes apart from lo) stay inside [lo, hi).  For rows of 16 bytes
    // or more, a row after the first starts at least 16 bytes past lo, so a
    // chunk there (at most 15 bytes before the segment) starts at or after
    // lo; a row before the last ends at least 16 bytes before hi, so a chunk
    // there (at most 15 bytes past the segment) ends at or before hi.  The
    // first and last rows are checked exactly whenever the segment's columns
    // change, and kept as lo_bad / last_bad where their chunks leave the
    // buffer (null otherwise).  Narrower rows are always staged with checks.
    const uint8_t *const last_row = hi - row_bytes;
    const bool wide_rows = row_bytes >= 16;
    const uint8_t *lo_bad = nullptr, *last_bad = nullptr;
    auto edge_rows = [&]() {
        auto leaves = [&](const uint8_t *row) {
            const uint8_t *p = row + (size_t)psa * PB;
            const int mis = (int)((uintptr_t)p & 15);
            const uint8_t *b = p - mis;
            return b < lo || b + 16 * (size_t)((mis + pbytes + 15) >> 4) > hi;
        };
        lo_bad = leaves(lo) ? lo : nullptr;
        last_bad = leaves(last_row) ? last_row : nullptr;
    };
    edge_rows();
    auto chunks_inside = [&](const uint8_t *row) {
        return wide_rows && row != lo_bad && row != last_bad;
    };
    // Choose the source rows, weights and LDS slots of the planned row; the
    // slots are claimed now, their contents land at the next commit.
    auto plan_row = [&](RowPlan &P) {
        int ya, yb;
        P.wy1 = 0;
        P.wyf = 0.f;
        const int Hc = crop.h;
        if constexpr (B != kBorderClamp) {
            int qa, qb, rr;
            border_taps<B>(ys.q, ys.r, ys.den, Hc, qa, qb, rr);
            ya = qa < 0 ? qa + Hc : qa;               // wrap: row -1 is row H - 1
            yb = qb > Hc - 1 ? qb - Hc : qb;          // wrap: row H is row 0
            Tap t;
            t.r = rr;
            t.den = ys.den;
            if constexpr (sizeof(T) == 1) P.wy1 = weight11(t);
            else P.wyf = weightf(t);
        } else if constexpr (NEAREST) {
            const int k = ys.q;          // the mapping's floor (non-negative)
            ya = yb = k > Hc - 1 ? Hc - 1 : (k < 0 ? 0 : k);
        } else {
            const int q = ys.q;
            ya = q < 0 ? 0 : (q > Hc - 1 ? Hc - 1 : q);
            yb = q + 1 < 0 ? 0 : (q + 1 > Hc - 1 ? Hc - 1 : q + 1);
            Tap t;
            t.r = ys.r;
            t.den = ys.den;
            if constexpr (sizeof(T) == 1) P.wy1 = weight11(t);
            else P.wyf = weightf(t);
        }
        // rows within the image: one 32 x 32 -> 64-bit product each
        const uint8_t *ra = pimg + (size_t)((unsigned)(crop.y + ya)) * row_bytes32;
        const uint8_t *rb = pimg + (size_t)((unsigned)(crop.y + yb)) * row_bytes32;
        int sa_slot = held0 == ra ? 0 : (held1 == ra ? 1 : -1);
        int sb_slot = held0 == rb ? 0 : (held1 == rb ? 1 : -1);
        const bool need_a = sa_slot < 0;
        if (need_a) sa_slot = (sb_slot == 0) ? 1 : 0;
        if (rb == ra) sb_slot = sa_slot;
        const bool need_b = sb_slot < 0;
        if (need_b) sb_slot = 1 - sa_slot;
        P.A.plan(need_a, lds + sa_slot * slot_bytes + PAD, ra + (size_t)psa * PB, pbytes);
        P.B.plan(need_b, lds + sb_slot * slot_bytes + PAD, rb + (size_t)psa * PB, pbytes);
        P.A.clean = chunks_inside(ra);
        P.B.clean = chunks_inside(rb);
        P.row_a = ra;
        P.row_b = rb;
        if (need_a) {
            if (sa_slot == 0) { held0 = ra; mis0 = P.A.mis; } else { held1 = ra; mis1 = P.A.mis; }
        }
        if (need_b) {
            if (sb_slot == 0) { held0 = rb; mis0 = P.B.mis; } else { held1 = rb; mis1 = P.B.mis; }
        }
        // LDS offset of column sa: the staged bytes start at column psa
        const int front = B == kBorderWrap && halo_l ? PB : 0;
        P.la = sa_slot * slot_bytes + PAD + (sa_slot == 0 ? mis0 : mis1) - front;
        P.lb = sb_slot * slot_bytes + PAD + (sb_slot == 0 ? mis0 : mis1) - front;
        P.n = pn;
        P.dy = pdy;
    };
    // Step the planning state to the next output row.
    auto advance = [&]() {
        if (++pdy == dH) {
            pdy = 0;
            ++pn;
            pimg += img_bytes;
            if constexpr (ROI) {
                crop = load_crop(rois, pn, H, W);
                set_segment();
                edge_rows();
            }
            row_init(0);
        } else {
            ys.next();
        }
    };

    // Wrap halo bytes: lanes 0 .. PB-1 carry column W - 1 of a staged row,
    // lanes 32 .. 32+PB-1 its column 0; loaded with the row, written after it.
    const bool halo_lane = (lane < PB && halo_l) || (lane >= 32 && lane < 32 + PB && halo_r);
    auto halo_load = [&](const Segment &S, const uint8_t *row) -> unsigned {
        if constexpr (B == kBorderWrap) {
            if (S.on && halo_lane)
                return lane < 32 ? row[(size_t)(W - 1) * PB + lane] : row[lane - 32];
        }
        return 0;
    };
    auto halo_store = [&](const Segment &S, unsigned v) {
        if constexpr (B == kBorderWrap) {
            if (S.on && halo_lane) {
                if (lane < 32) S.slot[S.mis - PB + lane] = (uint8_t)v;
                else S.slot[S.mis + pbytes + lane - 32] = (uint8_t)v;
            }
        }
    };

    seg_v4u va[KMAX], vb[KMAX];
    unsigned ha = 0, hb = 0;
    RowPlan P;
    plan_row(P);
    issue_segment<KMAX, NT>(P.A, va);
    issue_segment<KMAX, NT>(P.B, vb);
    if constexpr (B == kBorderWrap) {
        ha = halo_load(P.A, P.row_a);
        hb = halo_load(P.B, P.row_b);
    }
    // the lanes' column table (one division per lane) is built while the
    // band's first rows load: nothing before the first commit reads it
    if constexpr (LDS_TABLE) {
#pragma unroll
        for (int p = 0; p < PX; ++p) {
            const uint32_t e0 = ctab[(lane * PX + p) * TWORDS];
            toff[p] = (int)(e0 >> 13);
            tnext[p] = (e0 >> 12) & 1u;
            twp[p] = weight_pair(e0 & 4095u, (e0 >> 12) & 1u);
            if constexpr (TWORDS == 2) twf[p] = __builtin_bit_cast(float, ctab[(lane * PX + p) * TWORDS + 1]);
        }
    } else {
        lane_table(crop, seg_sa);
    }

    // uint8 RGB(A) -> grey resizes whose output rows share source rows
    // (staging loads cached, NT false: a row step below 2) keep each source
    // row's horizontal sums of grey values for as long as the row is in
    // use: a row that repeats from one output row to the next is neither
    // converted nor blended again, and each output row costs one vertical
    // multiply-add pair per pixel.  The arithmetic is that of
    // blend_u8_pairs.  The sums are keyed by the source row's address, and
    // a lane's column table changes only with the image, whose rows have
    // other addresses.  (1080p RGB -> grey 1620x2880: 16.0 -> 13.7 us.  The
    // same for colour output held 12-16 more VGPRs per lane and lost:
    // 4K -> 1440x2560 RGB 11.7 -> 15.0 us, crops 38.8 -> 41.1.)
    constexpr bool HSEP = sizeof(T) == 1 && !NEAREST && C >= 3 && !NT && OUT == kOutGrey;
    constexpr int NH = HSEP ? (OUT == kOutGrey ? PX : PX * C) : 1;
    [[maybe_unused]] uint32_t hA[NH], hB[NH];
    [[maybe_unused]] const uint8_t *hrow_a = nullptr, *hrow_b = nullptr;
    [[maybe_unused]] auto hrow = [&](const uint8_t *l, uint32_t (&h)[NH]) __attribute__((always_inline)) {
        if constexpr (HSEP) {
#pragma unroll
            for (int p = 0; p < PX; ++p) {
                // tap a = bytes [0, C), tap b = bytes [C, 2C); where tap b is
                // not the next column its weight is 0 (see blend_u8_pairs)
                uint32_t w_lo, w_hi;
                lds_bytes8(l + toff[p], w_lo, w_hi);
                if constexpr (OUT == kOutGrey) {
                    auto gr = [](uint32_t w) {
                        return grey_u8(w & 255u, (w >> 8) & 255u, (w >> 16) & 255u);
                    };
                    const uint32_t w2 = C == 4 ? w_hi : __builtin_amdgcn_alignbyte(w_hi, w_lo, C);
                    h[p] = row_sum_u8(gr(w_lo) | (gr(w2) << 16), twp[p]);
                } else {
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        const uint32_t sel = 0x0c000c00u | ((uint32_t)(C + c) << 16) | (uint32_t)c;
                        h[p * C + c] = row_sum_u8(__builtin_amdgcn_perm(w_hi, w_lo, sel), twp[p]);
                    }
                }
            }
        }
    };

    for (; g < g_end; ++g) {
        commit_segment<KMAX>(P.A, va, lo, hi);
        commit_segment<KMAX>(P.B, vb, lo, hi);
        if constexpr (B == kBorderWrap) {
            halo_store(P.A, ha);
            halo_store(P.B, hb);
        }
        wave_sync();

        const uint8_t *la = lds + P.la;
        const uint8_t *lb = lds + P.lb;
        [[maybe_unused]] const uint8_t *cur_a = P.row_a, *cur_b = P.row_b;
        const unsigned wy1 = P.wy1;
        const float wyf = P.wyf;
        const long long n = P.n;
        const int dy = P.dy;
        const bool more = g + 1 < g_end;
        if (more) {
            advance();
            plan_row(P);
            issue_segment<KMAX, NT>(P.A, va);
            issue_segment<KMAX, NT>(P.B, vb);
            if constexpr (B == kBorderWrap) {
                ha = halo_load(P.A, P.row_a);
                hb = halo_load(P.B, P.row_b);
            }
        }

        T res[PX * C];
        T resg[PX];                   // kOutGrey: one grey value per pixel
        // uint8 linear: each result in bits 24..31 of a word (blend_u8_pairs)
        constexpr bool U8LIN = sizeof(T) == 1 && !NEAREST;
        static_assert(!U8LIN || (PX * C) % 4 == 0, "whole words of results");
        [[maybe_unused]] uint32_t fx[U8LIN ? (OUT == kOutGrey ? PX : PX * C) : 1];
        [[maybe_unused]] const uint32_t wy0x4 = (2048u - wy1) << 2, wy1x4 = wy1 << 2;
        if constexpr (HSEP) {
            // new rows blended, repeated ones kept (uniform branches)
            if (cur_a != hrow_a) {
                if (cur_a == hrow_b) {
#pragma unroll
                    for (int k = 0; k < NH; ++k) hA[k] = hB[k];
                } else {
                    hrow(la, hA);
                }
            }
            if (cur_b == cur_a) {
#pragma unroll
                for (int k = 0; k < NH; ++k) hB[k] = hA[k];
            } else if (cur_b != hrow_b) {
                hrow(lb, hB);
            }
            hrow_a = cur_a;
            hrow_b = cur_b;
#pragma unroll
            for (int k = 0; k < NH; ++k) fx[k] = col_sum_u8(hA[k], hB[k], wy0x4, wy1x4);
        }
#pragma unroll
        for (int p = 0; p < PX && !HSEP; ++p) {
            if constexpr (NEAREST) {
                // one pixel, read with aligned accesses (see lds_bytes4)
                T v[C];
                if constexpr (sizeof(T) == 1 && C > 1) {
                    // bytes by shifts: a 3-byte memcpy out of the word went
                    // through scratch memory on every pixel
                    const uint32_t w = lds_bytes4(la + toff[p]);
#pragma unroll
                    for (int c = 0; c < C; ++c) v[c] = (T)(w >> (8 * c));
                } else if constexpr (sizeof(T) == 1 || PB % 16 == 0) {
                    __builtin_memcpy(v, la + toff[p], PB);
                } else {
                    __builtin_memcpy(v, __builtin_assume_aligned(la + toff[p], 4), PB);
                }
#pragma unroll
                for (int c = 0; c < C; ++c) res[p * C + c] = v[c];
            } else {
                // both taps of a row in one read: tap a at [0, PB), tap b at
                // [PB, 2 PB); uint8 taps come in one 4- or 8-byte word so the
                // read issues as a single (unaligned) LDS access.
                if constexpr (sizeof(T) == 1) {
                    // Each channel's two taps of a row as the 16-bit halves
                    // of one register (blend_u8_pairs).  Where tap b is not
                    // the next column its weight is 0, so the byte read
                    // there (inside the slot's read slack) does not count.
                    uint32_t pa[OUT == kOutGrey ? 1 : C], pb[OUT == kOutGrey ? 1 : C];
                    if constexpr (C == 1) {
                        // two byte reads beat one shifted dword pair here
                        const uint8_t *qa = la + toff[p], *qb = lb + toff[p];
                        pa[0] = (uint32_t)qa[0] | ((uint32_t)qa[1] << 16);
                        pb[0] = (uint32_t)qb[0] | ((uint32_t)qb[1] << 16);
                    } else {
                        // tap a = bytes [0, C), tap b = bytes [C, 2C)
                        uint32_t a_lo, a_hi, b_lo, b_hi;
                        lds_bytes8(la + toff[p], a_lo, a_hi);
                        lds_bytes8(lb + toff[p], b_lo, b_hi);
                        if constexpr (OUT == kOutGrey) {
                            auto gr = [](uint32_t w) {
                                return grey_u8(w & 255u, (w >> 8) & 255u, (w >> 16) & 255u);
                            };
                            const uint32_t a2 = C == 4 ? a_hi : __builtin_amdgcn_alignbyte(a_hi, a_lo, C);
                            const uint32_t b2 = C == 4 ? b_hi : __builtin_amdgcn_alignbyte(b_hi, b_lo, C);
                            pa[0] = gr(a_lo) | (gr(a2) << 16);
                            pb[0] = gr(b_lo) | (gr(b2) << 16);
                        } else {
#pragma unroll
                            for (int c = 0; c < C; ++c) {
                                // bytes c and C + c to the two halves
                                const uint32_t sel = 0x0c000c00u | ((uint32_t)(C + c) << 16) | (uint32_t)c;
                                pa[c] = __builtin_amdgcn_perm(a_hi, a_lo, sel);
                                pb[c] = __builtin_amdgcn_perm(b_hi, b_lo, sel);
                            }
                        }
                    }
                    if constexpr (OUT == kOutGrey) {
                        fx[p] = blend_u8_pairs(pa[0], pb[0], twp[p], wy0x4, wy1x4);
                    } else {
#pragma unroll
                        for (int c = 0; c < C; ++c)
                            fx[p * C + c] = blend_u8_pairs(pa[c], pb[c], twp[p], wy0x4, wy1x4);
                    }
                } else {
                    // float taps sit at 4-byte aligned LDS addresses (the
                    // source is 4-byte aligned and so is every pixel), which
                    // lets C = 1 and 3 read dword pairs.  RGBA pixels are
                    // 16 bytes and, with a 16-byte aligned source (the usual
                    // case), 16-byte aligned, so they keep 16-byte reads.
                    T ra2[2 * C], rb2[2 * C];
                    if constexpr (PB % 16 == 0) {
                        __builtin_memcpy(ra2, la + toff[p], 2 * PB);
                        __builtin_memcpy(rb2, lb + toff[p], 2 * PB);
                    } else {
                        __builtin_memcpy(ra2, __builtin_assume_aligned(la + toff[p], 4), 2 * PB);
                        __builtin_memcpy(rb2, __builtin_assume_aligned(lb + toff[p], 4), 2 * PB);
                    }
                    if constexpr (OUT == kOutGrey) {
                        const float a0 = grey_f32(ra2[0], ra2[1], ra2[2]);
                        const float b0 = grey_f32(rb2[0], rb2[1], rb2[2]);
                        const float a1 = tnext[p] ? grey_f32(ra2[C], ra2[C + 1], ra2[C + 2]) : a0;
                        const float b1 = tnext[p] ? grey_f32(rb2[C], rb2[C + 1], rb2[C + 2]) : b0;
                        resg[p] = blend_f32(a0, a1, b0, b1, twf[p], wyf);
                    } else {
#pragma unroll
                        for (int c = 0; c < C; ++c) {
                            const T a0 = ra2[c], a1 = tnext[p] ? ra2[C + c] : ra2[c];
                            const T b0 = rb2[c], b1 = tnext[p] ? rb2[C + c] : rb2[c];
                            res[p * C + c] = blend_f32(a0, a1, b0, b1, twf[p], wyf);
                        }
                    }
                }
            }
        }
        if constexpr (U8LIN && OUT == kOutSame) {
            uint32_t wds[PX * C / 4];
#pragma unroll
            for (int k = 0; k < PX * C / 4; ++k)
                wds[k] = pack_byte3(fx[4 * k], fx[4 * k + 1], fx[4 * k + 2], fx[4 * k + 3]);
            __builtin_memcpy(res, wds, sizeof(wds));
        } else if constexpr (U8LIN && OUT == kOutGrey) {
#pragma unroll
            for (int p = 0; p < PX; ++p) resg[p] = (T)(fx[p] >> 24);
        }
        if (valid_px > 0) {
            if constexpr (OUT == kOutSame && NSTAGE > 0) {
                if (nstaged) {
#pragma unroll
                    for (int k = 0; k < PX * C / 4; ++k) {
                        u32x4_t q;
                        __builtin_memcpy(&q, (const float *)res + 4 * k, 16);
                        *(u32x4_t *)(lds_n + lane * PX * C * 4 + 16 * k) = q;
                    }
                } else {
                    store_chunk<T, PX * C>(out_lane + (size_t)g * dW * C, res, valid_px * C);
                }
            } else if constexpr (OUT == kOutSame) {
                store_chunk<T, PX * C>(out_lane + (size_t)g * dW * C, res, valid_px * C);
            } else if constexpr (OUT == kOutGrey) {
                store_chunk<T, PX>(dst + (size_t)g * dW + x0, resg, valid_px);
            } else {
                float f[PX * C];
#pragma unroll
                for (int k = 0; k < PX * C; ++k) {
                    float v;
                    if constexpr (U8LIN) v = (float)(fx[k] >> 24);   // byte 3, converted directly
                    else v = (float)res[k];
                    f[k] = fmaf(v, aff.scale[k % C], aff.bias[k % C]);
                }
                float *dstf = (float *)dst_v;
                if constexpr (OUT == kOutNormNHWC) {
                    if (nstaged) {
#pragma unroll
                        for (int k = 0; k < PX * C / 4; ++k) {
                            u32x4_t q;
                            __builtin_memcpy(&q, f + 4 * k, 16);
                            *(u32x4_t *)(lds_n + lane * PX * C * 4 + 16 * k) = q;
                        }
                    } else {
                        store_chunk<float, PX * C>(dstf + ((size_t)g * dW + x0) * C, f,
                                                   valid_px * C);
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        float plane[PX];
#pragma unroll
                        for (int p = 0; p < PX; ++p) plane[p] = f[p * C + c];
                        store_chunk<float, PX>(dstf + (((size_t)n * C + c) * dH + dy) * dW + x0,
                                               plane, valid_px);
                    }
                }
            }
        }
        if constexpr (NSTAGE > 0) {
            if (nstaged) {
                // the segment's bytes: a multiple of 16, since dW C 4 and
                // the segment's start both are
                wave_sync();
                const int seg_bytes = (wx1 - wx0 + 1) * C * 4;
                uint8_t *o = (uint8_t *)((float *)dst_v + ((size_t)g * dW + wx0) * C);
#pragma unroll
                for (int k = 0; k < (NSTAGE + 1023) / 1024; ++k) {
                    const int bb = 1024 * k + 16 * lane;
                    if (bb < seg_bytes)
                        __builtin_nontemporal_store(*(const u32x4_t *)(lds_n + bb),
                                                    (u32x4_t *)(o + bb));
                }
            }
        }
        // the next image's crop changes this lane's column table
        if constexpr (ROI) {
            if (more && P.n != n) lane_table(crop, seg_sa);
        }
        // the compute above reads the LDS slots the next commit may overwrite
        wave_sync();
    }
}

// --------------------------------------------------------------------------
// Row enlargements of uint8 images by 2-D tiles (linear, clamp, plain output).
//
// A workgroup takes TH consecutive output rows of one image and the 64 PX
// output columns of one segment.  Every source row those rows touch - at
// most (TH - 1) H / dH + 3 of them, since the row step is below one - is
// staged over the segment's source columns into LDS at once, so all of the
// tile's 16-byte loads are in flight together; after one barrier the four
// waves blend TH / 4 rows each from LDS.  The row-segment kernel walks a
// band with one row of loads in flight, and an enlargement leaves each of
// its waves so few rows that the chain of round trips per band, not
// bandwidth or instruction issue, sets the time there.
//
// The column table (tap a's byte offset from column sa << 13, the
// next-column flag << 12, the 11-bit weight) is built into LDS by all
// threads, as in rowseg, and the blend is blend_u8_pairs: the results are
// those of every other kernel, bit for bit.
// --------------------------------------------------------------------------
constexpr int kTileWaves = 4;

// The launch's tile geometry (host-computed).
struct TileGeom {
    int tiles_x;           // column segments of 64 PX output columns per row
    int tiles_y;           // row tiles of TH output rows per image
    FastDiv by_tiles_x, by_tiles_y, by_n16;
    int n16cap;            // 16-byte chunks staged per source row, at most
    int pitch;             // LDS bytes per staged row: 16 (n16cap + 1)
};

// Stages a tile's nr source rows into LDS, row k at rows + k tg.pitch: the
// row's first needed byte is p0 + k row_bytes, at offset (mis0 + k rstep)
// mod 16 in its 16-byte chunk, and the row's chunks from that boundary on
// (tg.n16cap of them) are copied whole.
template <int KL>
__device__ __forceinline__ void tile_stage(uint8_t *rows, const uint8_t *p0, unsigned mis0,
                                           unsigned rstep, size_t row_bytes, int nr,
                                           const TileGeom &tg, const uint8_t *lo,
                                           const uint8_t *hi)
{
    // Stage: chunk i = k n16cap + j is chunk j of staged row k, from the
    // 16-byte boundary at or below the row's first needed byte.  A row's
    // chunks end at most 16 n16cap bytes past that boundary, so unless the
    // tile holds the buffer's first or last rows every chunk lies inside
    // the source buffer.  Then the chunks go in rounds of KL per thread,
    // each round's loads all issued before its LDS writes, with no divergent
    // branch: a lane past the last chunk repeats it (the same bytes to the
    // same place), and a round wholly past the tile is skipped (a uniform
    // test, so a launch sized for its largest tile costs smaller ones
    // nothing).  Tiles at the buffer's ends stage chunk by chunk, and a
    // chunk that leaves the buffer byte by byte with checks.
    constexpr int NT = 64 * kTileWaves;
    const int tid = (int)threadIdx.x;
    const int total = nr * tg.n16cap;
    auto chunk = [&](int i, const uint8_t *&q, int &off) {
        const int k = (int)fast_div((unsigned)i, tg.by_n16);
        const int j = i - k * tg.n16cap;
        const unsigned mis = (mis0 + (unsigned)k * rstep) & 15u;
        q = p0 + (size_t)k * row_bytes - mis + 16 * j;
        off = k * tg.pitch + 16 * j;
    };
    const unsigned mis_last = (mis0 + (unsigned)(nr - 1) * rstep) & 15u;
    const bool inside = p0 - mis0 >= lo &&
                        p0 + (size_t)(nr - 1) * row_bytes - mis_last + 16 * (size_t)tg.n16cap <= hi;
    if (inside) {
#pragma unroll 1
        for (int base = 0; base < total; base += KL * NT) {
            u32x4_t v[KL];
            int loff[KL];
#pragma unroll
            for (int t = 0; t < KL; ++t) {
                if (base + t * NT < total) {
                    const uint8_t *q;
                    chunk(min(base + tid + t * NT, total - 1), q, loff[t]);
                    v[t] = *(const u32x4_t *)q;
                }
            }
#pragma unroll
            for (int t = 0; t < KL; ++t)
                if (base + t * NT < total) *(u32x4_t *)(rows + loff[t]) = v[t];
        }
    } else {
#pragma unroll 1
        for (int i = tid; i < total; i += NT) {
            const uint8_t *q;
            int off;
            chunk(i, q, off);
            if (q >= lo && q + 16 <= hi) {
                *(u32x4_t *)(rows + off) = *(const u32x4_t *)q;
            } else {
#pragma unroll 1
                for (int b = 0; b < 16; ++b)
                    rows[off + b] = (q + b >= lo && q + b < hi) ? q[b] : (uint8_t)0;
            }
        }
    }
}

template <int C, int PX, int TH, int KL, bool NEAREST, int OUT>
__global__ __launch_bounds__(64 * kTileWaves) void tile_u8(
    const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int H, int W, int dH, int dW,
    long long src_bytes, TileGeom tg, int nn_map)
{
    constexpr int COLS = 64 * PX;
    constexpr int NT = 64 * kTileWaves;
    static_assert(TH % kTileWaves == 0 && (PX * C) % 4 == 0, "tile shape");
    static_assert(OUT == kOutSame || (OUT == kOutGrey && !NEAREST && C >= 3), "tile output");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_all[];
    uint32_t *const ctab = (uint32_t *)lds_all;      // COLS packed column entries
    uint8_t *const rows = lds_all + COLS * 4;        // staged rows, tg.pitch bytes apart
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // workgroup -> (image n, row tile ty, column segment tx)
    const unsigned r1 = fast_div(blockIdx.x, tg.by_tiles_x);
    const int tx = (int)(blockIdx.x - r1 * (unsigned)tg.tiles_x);
    const unsigned n = fast_div(r1, tg.by_tiles_y);
    const int ty = (int)(r1 - n * (unsigned)tg.tiles_y);

    const int wx0 = tx * COLS, wx1 = min(wx0 + COLS, dW) - 1;
    const int dy0 = ty * TH, dy1 = min(dy0 + TH, dH) - 1;
    // source columns [sa, sb] and rows [ra0, rb1] the tile touches (both
    // maps are non-decreasing, so the end points bound them)
    int sa, sb, ra0, rb1;
    if constexpr (NEAREST) {
        sa = nearest_index(wx0, W, dW, nn_map);
        sb = nearest_index(wx1, W, dW, nn_map);
        ra0 = nearest_index(dy0, H, dH, nn_map);
        rb1 = nearest_index(dy1, H, dH, nn_map);
    } else {
        sa = axis_tap(wx0, W, dW).a;
        sb = axis_tap(wx1, W, dW).b;
        ra0 = axis_tap(dy0, H, dH).a;
        rb1 = axis_tap(dy1, H, dH).b;
    }
    const int nr = rb1 - ra0 + 1;                    // staged rows, at most the launch's cap
    const unsigned bytes = (unsigned)(sb - sa + 1) * C;
    const size_t row_bytes = (size_t)W * C;
    const uint8_t *const lo = src;
    const uint8_t *const hi = src + src_bytes;
    // first needed byte of staged row k: p0 + k row_bytes; its offset in its
    // 16-byte chunk steps by row_bytes mod 16 from row to row
    const uint8_t *const p0 =
        src + ((size_t)n * H + ra0) * row_bytes + (size_t)sa * C;
    const unsigned mis0 = (unsigned)(uintptr_t)p0 & 15u;
    const unsigned rstep = (unsigned)(row_bytes & 15u);

    tile_stage<KL>(rows, p0, mis0, rstep, row_bytes, nr, tg, lo, hi);
    // the segment's column table (nearest: the byte offset alone); columns
    // past dW - 1 repeat the last one
    for (int c = tid; c < COLS; c += NT) {
        if constexpr (NEAREST) {
            ctab[c] = (uint32_t)((nearest_index(min(wx0 + c, dW - 1), W, dW, nn_map) - sa) * C);
        } else {
            const Tap t = axis_tap(min(wx0 + c, dW - 1), W, dW);
            ctab[c] = ((uint32_t)((t.a - sa) * C) << 13) | ((uint32_t)(t.b != t.a) << 12) |
                      weight11(t);
        }
    }
    __syncthreads();

    int toff[PX];
    uint32_t twp[PX];
#pragma unroll
    for (int p = 0; p < PX; ++p) {
        const uint32_t e = ctab[lane * PX + p];
        toff[p] = NEAREST ? (int)e : (int)(e >> 13);
        twp[p] = weight_pair(e & 4095u, (e >> 12) & 1u);
    }
    const int x0 = wx0 + lane * PX;
    const int valid_px = max(0, min(PX, dW - x0));
    constexpr int RW = TH / kTileWaves;
    if constexpr (NEAREST) {
        // one source row per output row; an output row that maps to the
        // same source row as the one before repeats its bytes
        uint8_t res[PX * C];
        int iK = -1;                                  // staged row held in res (uniform)
        for (int r = 0; r < RW; ++r) {
            const int dy = dy0 + wave * RW + r;
            if (dy > dy1) break;                      // a short last tile (uniform)
            const int k = nearest_index(dy, H, dH, nn_map) - ra0;
            if (k != iK) {
                const uint8_t *l = rows + k * tg.pitch + ((mis0 + (unsigned)k * rstep) & 15u);
#pragma unroll
                for (int p = 0; p < PX; ++p) {
                    if constexpr (C == 1) {
                        res[p] = l[toff[p]];
                    } else {
                        const uint32_t w = lds_bytes4(l + toff[p]);
#pragma unroll
                        for (int c = 0; c < C; ++c) res[p * C + c] = (uint8_t)(w >> (8 * c));
                    }
                }
                iK = k;
            }
            if (valid_px > 0)
                store_chunk<uint8_t, PX * C>(dst + (((size_t)n * dH + dy) * dW + x0) * C, res,
                                             valid_px * C);
        }
        return;
    }
    // Each staged row's horizontal sums (row_sum_u8 per channel and pixel,
    // or per pixel of grey values for grey output) are kept for as long as
    // consecutive output rows use the row: a wave walks its rows downwards,
    // so the last two rows it summed suffice.
    constexpr int NH = OUT == kOutGrey ? PX : PX * C;
    uint32_t hA[NH], hB[NH];
    int iA = -1, iB = -1;                             // rows held in hA, hB (uniform)
    auto hrow = [&](int k, uint32_t (&h)[NH]) __attribute__((always_inline)) {
        const uint8_t *l = rows + k * tg.pitch + ((mis0 + (unsigned)k * rstep) & 15u);
#pragma unroll
        for (int p = 0; p < PX; ++p) {
            if constexpr (C == 1) {
                const uint8_t *q = l + toff[p];
                h[p] = row_sum_u8((uint32_t)q[0] | ((uint32_t)q[1] << 16), twp[p]);
            } else if constexpr (OUT == kOutGrey) {
                // both taps to grey first (tap b at byte C), then the sum
                uint32_t w_lo, w_hi;
                lds_bytes8(l + toff[p], w_lo, w_hi);
                auto gr = [](uint32_t w) {
                    return grey_u8(w & 255u, (w >> 8) & 255u, (w >> 16) & 255u);
                };
                const uint32_t w2 = C == 4 ? w_hi : __builtin_amdgcn_alignbyte(w_hi, w_lo, C);
                h[p] = row_sum_u8(gr(w_lo) | (gr(w2) << 16), twp[p]);
            } else {
                uint32_t w_lo, w_hi;
                lds_bytes8(l + toff[p], w_lo, w_hi);
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const uint32_t sel = 0x0c000c00u | ((uint32_t)(C + c) << 16) | (uint32_t)c;
                    h[p * C + c] = row_sum_u8(__builtin_amdgcn_perm(w_hi, w_lo, sel), twp[p]);
                }
            }
        }
    };
    for (int r = 0; r < RW; ++r) {
        const int dy = dy0 + wave * RW + r;
        if (dy > dy1) break;                          // a short last tile (uniform)
        const Tap t = axis_tap(dy, H, dH);
        const int ka = t.a - ra0, kb = t.b - ra0;
        if (ka != iA) {
            if (ka == iB) {
#pragma unroll
                for (int k = 0; k < NH; ++k) hA[k] = hB[k];
            } else {
                hrow(ka, hA);
            }
            iA = ka;
        }
        if (kb != iB) {
            if (kb == iA) {
#pragma unroll
                for (int k = 0; k < NH; ++k) hB[k] = hA[k];
            } else {
                hrow(kb, hB);
            }
            iB = kb;
        }
        const unsigned wy1 = weight11(t);
        const uint32_t wy0x4 = (2048u - wy1) << 2, wy1x4 = wy1 << 2;
        uint32_t fx[NH];
#pragma unroll
        for (int k = 0; k < NH; ++k) fx[k] = col_sum_u8(hA[k], hB[k], wy0x4, wy1x4);
        if constexpr (OUT == kOutGrey) {
            uint8_t resg[PX];
#pragma unroll
            for (int p = 0; p < PX; ++p) resg[p] = (uint8_t)(fx[p] >> 24);
            if (valid_px > 0)
                store_chunk<uint8_t, PX>(dst + ((size_t)n * dH + dy) * dW + x0, resg, valid_px);
            continue;
        }
        uint32_t wds[PX * C / 4];
#pragma unroll
        for (int k = 0; k < PX * C / 4; ++k)
            wds[k] = pack_byte3(fx[4 * k], fx[4 * k + 1], fx[4 * k + 2], fx[4 * k + 3]);
        uint8_t res[PX * C];
        __builtin_memcpy(res, wds, sizeof(wds));
        if (valid_px > 0)
            store_chunk<uint8_t, PX * C>(dst + (((size_t)n * dH + dy) * dW + x0) * C, res,
                                         valid_px * C);
    }
}

// Row enlargements of float32 images by 2-D tiles (linear, clamp): the tile
// geometry and staging of tile_u8, and blend_f32's arithmetic - the
// horizontal lerp of each source row (kept across output rows, as in
// tile_u8), then the vertical lerp - so the results equal the other
// kernels' bit for bit.  The column table holds two words per column: the
// byte offset of tap a from column sa << 1 | whether tap b is the next
// column, and the weight's bits.  Source rows are 4-byte aligned, and so
// is every staged pixel.  Launched for one channel (PX 8) and RGBA (PX 1,
// one contiguous 16-byte store per lane).  Float RGB enlargements measured
// faster on the direct kernel, which gathers their 12-byte pixels from
// cache and stages its stores (720p -> 1080p RGB 9.1 against 10.1 us here
// with the row staged for contiguous stores, 17.8 without).
template <int C, int PX, int TH, int KL>
__global__ __launch_bounds__(64 * kTileWaves) void tile_f32(
    const float *__restrict__ src, float *__restrict__ dst, int H, int W, int dH, int dW,
    long long src_bytes, TileGeom tg)
{
    constexpr int COLS = 64 * PX;
    constexpr int NT = 64 * kTileWaves;
    constexpr int PB = 4 * C;                        // bytes per pixel
    static_assert(TH % kTileWaves == 0, "tile shape");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_all[];
    uint32_t *const ctab = (uint32_t *)lds_all;      // 2 COLS words
    uint8_t *const rows = lds_all + COLS * 8;        // staged rows, tg.pitch bytes apart
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const unsigned r1 = fast_div(blockIdx.x, tg.by_tiles_x);
    const int tx = (int)(blockIdx.x - r1 * (unsigned)tg.tiles_x);
    const unsigned n = fast_div(r1, tg.by_tiles_y);
    const int ty = (int)(r1 - n * (unsigned)tg.tiles_y);
    const int wx0 = tx * COLS, wx1 = min(wx0 + COLS, dW) - 1;
    const int dy0 = ty * TH, dy1 = min(dy0 + TH, dH) - 1;
    const int sa = axis_tap(wx0, W, dW).a;
    const int ra0 = axis_tap(dy0, H, dH).a, rb1 = axis_tap(dy1, H, dH).b;
    const int nr = rb1 - ra0 + 1;
    const size_t row_bytes = (size_t)W * PB;
    const uint8_t *const lo = (const uint8_t *)src;
    const uint8_t *const p0 = lo + ((size_t)n * H + ra0) * row_bytes + (size_t)sa * PB;
    const unsigned mis0 = (unsigned)(uintptr_t)p0 & 15u;
    const unsigned rstep = (unsigned)(row_bytes & 15u);
    tile_stage<KL>(rows, p0, mis0, rstep, row_bytes, nr, tg, lo, lo + src_bytes);
    for (int c = tid; c < COLS; c += NT) {
        const Tap t = axis_tap(min(wx0 + c, dW - 1), W, dW);
        ctab[2 * c] = ((uint32_t)((t.a - sa) * PB) << 1) | (uint32_t)(t.b != t.a);
        ctab[2 * c + 1] = __builtin_bit_cast(uint32_t, weightf(t));
    }
    __syncthreads();

    int toff[PX];
    bool tnext[PX];
    float wx[PX];
#pragma unroll
    for (int p = 0; p < PX; ++p) {
        const uint32_t e = ctab[2 * (lane * PX + p)];
        toff[p] = (int)(e >> 1);
        tnext[p] = e & 1u;
        wx[p] = __builtin_bit_cast(float, ctab[2 * (lane * PX + p) + 1]);
    }
    const int x0 = wx0 + lane * PX;
    const int valid_px = max(0, min(PX, dW - x0));
    constexpr int RW = TH / kTileWaves;
    constexpr int NH = PX * C;
    float hA[NH], hB[NH];
    int iA = -1, iB = -1;                             // rows held in hA, hB (uniform)
    auto hrow = [&](int k, float (&h)[NH]) __attribute__((always_inline)) {
        const uint8_t *l = rows + k * tg.pitch + ((mis0 + (unsigned)k * rstep) & 15u);
#pragma unroll
        for (int p = 0; p < PX; ++p) {
            const float *q = (const float *)__builtin_assume_aligned(l + toff[p], 4);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const float a = q[c], b = tnext[p] ? q[C + c] : a;
                h[p * C + c] = fmaf(wx[p], b - a, a);
            }
        }
    };
    for (int r = 0; r < RW; ++r) {
        const int dy = dy0 + wave * RW + r;
        if (dy > dy1) break;                          // a short last tile (uniform)
        const Tap t = axis_tap(dy, H, dH);
        const int ka = t.a - ra0, kb = t.b - ra0;
        if (ka != iA) {
            if (ka == iB) {
#pragma unroll
                for (int k = 0; k < NH; ++k) hA[k] = hB[k];
            } else {
                hrow(ka, hA);
            }
            iA = ka;
        }
        if (kb != iB) {
            if (kb == iA) {
#pragma unroll
                for (int k = 0; k < NH; ++k) hB[k] = hA[k];
            } else {
                hrow(kb, hB);
            }
            iB = kb;
        }
        const float wy = weightf(t);
        float res[NH];
#pragma unroll
        for (int k = 0; k < NH; ++k) res[k] = fmaf(wy, hB[k] - hA[k], hA[k]);
        if (valid_px > 0)
            store_chunk<float, NH>(dst + (((size_t)n * dH + dy) * dW + x0) * C, res, valid_px * C);
    }
}

// --------------------------------------------------------------------------
// Plain copy for bandwidth calibration: 16-byte units, grid-stride, each lane
// keeping kCopyUnroll loads in flight before it stores them (one load then
// one store per pass would wait a full memory latency per chunk), with the
// streaming hints a one-pass copy wants.  A byte copy covers a ragged tail.
// --------------------------------------------------------------------------
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kBlock) void copy_16(const uint4 *__restrict__ src,
                                                  uint4 *__restrict__ dst, long long n16)
{
    const u32x4_t *s = (const u32x4_t *)src;
    u32x4_t *d = (u32x4_t *)dst;
    const long long stride = (long long)gridDim.x * kBlock;
    long long i = (long long)blockIdx.x * kBlock + threadIdx.x;
    for (; i + (kCopyUnroll - 1) * stride < n16; i += kCopyUnroll * stride) {
        u32x4_t v[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(s + i + u * stride);
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], d + i + u * stride);
    }
    for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

__global__ __launch_bounds__(kBlock) void copy_1(const uint8_t *__restrict__ src,
                                                 uint8_t *__restrict__ dst, long long n)
{
    const long long stride = (long long)gridDim.x * kBlock;
    for (long long i = (long long)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

}  // namespace mirsz
