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

namespace mirsz {

constexpr int kBlock = 256;   // 4 wave64 per workgroup

// --------------------------------------------------------------------------
// Coordinate map for one axis.  Output index d of an axis of n_out samples
// taken from n_in samples: x = (d + 1/2) n_in / n_out - 1/2 = num / den with
// num = (2d + 1) n_in - n_out, den = 2 n_out.  x0 = floor(x) and the
// remainder r = num - x0 den in [0, den) are exact: num < 2^34 is exact in
// double, the quotient is below 2^16, so its rounding error (< 2^-36) is far
// smaller than the gap 1/den >= 2^-17 to the next integer, and the fix-up
// below only guards the argument.  Taps are clamped to the edge.
// --------------------------------------------------------------------------
struct Tap {
    int a;      // clamp(x0, 0, n_in - 1)
    int b;      // clamp(x0 + 1, 0, n_in - 1)
    int r;      // remainder, u = r / den
    int den;    // 2 * n_out
};

__device__ __forceinline__ Tap axis_tap(int d, int n_in, int n_out)
{
    const long long num = (long long)(2 * d + 1) * n_in - n_out;
    const int den = 2 * n_out;
    long long q = (long long)floor((double)num / (double)den);
    long long r = num - q * den;
    if (r < 0) { q -= 1; r += den; }
    else if (r >= den) { q += 1; r -= den; }
    Tap t;
    t.a = (int)(q < 0 ? 0 : (q > n_in - 1 ? n_in - 1 : q));
    t.b = (int)(q + 1 < 0 ? 0 : (q + 1 > n_in - 1 ? n_in - 1 : q + 1));
    t.r = (int)r;
    t.den = den;
    return t;
}

// u rounded half up to 11 fractional bits: floor((4096 r + den) / (2 den)),
// in [0, 2048].  4096 r + den < 2^31 for den <= 131070.
__device__ __forceinline__ unsigned weight11(const Tap &t)
{
    return ((unsigned)t.r * 4096u + (unsigned)t.den) / (2u * (unsigned)t.den);
}

// u as float: r and den are below 2^24, so both convert exactly and the
// quotient is correctly rounded.
__device__ __forceinline__ float weightf(const Tap &t)
{
    return (float)t.r / (float)t.den;
}

// Nearest source index: the half-pixel coordinate rounded half up,
// floor((2d + 1) n_in / (2 n_out)), limited to n_in - 1 (exact by the same
// argument as axis_tap).
__device__ __forceinline__ int nearest_index(int d, int n_in, int n_out)
{
    const long long num = (long long)(2 * d + 1) * n_in;
    const long long den = 2LL * n_out;
    long long q = (long long)floor((double)num / (double)den);
    long long r = num - q * den;
    if (r < 0) q -= 1;
    else if (r >= den) q += 1;
    return (int)(q > n_in - 1 ? n_in - 1 : q);
}

// 11-bit fixed-point blend of one channel, exact in 32 bits:
// every partial sum is below 2048 * 2048 * 255 + 2^21 < 2^31.
__device__ __forceinline__ unsigned blend_u8(unsigned p00, unsigned p01, unsigned p10,
                                             unsigned p11, unsigned wx1, unsigned wy1)
{
    const unsigned wx0 = 2048u - wx1, wy0 = 2048u - wy1;
    const unsigned top = __umul24(wx0, p00) + __umul24(wx1, p01);
    const unsigned bot = __umul24(wx0, p10) + __umul24(wx1, p11);
    return (__umul24(wy0, top) + __umul24(wy1, bot) + (1u << 21)) >> 22;
}

__device__ __forceinline__ float blend_f32(float p00, float p01, float p10, float p11,
                                           float wx, float wy)
{
    const float t = fmaf(wx, p01 - p00, p00);
    const float b = fmaf(wx, p11 - p10, p10);
    return fmaf(wy, b - t, t);
}

// --------------------------------------------------------------------------
// Generic linear resize, any scale, C in {1, 3, 4}.  Grid: 1-D,
// blockIdx = row_block * col_blocks + col_block.  A block covers kBlock
// output columns of `rows_per_block` consecutive global rows; one lane per
// output pixel per row.  PIX4: C == 4 and the buffers are aligned so that a
// whole pixel moves as one 4-byte (u8) or 16-byte (f32) access.
// --------------------------------------------------------------------------
template <typename T, int C, bool PIX4>
__global__ __launch_bounds__(kBlock) void linear_generic(
    const T *__restrict__ src, T *__restrict__ dst, int H, int W, int dH, int dW,
    long long rows_total, int rows_per_block, int col_blocks)
{
    const int cb = (int)(blockIdx.x % (unsigned)col_blocks);
    const long long rb = blockIdx.x / (unsigned)col_blocks;
    const int x = cb * kBlock + (int)threadIdx.x;
    if (x >= dW) return;

    const Tap tx = axis_tap(x, W, dW);
    const int xa = tx.a * C, xb = tx.b * C;
    unsigned wx1 = 0;
    float wxf = 0.f;
    if constexpr (sizeof(T) == 1) wx1 = weight11(tx);
    else wxf = weightf(tx);

    long long g = rb * rows_per_block;
    long long g_end = g + rows_per_block;
    if (g_end > rows_total) g_end = rows_total;
    long long n = g / dH;
    int dy = (int)(g - n * dH);
    const size_t img_elems = (size_t)H * W * C;
    const size_t row_elems = (size_t)W * C;

    for (; g < g_end; ++g) {
        const Tap ty = axis_tap(dy, H, dH);
        const T *img = src + (size_t)n * img_elems;
        const T *r0 = img + (size_t)ty.a * row_elems;
        const T *r1 = img + (size_t)ty.b * row_elems;
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
                *(uint32_t *)out = o;
            } else {
#pragma unroll
                for (int k = 0; k < C; ++k)
                    out[k] = (uint8_t)blend_u8(r0[xa + k], r0[xb + k], r1[xa + k], r1[xb + k],
                                               wx1, wy1);
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
                *(float4 *)out = o;
            } else {
#pragma unroll
                for (int k = 0; k < C; ++k)
                    out[k] = blend_f32(r0[xa + k], r0[xb + k], r1[xa + k], r1[xb + k], wxf, wyf);
            }
        }
        if (++dy == dH) { dy = 0; ++n; }
    }
}

// --------------------------------------------------------------------------
// Exact 2:1 downscale of uint8 (H = 2 dH, W = 2 dW).  The half-pixel centre
// of output pixel d lands exactly between source pixels 2d and 2d + 1
// (x = 2d + 1/2), so both 11-bit weights are 1024 on both axes and the
// general formula reduces, bit for bit, to the rounded 2x2 mean
// (a + b + c + d + 2) >> 2.  No tap is ever clamped.
//
// A lane owns PX consecutive output pixels of one row: it loads 2 PX C bytes
// from each of the two source rows and stores PX C bytes, with PX chosen so
// that a lane moves 32-48 source bytes (C = 1: 8 px, 16 B per row; C = 3:
// 4 px, 24 B per row; C = 4: 2 px, 16 B per row).  Measured on the 4K RGB
// frame, lanes this small beat 8- and 16-pixel lanes: more lanes in flight
// hide more HBM latency, and a lane's loads of both rows go out together.
// Grid: x = 64-lane workgroups across a row, y = output rows (stride
// gridDim.y).  Needs dW % PX == 0 and 16-byte aligned src / dst; then every
// lane's accesses are naturally aligned.  Output row g reads source rows 2g
// and 2g + 1 of the flattened N*H rows, because H = 2 dH.
// --------------------------------------------------------------------------
template <int C> struct HalfShape;
template <> struct HalfShape<1> { static constexpr int PX = 8; using LV = uint4; using SV = uint2; };
template <> struct HalfShape<3> { static constexpr int PX = 4; using LV = uint2; using SV = uint32_t; };
template <> struct HalfShape<4> { static constexpr int PX = 2; using LV = uint4; using SV = uint2; };

constexpr int kHalfBlock = 64;

template <int C>
__global__ __launch_bounds__(kHalfBlock) void linear_half_u8(
    const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int dW, long long rows,
    int chunks_per_row)
{
    using S = HalfShape<C>;
    using LV = typename S::LV;
    using SV = typename S::SV;
    constexpr int INB = 2 * S::PX * C;            // source bytes per row per lane
    constexpr int NIN = INB / (int)sizeof(LV);
    constexpr int NOUT = S::PX * C;               // output bytes per lane
    constexpr int NST = NOUT / (int)sizeof(SV);
    const int j = blockIdx.x * kHalfBlock + threadIdx.x;
    if (j >= chunks_per_row) return;
    const size_t src_row = (size_t)2 * dW * C;
    const size_t dst_row = (size_t)dW * C;
    for (long long g = blockIdx.y; g < rows; g += gridDim.y) {
        const LV *s0 = (const LV *)(src + (size_t)(2 * g) * src_row + (size_t)j * INB);
        const LV *s1 = (const LV *)((const uint8_t *)s0 + src_row);
        LV a[NIN], b[NIN];
#pragma unroll
        for (int k = 0; k < NIN; ++k) {
            a[k] = s0[k];
            b[k] = s1[k];
        }
        const uint8_t *pa = (const uint8_t *)a;
        const uint8_t *pb = (const uint8_t *)b;
        SV r[NST];
        uint8_t *pr = (uint8_t *)r;
#pragma unroll
        for (int k = 0; k < NOUT; ++k) {
            const int p = 2 * k - k % C;          // first source byte of output byte k
            const unsigned s = (unsigned)pa[p] + pa[p + C] + pb[p] + pb[p + C] + 2u;
            pr[k] = (uint8_t)(s >> 2);
        }
        SV *o = (SV *)(dst + (size_t)g * dst_row + (size_t)j * NOUT);
#pragma unroll
        for (int k = 0; k < NST; ++k) o[k] = r[k];
    }
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

template <int BPP, int UNIT>
__global__ __launch_bounds__(kBlock) void nearest_generic(
    const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int H, int W, int dH, int dW,
    long long rows_total, int rows_per_block, int col_blocks)
{
    using U = typename CopyUnit<UNIT>::type;
    constexpr int K = BPP / UNIT;
    const int cb = (int)(blockIdx.x % (unsigned)col_blocks);
    const long long rb = blockIdx.x / (unsigned)col_blocks;
    const int x = cb * kBlock + (int)threadIdx.x;
    if (x >= dW) return;
    const size_t sx = (size_t)nearest_index(x, W, dW) * BPP;

    long long g = rb * rows_per_block;
    long long g_end = g + rows_per_block;
    if (g_end > rows_total) g_end = rows_total;
    long long n = g / dH;
    int dy = (int)(g - n * dH);
    for (; g < g_end; ++g) {
        const int sy = nearest_index(dy, H, dH);
        const U *from = (const U *)(src + (((size_t)n * H + sy) * W) * BPP + sx);
        U *to = (U *)(dst + ((size_t)g * dW + x) * BPP);
#pragma unroll
        for (int k = 0; k < K; ++k) to[k] = from[k];
        if (++dy == dH) { dy = 0; ++n; }
    }
}

// --------------------------------------------------------------------------
// Plain copy (16-byte units, grid-stride) for bandwidth calibration, and a
// byte copy for a ragged tail.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void copy_16(const uint4 *__restrict__ src,
                                                  uint4 *__restrict__ dst, long long n16)
{
    const long long stride = (long long)gridDim.x * kBlock;
    for (long long i = (long long)blockIdx.x * kBlock + threadIdx.x; i < n16; i += stride)
        dst[i] = src[i];
}

__global__ __launch_bounds__(kBlock) void copy_1(const uint8_t *__restrict__ src,
                                                 uint8_t *__restrict__ dst, long long n)
{
    const long long stride = (long long)gridDim.x * kBlock;
    for (long long i = (long long)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

}  // namespace mirsz
