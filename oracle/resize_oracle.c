/*
 * Plain CPU oracle for image resize: linear (bilinear) and nearest-neighbour.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library: it is a second, deliberately slow and literal statement of
 * what the resize computes, written so that it can be checked against the
 * pages by eye.
 *
 * Sources followed (web pages, cited by title and section):
 *  [P1] "From Prototype to Performance: Optimizing OpenCV Resize on Volcanic
 *       GPUs" (Imagination blog).  Sections "Step 1: Build a reliable
 *       reference path" (each output pixel is mapped back into the input and
 *       sampled there) and "Naive resize with linear sampling" (the output
 *       pixel centre, coordinate + 0.5, is scaled into the input and handed to
 *       a linear sampler, which filters around the texel centres).
 *  [P3] hnwysp.cn news/129086, CUDA nearest and bilinear interpolation:
 *       s2.1 (nearest: map, round to nearest, take that pixel),
 *       s2.2 (bilinear: i = floor(x), j = floor(y), u = x - i, v = y - j and
 *       the four-term weighted sum), s3.3 (the right/bottom neighbour index is
 *       limited to the last pixel), s6.1 (clamping of coordinates to
 *       [0, size - 1]) and s6.2 (fixed-point arithmetic for precision).
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes):
 *  - Coordinate map: half-pixel centres, x = (dx + 0.5) * W / dW - 0.5.  [P1]
 *    adds 0.5 before scaling and samples with a linear filter whose taps sit at
 *    texel centres, which is this map.  The scale is taken per axis from the
 *    sizes (W / dW and H / dH), as an exact rational number.
 *  - x is carried as the exact fraction num / den with num = (2 dx + 1) W - dW
 *    and den = 2 dW, so floor and remainder are exact integer operations.
 *  - Border: by default the coordinate is clamped to [0, size - 1] ([P3] s6.1)
 *    and the second neighbour to size - 1 ([P3] s3.3).  The *_border entry
 *    points also take [P3] s6.1's two other rules, mirror (reflection about
 *    the outermost pixel centres) and wrap (periodic image), applied to the
 *    exact coordinate.
 *  - uint8: u and v are quantised to 11 fractional bits (2048 = 1.0), rounding
 *    half up; the four products of [P3] s2.2 are formed exactly in integers and
 *    rounded once, half up, at 2^22.  No intermediate rounding.
 *  - float32: u, v and the four-term sum of [P3] s2.2 are evaluated in double
 *    and rounded to float once.
 *  - Nearest: the same half-pixel map, then round half up ([P3] s2.1 rounds to
 *    the nearest pixel), then clamp ([P3] s3.2 / s6.1).  Two corner-aligned
 *    mappings are offered beside it (oracle_nearest_map): [P3] s3.2's kernel
 *    as printed, x = dx / scale rounded half up; and the same coordinate
 *    taken with floor, the legacy nearest of image libraries.
 *
 * Layout: src is N x H x W x C (interleaved channels, "HWC" per image),
 * dst is N x dH x dW x C, both contiguous.  Output rows are numbered
 * globally as r = n * dH + dy; a call computes rows [row_begin, row_end).
 */
#include <stdint.h>
#include <stddef.h>

/* floor(a / b) for b > 0, any sign of a (C's '/' truncates toward zero). */
static int64_t floor_div(int64_t a, int64_t b)
{
    int64_t q = a / b;
    if ((a % b != 0) && (a < 0))
        q -= 1;
    return q;
}

/*
 * One axis of the coordinate map ([P1] linear sampling; [P3] s2.2, s6.1).
 * Output index d of an axis of out_len samples drawn from in_len samples.
 * The source coordinate x = (d + 1/2) * in_len / out_len - 1/2 equals num/den.
 * A coordinate outside [0, in_len - 1] is brought back by the border rule of
 * [P3] s6.1:
 *   BORDER_CLAMP   clamp it to [0, in_len - 1];
 *   BORDER_MIRROR  reflect it symmetrically about the outermost pixel
 *                  centres (x -> -x below 0, x -> 2 (in_len - 1) - x above);
 *   BORDER_WRAP    treat the image as periodic (x -> x + in_len below 0,
 *                  x -> x - in_len above in_len - 1).
 * Then *i = floor(x), and the fractional part u = x - i is returned as the
 * exact fraction (*u_num) / (*u_den).
 */
enum { BORDER_CLAMP = 0, BORDER_MIRROR = 1, BORDER_WRAP = 2 };

static void map_axis_border(int64_t d, int64_t in_len, int64_t out_len, int border,
                            int64_t *i, int64_t *u_num, int64_t *u_den)
{
    int64_t num = (2 * d + 1) * in_len - out_len;
    int64_t den = 2 * out_len;
    *u_den = den;
    if (in_len == 1) {                  /* a single pixel: every rule gives it */
        *i = 0;
        *u_num = 0;
        return;
    }
    if (border == BORDER_MIRROR) {
        if (num < 0)
            num = -num;
        if (num > (in_len - 1) * den)
            num = 2 * (in_len - 1) * den - num;
    } else if (border == BORDER_WRAP) {
        if (num < 0)
            num += in_len * den;
        if (num >= in_len * den)
            num -= in_len * den;
    }
    if (num < 0) {                      /* x < 0: clamp to 0 */
        *i = 0;
        *u_num = 0;
        return;
    }
    if (num > (in_len - 1) * den) {     /* x > in_len - 1: clamp (clamp rule, */
        *i = in_len - 1;                /* or the wrap rule's last interval  */
        *u_num = num - (in_len - 1) * den;   /* handled below)              */
        if (border != BORDER_WRAP)
            *u_num = 0;
        return;
    }
    *i = floor_div(num, den);
    *u_num = num - (*i) * den;          /* x - i, times den; in [0, den) */
}

/* Second neighbour, limited to the last pixel ([P3] s3.3). */
static int64_t next_index(int64_t i, int64_t len)
{
    return (i + 1 < len) ? (i + 1) : (len - 1);
}

/* Second neighbour under a border rule: under wrap the pixel after the last
 * is the first (periodic image); otherwise as next_index. */
static int64_t next_index_border(int64_t i, int64_t len, int border)
{
    if (border == BORDER_WRAP)
        return (i + 1 < len) ? (i + 1) : 0;
    return next_index(i, len);
}

/* u quantised to 11 fractional bits: round-half-up of 2048 * u_num / u_den. */
static int64_t quantise_11(int64_t u_num, int64_t u_den)
{
    return floor_div(4096 * u_num + u_den, 2 * u_den);
}

int oracle_linear_u8_border(const uint8_t *src, uint8_t *dst,
                            int N, int H, int W, int C, int dH, int dW,
                            int64_t row_begin, int64_t row_end, int border)
{
    if (!src || !dst || N < 1 || H < 1 || W < 1 || C < 1 || dH < 1 || dW < 1)
        return 1;
    if (border < BORDER_CLAMP || border > BORDER_WRAP)
        return 3;
    if (row_begin < 0 || row_end > (int64_t)N * dH || row_begin > row_end)
        return 2;
    for (int64_t r = row_begin; r < row_end; ++r) {
        int64_t n = r / dH, y = r % dH;
        int64_t j, v_num, v_den;
        map_axis_border(y, H, dH, border, &j, &v_num, &v_den);
        int64_t j1 = next_index_border(j, H, border);
        int64_t V = quantise_11(v_num, v_den);           /* v * 2048 */
        const uint8_t *img = src + (size_t)n * H * W * C;
        for (int64_t x = 0; x < dW; ++x) {
            int64_t i, u_num, u_den;
            map_axis_border(x, W, dW, border, &i, &u_num, &u_den);
            int64_t i1 = next_index_border(i, W, border);
            int64_t U = quantise_11(u_num, u_den);       /* u * 2048 */
            for (int64_t c = 0; c < C; ++c) {
                /* src(i, j): column i, row j */
                int64_t s_ij   = img[((size_t)j  * W + i ) * C + c];
                int64_t s_i1j  = img[((size_t)j  * W + i1) * C + c];
                int64_t s_ij1  = img[((size_t)j1 * W + i ) * C + c];
                int64_t s_i1j1 = img[((size_t)j1 * W + i1) * C + c];
                /* [P3] s2.2 with (1-u) -> (2048-U), u -> U, etc. */
                int64_t sum = (2048 - U) * (2048 - V) * s_ij
                            + U * (2048 - V) * s_i1j
                            + (2048 - U) * V * s_ij1
                            + U * V * s_i1j1;
                int64_t out = (sum + ((int64_t)1 << 21)) >> 22;
                dst[(((size_t)n * dH + y) * dW + x) * C + c] = (uint8_t)out;
            }
        }
    }
    return 0;
}

int oracle_linear_f32_border(const float *src, float *dst,
                             int N, int H, int W, int C, int dH, int dW,
                             int64_t row_begin, int64_t row_end, int border)
{
    if (!src || !dst || N < 1 || H < 1 || W < 1 || C < 1 || dH < 1 || dW < 1)
        return 1;
    if (border < BORDER_CLAMP || border > BORDER_WRAP)
        return 3;
    if (row_begin < 0 || row_end > (int64_t)N * dH || row_begin > row_end)
        return 2;
    for (int64_t r = row_begin; r < row_end; ++r) {
        int64_t n = r / dH, y = r % dH;
        int64_t j, v_num, v_den;
        map_axis_border(y, H, dH, border, &j, &v_num, &v_den);
        int64_t j1 = next_index_border(j, H, border);
        double v = (double)v_num / (double)v_den;
        const float *img = src + (size_t)n * H * W * C;
        for (int64_t x = 0; x < dW; ++x) {
            int64_t i, u_num, u_den;
            map_axis_border(x, W, dW, border, &i, &u_num, &u_den);
            int64_t i1 = next_index_border(i, W, border);
            double u = (double)u_num / (double)u_den;
            for (int64_t c = 0; c < C; ++c) {
                double s_ij   = img[((size_t)j  * W + i ) * C + c];
                double s_i1j  = img[((size_t)j  * W + i1) * C + c];
                double s_ij1  = img[((size_t)j1 * W + i ) * C + c];
                double s_i1j1 = img[((size_t)j1 * W + i1) * C + c];
                double sum = (1.0 - u) * (1.0 - v) * s_ij
                           + u * (1.0 - v) * s_i1j
                           + (1.0 - u) * v * s_ij1
                           + u * v * s_i1j1;
                dst[(((size_t)n * dH + y) * dW + x) * C + c] = (float)sum;
            }
        }
    }
    return 0;
}

int oracle_linear_u8(const uint8_t *src, uint8_t *dst, int N, int H, int W, int C,
                     int dH, int dW, int64_t row_begin, int64_t row_end)
{
    return oracle_linear_u8_border(src, dst, N, H, W, C, dH, dW, row_begin, row_end,
                                   BORDER_CLAMP);
}

int oracle_linear_f32(const float *src, float *dst, int N, int H, int W, int C,
                      int dH, int dW, int64_t row_begin, int64_t row_end)
{
    return oracle_linear_f32_border(src, dst, N, H, W, C, dH, dW, row_begin, row_end,
                                    BORDER_CLAMP);
}

/*
 * Nearest neighbour ([P3] s2.1): map the output pixel centre into the input
 * (same half-pixel map as above), round half up, clamp to the image.  The
 * element is copied bit for bit, so one routine serves every element size.
 */
static int64_t nearest_index(int64_t d, int64_t in_len, int64_t out_len)
{
    int64_t num = (2 * d + 1) * in_len - out_len;   /* x = num / den */
    int64_t den = 2 * out_len;
    int64_t k = floor_div(num + den / 2, den);      /* round(x), half up */
    if (k < 0) k = 0;
    if (k > in_len - 1) k = in_len - 1;
    return k;
}

/*
 * Corner-aligned nearest ([P3] s3.2: the source coordinate is dx / scale with
 * scale = out_len / in_len, no half-pixel shift): x = d * in_len / out_len.
 *   NEAREST_ROUND  round x half up, as [P3] s3.2's kernel does
 *                  (floor(x + 0.5)), then clamp to the image;
 *   NEAREST_FLOOR  floor(x), which never leaves the image.
 */
enum { NEAREST_HALF_PIXEL = 0, NEAREST_FLOOR = 1, NEAREST_ROUND = 2 };

static int64_t nearest_index_corner(int64_t d, int64_t in_len, int64_t out_len, int mapping)
{
    int64_t k;
    if (mapping == NEAREST_FLOOR)
        k = floor_div(d * in_len, out_len);
    else
        k = floor_div(2 * d * in_len + out_len, 2 * out_len);   /* floor(x + 1/2) */
    if (k > in_len - 1) k = in_len - 1;
    return k;
}

static int64_t nearest_index_map(int64_t d, int64_t in_len, int64_t out_len, int mapping)
{
    if (mapping == NEAREST_HALF_PIXEL)
        return nearest_index(d, in_len, out_len);
    return nearest_index_corner(d, in_len, out_len, mapping);
}

int oracle_nearest_map(const void *src_v, void *dst_v, int elem_bytes,
                       int N, int H, int W, int C, int dH, int dW,
                       int64_t row_begin, int64_t row_end, int mapping)
{
    const unsigned char *src = (const unsigned char *)src_v;
    unsigned char *dst = (unsigned char *)dst_v;
    if (!src || !dst || elem_bytes < 1 || N < 1 || H < 1 || W < 1 || C < 1 ||
        dH < 1 || dW < 1)
        return 1;
    if (row_begin < 0 || row_end > (int64_t)N * dH || row_begin > row_end)
        return 2;
    if (mapping < NEAREST_HALF_PIXEL || mapping > NEAREST_ROUND)
        return 3;
    size_t px = (size_t)C * (size_t)elem_bytes;
    for (int64_t r = row_begin; r < row_end; ++r) {
        int64_t n = r / dH, y = r % dH;
        int64_t sy = nearest_index_map(y, H, dH, mapping);
        for (int64_t x = 0; x < dW; ++x) {
            int64_t sx = nearest_index_map(x, W, dW, mapping);
            const unsigned char *from =
                src + (((size_t)n * H + sy) * W + sx) * px;
            unsigned char *to = dst + (((size_t)n * dH + y) * dW + x) * px;
            for (size_t b = 0; b < px; ++b)
                to[b] = from[b];
        }
    }
    return 0;
}

int oracle_nearest(const void *src_v, void *dst_v, int elem_bytes,
                   int N, int H, int W, int C, int dH, int dW,
                   int64_t row_begin, int64_t row_end)
{
    return oracle_nearest_map(src_v, dst_v, elem_bytes, N, H, W, C, dH, dW, row_begin, row_end,
                              NEAREST_HALF_PIXEL);
}
