/*
 * mi_resize.h - C ABI of the gfx950 image-resize library (libmi_resize.so).
 *
 * Operations
 *   resize_linear   linear (bilinear) interpolation, OpenCV INTER_LINEAR
 *                   style.  Defined by "From Prototype to Performance:
 *                   Optimizing OpenCV Resize on Volcanic GPUs" (Imagination
 *                   blog), sections "Step 1: Build a reliable reference path"
 *                   and "Naive resize with linear sampling" (each output pixel
 *                   centre, coordinate + 0.5, is scaled back into the input and
 *                   sampled with a linear filter), and by hnwysp.cn news/129086
 *                   s2.2 (the four-neighbour weighted sum), s3.3 (the second
 *                   neighbour is limited to the last pixel), s6.1 (clamping)
 *                   and s6.2 (fixed point).
 *   resize_nearest  nearest neighbour, hnwysp.cn news/129086 s2.1 (map the
 *                   output pixel into the input and round to the nearest
 *                   pixel) with the same half-pixel map and clamping.
 *
 * What is computed, per image n, output pixel (dy, dx), channel c:
 *   - source coordinate x = (dx + 0.5) * W / dW - 0.5 (and likewise y with
 *     H / dH), carried as an exact fraction; x0 = floor(x), u = x - x0;
 *     neighbour columns clamp(x0, 0, W-1) and clamp(x0 + 1, 0, W-1)
 *     ("clamp to edge"); rows the same.
 *   - uint8: u and v are rounded half up to 11 fractional bits
 *     (U = round(2048 u) in [0, 2048]); the result is
 *       ((2048-V)((2048-U) p00 + U p01) + V((2048-U) p10 + U p11) + 2^21) >> 22
 *     evaluated exactly in integers (rounded once, half up).
 *   - float32: u = r / den computed from the exact remainder, then
 *       t = p00 + u (p01 - p00), b = p10 + u (p11 - p10), out = t + v (b - t)
 *     in float32 fused multiply-adds.  Agrees with the exact real-valued
 *     bilinear value to well within 1e-5 for inputs in [0, 1].
 *   - nearest: source column min(floor((dx + 0.5) * W / dW), W - 1) (the
 *     half-pixel coordinate rounded half up), likewise the row; the element
 *     bytes are copied unchanged.
 *
 * Layout: src is batch x H x W x C, dst is batch x dst_H x dst_W x C, both
 * contiguous with interleaved channels (HWC per image, images back to back),
 * same element type.  Element type: dtype MI_RESIZE_U8 (uint8_t) or
 * MI_RESIZE_F32 (float).  C is 1, 3 or 4.
 *
 * Pointers: src and dst are DEVICE pointers (hipMalloc'ed memory or memory
 * the device can access, e.g. torch CUDA tensors) owned by the caller.  The
 * library allocates nothing, keeps no state between calls and never takes
 * ownership.  The two byte ranges must not overlap.  Any alignment is
 * accepted for uint8; float32 buffers must be 4-byte aligned (element
 * aligned).  16-byte aligned buffers take the vectorised paths.
 *
 * Stream: the work is enqueued on `stream` (a hipStream_t; NULL means the
 * null stream) and the call returns without waiting.  The caller synchronises
 * before reading dst.  Calls are re-entrant and thread safe.
 *
 * Errors: every argument is checked before anything is enqueued; on a bad
 * argument the call returns a non-zero status, enqueues nothing and leaves
 * dst untouched.  A failed kernel launch returns MI_RESIZE_ERR_HIP.  A fault
 * during execution (e.g. a host pointer passed as src) is reported by the HIP
 * runtime at the caller's next synchronisation.
 *
 * Limits: 1 <= H, W, dst_H, dst_W <= 65535; batch >= 1;
 * batch * H * W <= 2^40 and batch * dst_H * dst_W <= 2^40.
 */
#ifndef MI_RESIZE_H
#define MI_RESIZE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MI_RESIZE_ABI_VERSION 6

enum mi_resize_dtype {
    MI_RESIZE_U8 = 0,   /* uint8_t elements  */
    MI_RESIZE_F32 = 1   /* float32 elements  */
};

enum mi_resize_border {
    MI_RESIZE_BORDER_CLAMP = 0,   /* clamp to the edge pixel (resize_linear)          */
    MI_RESIZE_BORDER_MIRROR = 1,  /* reflect about the outermost pixel centres        */
    MI_RESIZE_BORDER_WRAP = 2     /* periodic image                                   */
};

enum mi_resize_nearest_mapping {
    MI_RESIZE_NEAREST_HALF_PIXEL = 0,  /* pixel centres, rounded half up (resize_nearest) */
    MI_RESIZE_NEAREST_FLOOR = 1,       /* corner-aligned d * W / dW, floored (legacy)      */
    MI_RESIZE_NEAREST_ROUND = 2        /* corner-aligned d * W / dW, rounded half up       */
};

enum mi_resize_status {
    MI_RESIZE_OK = 0,
    MI_RESIZE_ERR_NULL = 1,      /* src or dst is NULL                        */
    MI_RESIZE_ERR_SHAPE = 2,     /* a size is out of the limits above         */
    MI_RESIZE_ERR_CHANNELS = 3,  /* C is not 1, 3 or 4                        */
    MI_RESIZE_ERR_DTYPE = 4,     /* dtype is not MI_RESIZE_U8 / MI_RESIZE_F32 */
    MI_RESIZE_ERR_OVERLAP = 5,   /* src and dst byte ranges overlap           */
    MI_RESIZE_ERR_HIP = 6,       /* the HIP runtime refused the launch        */
    MI_RESIZE_ERR_ALIGN = 7,     /* float32 src or dst not 4-byte aligned     */
    MI_RESIZE_ERR_PARAM = 8      /* bad parameter of an extended entry point  */
};

/* Linear (bilinear) resize; see the header comment for the exact result. */
int resize_linear(const void *src, void *dst, int batch, int H, int W, int C,
                  int dtype, int dst_H, int dst_W, void *stream);

/* Nearest-neighbour resize (half-pixel centres, rounding half up). */
int resize_nearest(const void *src, void *dst, int batch, int H, int W, int C,
                   int dtype, int dst_H, int dst_W, void *stream);

/*
 * Nearest-neighbour resize with a choice of coordinate mapping; per axis,
 * output index d of dW (or dH) picks source index
 *   MI_RESIZE_NEAREST_HALF_PIXEL  floor((d + 1/2) W / dW): identical to
 *                                 resize_nearest;
 *   MI_RESIZE_NEAREST_FLOOR       floor(d W / dW): the corner-aligned
 *                                 coordinate d / scale of hnwysp.cn news/129086
 *                                 s3.2 (scale = dW / W), floored - the legacy
 *                                 nearest of image libraries;
 *   MI_RESIZE_NEAREST_ROUND       floor(d W / dW + 1/2): the same coordinate
 *                                 rounded half up, as that section's kernel
 *                                 does;
 * each limited to W - 1, all in exact integer arithmetic.  Elements are copied
 * bit for bit.  Other arguments, layout and errors as resize_nearest; an
 * unknown mapping returns MI_RESIZE_ERR_PARAM.
 */
int resize_nearest_mapping(const void *src, void *dst, int batch, int H, int W, int C,
                           int dtype, int dst_H, int dst_W, int mapping, void *stream);

/*
 * Linear resize fused with normalisation, for batches fed to a network.
 * The resize fused with the step that follows it ("merge" of consecutive
 * kernels with the same work shape in "Performance Optimization of Object
 * Tracking Algorithms in OpenCV on GPUs", s4; fusing interpolation with later
 * processing in hnwysp.cn news/129086 s4.2 and s11, for the batched data
 * augmentation of s7.2).
 *
 * src: uint8, batch x H x W x C (as resize_linear).  dst: float32, either
 * batch x dst_H x dst_W x C (layout 0, NHWC) or batch x C x dst_H x dst_W
 * (layout 1, NCHW).  Each element is
 *     dst = (v * alpha - mean[c]) / std_dev[c]
 * where v is exactly the uint8 value resize_linear produces; the kernel
 * evaluates it as one float32 fused multiply-add with scale = alpha / std_dev
 * and bias = -mean / std_dev computed in double and rounded to float.
 * mean and std_dev are HOST arrays of C floats, read during the call.
 * Errors as above, plus MI_RESIZE_ERR_PARAM (mean / std_dev NULL, std_dev
 * zero or not finite, alpha not finite, layout not 0 / 1) and
 * MI_RESIZE_ERR_ALIGN (dst not 4-byte aligned).
 */
int resize_linear_normalize(const void *src, float *dst, int batch, int H, int W, int C,
                            int dst_H, int dst_W, float alpha, const float *mean,
                            const float *std_dev, int layout, void *stream);

/*
 * Batched crop-then-resize: image n's region {x, y, w, h} (columns x .. x+w-1,
 * rows y .. y+h-1) is resized linearly to dst_H x dst_W, exactly as
 * resize_linear would resize that crop taken as an image of its own
 * (half-pixel centres and clamp-to-edge relative to the crop).  This is the
 * "random crop then resize" of batched data augmentation (hnwysp.cn
 * news/129086 s7.2) and the differing input regions of multi-stream video
 * (s7.1).
 *
 * rois: DEVICE pointer to batch x 4 int32 {x, y, w, h}, 4-byte aligned,
 * read by the kernels (so it may be written by earlier work on the same
 * stream).  Values are clamped into the image on the device: x to [0, W-1],
 * w to [1, W - x], y and h likewise; no value can make a kernel read outside
 * src.  Other arguments, layout and errors as resize_linear (MI_RESIZE_ERR_NULL
 * for a NULL rois, MI_RESIZE_ERR_ALIGN for a misaligned one).
 */
int resize_linear_roi(const void *src, void *dst, int batch, int H, int W, int C, int dtype,
                      const int32_t *rois, int dst_H, int dst_W, void *stream);

/*
 * Linear resize with a choice of border rule for source coordinates beyond
 * the outermost pixel centres (hnwysp.cn news/129086 s6.1: clamp, mirror,
 * wrap).  The half-pixel map only leaves the image by less than half a pixel,
 * so the rule decides the second tap of the outermost output pixels of an
 * enlargement:
 *   MI_RESIZE_BORDER_CLAMP   x clamped to [0, W-1]: identical to resize_linear;
 *   MI_RESIZE_BORDER_MIRROR  x reflected about the first / last pixel centre
 *                            (x -> -x, x -> 2(W-1) - x) before the taps are
 *                            taken;
 *   MI_RESIZE_BORDER_WRAP    x taken modulo W (the pixel after the last is the
 *                            first).
 * Rows likewise.  Other arguments, layout, weights and errors as
 * resize_linear; an unknown border returns MI_RESIZE_ERR_PARAM.
 */
int resize_linear_border(const void *src, void *dst, int batch, int H, int W, int C, int dtype,
                         int dst_H, int dst_W, int border, void *stream);

/*
 * Linear resize fused with the RGB -> grey conversion that precedes it in
 * the pages' object-detection preprocessing (cvtColor's RGB2Gray, then
 * resize: "Performance Optimization of Object Tracking Algorithms in OpenCV
 * on GPUs" s3.1.1; kernels merged as in its s4).  Every source pixel becomes
 *     grey = 0.299 R + 0.587 G + 0.114 B      (ITU-R BT.601 luma weights)
 * - for uint8 exactly, rounded half up: (299 R + 587 G + 114 B + 500) / 1000;
 * for float32 as two fused multiply-adds - and the grey image is resized
 * exactly as resize_linear would resize it.
 *
 * src: batch x H x W x C with C = 3 (R, G, B) or 4 (R, G, B, alpha; alpha
 * ignored).  dst: batch x dst_H x dst_W x 1, same dtype.  Errors as
 * resize_linear; C other than 3 or 4 returns MI_RESIZE_ERR_CHANNELS.
 */
int resize_linear_grey(const void *src, void *dst, int batch, int H, int W, int C, int dtype,
                       int dst_H, int dst_W, void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *resize_status_string(int status);

/* MI_RESIZE_ABI_VERSION of the built library. */
int resize_abi_version(void);

/*
 * Bandwidth calibration: copy nbytes from src to dst (device pointers, no
 * overlap) with 16-byte loads and stores, enqueued on `stream`.  This is the
 * plain copy against which measured HBM traffic and bandwidth are scaled; it
 * is the counterpart of the 1:1 copy kernel that "From Prototype to
 * Performance" (section "Baseline: simple 1:1 copy behavior") uses as its
 * rough ceiling.  Returns a status code as above.
 */
int resize_copy_bytes(const void *src, void *dst, int64_t nbytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MI_RESIZE_H */
