"""CPU oracle for image resize (linear and nearest-neighbour).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never calls it and shares no code
with it.

The arithmetic lives in ``resize_oracle.c`` (plain C, built with gcc into
``liboracle_resize.so``); this module only marshals numpy arrays into it.
What the C file computes, and which passage of the pages each step follows,
is stated in its header:

* "From Prototype to Performance: Optimizing OpenCV Resize on Volcanic GPUs"
  (Imagination blog), sections "Step 1: Build a reliable reference path" and
  "Naive resize with linear sampling": each output pixel centre is mapped back
  into the input and sampled with a linear filter.
* hnwysp.cn news/129086 (CUDA nearest and bilinear interpolation), s2.1
  nearest formula, s2.2 bilinear formula, s3.3 last-pixel limit on the second
  neighbour, s6.1 clamping, s6.2 fixed point.

Pins (checked in ``tests/test_oracle_pins.py``): identity at scale 1,
constant images, exact 2:1 downscale = 2x2 average, linear ramps, nearest
closed form for integer upscales, exact-rational bilinear within the
quantisation bound, and torch's float64 ``interpolate`` as a library special
case.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "resize_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_resize.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, no intrinsics, no vectorisation hints)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        vp = ctypes.c_void_p
        for name in ("oracle_linear_u8_border", "oracle_linear_f32_border"):
            f = getattr(lib, name)
            f.argtypes = [vp, vp, ci, ci, ci, ci, ci, ci, i64, i64, ci]
            f.restype = ci
        lib.oracle_nearest.argtypes = [vp, vp, ci, ci, ci, ci, ci, ci, ci, i64, i64]
        lib.oracle_nearest.restype = ci
        lib.oracle_nearest_map.argtypes = [vp, vp, ci, ci, ci, ci, ci, ci, ci, i64, i64, ci]
        lib.oracle_nearest_map.restype = ci
        _lib = lib
    return _lib


def _as_nhwc(src: np.ndarray) -> np.ndarray:
    if src.ndim == 2:
        src = src[None, :, :, None]
    elif src.ndim == 3:
        src = src[None]
    if src.ndim != 4:
        raise ValueError("expected HW, HWC or NHWC array, got shape %r" % (src.shape,))
    return np.ascontiguousarray(src)


def _rows(N, dH, rows):
    if rows is None:
        return 0, N * dH
    r0, r1 = rows
    if not (0 <= r0 <= r1 <= N * dH):
        raise ValueError("row range out of bounds")
    return r0, r1


BORDERS = {"clamp": 0, "mirror": 1, "wrap": 2}


def resize_linear(src: np.ndarray, dH: int, dW: int, rows=None, border: str = "clamp") -> np.ndarray:
    """Linear (bilinear) resize of an NHWC uint8 or float32 array to dH x dW.

    ``rows=(r0, r1)`` computes only global output rows r0..r1-1 (row index
    n * dH + dy) and returns them as an array of shape (r1 - r0, dW, C);
    without it the whole N x dH x dW x C result is returned.  ``border``
    ("clamp", "mirror" or "wrap") is the rule for coordinates beyond the
    outermost pixel centres (hnwysp.cn news/129086 s6.1).
    """
    src = _as_nhwc(src)
    N, H, W, C = src.shape
    r0, r1 = _rows(N, dH, rows)
    lib = _load()
    if src.dtype == np.uint8:
        fn = lib.oracle_linear_u8_border
    elif src.dtype == np.float32:
        fn = lib.oracle_linear_f32_border
    else:
        raise TypeError("oracle supports uint8 and float32, got %s" % src.dtype)
    full = np.empty((N * dH, dW, C), dtype=src.dtype)
    rc = fn(src.ctypes.data, full.ctypes.data, N, H, W, C, dH, dW, r0, r1, BORDERS[border])
    if rc != 0:
        raise ValueError("oracle rejected arguments (code %d)" % rc)
    if rows is not None:
        return full[r0:r1].copy()
    return full.reshape(N, dH, dW, C)


def resize_linear_normalize(src: np.ndarray, dH: int, dW: int, alpha, mean, std,
                            layout: str = "NCHW") -> np.ndarray:
    """Linear resize of a uint8 NHWC array followed by normalisation:
    (v * alpha - mean[c]) / std[c] evaluated in float64 on the exact uint8
    resize result v, rounded to float32 once, then laid out NHWC or NCHW.
    The resize is the pinned uint8 oracle above; the affine map is applied as
    written (fusing resize with the step after it, as "Performance
    Optimization of Object Tracking Algorithms in OpenCV on GPUs" s4 merges
    kernels and hnwysp.cn news/129086 s4.2 / s11 fuse interpolation with later
    processing)."""
    src = _as_nhwc(src)
    if src.dtype != np.uint8:
        raise TypeError("normalisation takes a uint8 source")
    v = resize_linear(src, dH, dW).astype(np.float64)
    mean = np.asarray(mean, dtype=np.float64)
    std = np.asarray(std, dtype=np.float64)
    out = ((v * float(alpha) - mean) / std).astype(np.float32)
    if layout == "NCHW":
        return np.ascontiguousarray(out.transpose(0, 3, 1, 2))
    if layout == "NHWC":
        return out
    raise ValueError("layout must be NCHW or NHWC")


def rgb_to_grey(src: np.ndarray) -> np.ndarray:
    """Per-pixel grey value of an NHWC RGB(A) array (channels R, G, B first;
    a fourth channel is ignored), with the luma weights of ITU-R BT.601,
    0.299 R + 0.587 G + 0.114 B.  uint8: the exact value rounded half up,
    (299 R + 587 G + 114 B + 500) // 1000.  float32: evaluated in float64 and
    rounded to float32 once.  Returns N x H x W x 1 of the source dtype."""
    src = _as_nhwc(src)
    if src.shape[3] not in (3, 4):
        raise ValueError("grey conversion needs 3 or 4 channels")
    r, g, b = (src[..., k:k + 1] for k in range(3))
    if src.dtype == np.uint8:
        r, g, b = (v.astype(np.int64) for v in (r, g, b))
        return ((299 * r + 587 * g + 114 * b + 500) // 1000).astype(np.uint8)
    r, g, b = (v.astype(np.float64) for v in (r, g, b))
    return (0.299 * r + 0.587 * g + 0.114 * b).astype(np.float32)


def resize_linear_grey(src: np.ndarray, dH: int, dW: int) -> np.ndarray:
    """RGB(A) -> grey, then linear resize of the grey image: the pages'
    object-detection preprocessing runs cvtColor (RGB2Gray) before resize
    ("Performance Optimization of Object Tracking Algorithms in OpenCV on
    GPUs" s3.1.1), here fused into one pass.  The grey image is the exact
    per-pixel conversion above; the resize is the pinned resize_linear."""
    return resize_linear(rgb_to_grey(src), dH, dW)


def clamp_roi(roi, H: int, W: int):
    """The crop {x, y, w, h} clamped into an H x W image: x to [0, W-1],
    w to [1, W - x], y and h likewise (the library's documented rule)."""
    x, y, w, h = (int(v) for v in roi)
    x = min(max(x, 0), W - 1)
    y = min(max(y, 0), H - 1)
    w = min(max(w, 1), W - x)
    h = min(max(h, 1), H - y)
    return x, y, w, h


def resize_linear_roi(src: np.ndarray, rois, dH: int, dW: int) -> np.ndarray:
    """Crop then resize, per image: image n's clamped crop is cut out and
    resized with resize_linear as an image of its own (the random crop then
    resize of batched augmentation, hnwysp.cn news/129086 s7.2)."""
    src = _as_nhwc(src)
    N, H, W, C = src.shape
    out = np.empty((N, dH, dW, C), dtype=src.dtype)
    for n in range(N):
        x, y, w, h = clamp_roi(rois[n], H, W)
        out[n] = resize_linear(np.ascontiguousarray(src[n:n + 1, y:y + h, x:x + w]), dH, dW)[0]
    return out


NEAREST_MAPPINGS = {"half_pixel": 0, "floor": 1, "round": 2}


def resize_nearest(src: np.ndarray, dH: int, dW: int, rows=None,
                   mapping: str = "half_pixel") -> np.ndarray:
    """Nearest-neighbour resize of an NHWC array (any element type) to dH x dW.

    ``mapping``: "half_pixel" (default; pixel centres, rounded half up),
    "floor" (corner-aligned x = d * n_in / n_out, floored: the legacy nearest)
    or "round" (the same coordinate rounded half up, as hnwysp.cn news/129086
    s3.2's kernel does), each clamped to the image."""
    src = _as_nhwc(src)
    N, H, W, C = src.shape
    r0, r1 = _rows(N, dH, rows)
    full = np.empty((N * dH, dW, C), dtype=src.dtype)
    rc = _load().oracle_nearest_map(src.ctypes.data, full.ctypes.data, src.itemsize,
                                    N, H, W, C, dH, dW, r0, r1, NEAREST_MAPPINGS[mapping])
    if rc != 0:
        raise ValueError("oracle rejected arguments (code %d)" % rc)
    if rows is not None:
        return full[r0:r1].copy()
    return full.reshape(N, dH, dW, C)
