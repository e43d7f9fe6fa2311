"""Linear (bilinear) and nearest-neighbour image resize on MI355X (gfx950).

The work is done by hand-written HIP kernels in ``libmi_resize.so``, reached
through its C ABI (``include/mi_resize.h``).  This module is a thin ctypes
binding with the same entry-point names: it checks and marshals arguments
(device pointers, sizes, the current HIP stream) and raises on a non-zero
status.  PyTorch supplies only device memory and streams; there is no CPU or
PyTorch fallback, and every call fails loudly if the library is not built.

    >>> import torch, bilinear_image_resize_amd as R
    >>> img = torch.randint(0, 256, (2160, 3840, 3), dtype=torch.uint8, device="cuda")
    >>> small = R.resize(img, (1080, 1920))              # linear, HWC in, HWC out
    >>> R.resize_linear(img, torch.empty_like(small))    # caller-owned output

Sizes are (height, width).  ``scale=`` sizes the output as
``(int(H * scale), int(W * scale))``, truncating like the OpenCV-style
driver in "From Prototype to Performance: Optimizing OpenCV Resize on Volcanic
GPUs" (section "Step 2: Make the GPU version correct first").
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "resize", "resize_linear", "resize_nearest", "resize_linear_normalize", "resize_linear_roi",
    "resize_linear_border",
    "resize_copy_bytes",
    "resize_status_string", "resize_abi_version", "library_path", "ResizeError",
    "U8", "F32",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmi_resize.so")

U8 = 0
F32 = 1
_ABI_VERSION = 6

_lib = None


class ResizeError(ValueError, RuntimeError):
    """A non-zero status from the C ABI, carrying resize_status_string's text.
    A ValueError (most statuses reject arguments) and a RuntimeError (a
    refused launch), so either kind of handler catches it."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, resize_status_string(status), status))


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            "libmi_resize.so is not built (expected at %s); run "
            "`python -c 'import __graft_entry__ as g; g.build()'` first" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, ci, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    for name in ("resize_linear", "resize_nearest"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, ci, ci, ci, ci, ci, ci, ci, vp]
        fn.restype = ci
    lib.resize_status_string.argtypes = [ci]
    lib.resize_status_string.restype = ctypes.c_char_p
    lib.resize_abi_version.argtypes = []
    lib.resize_abi_version.restype = ci
    lib.resize_copy_bytes.argtypes = [vp, vp, i64, vp]
    lib.resize_copy_bytes.restype = ci
    fp = ctypes.POINTER(ctypes.c_float)
    lib.resize_linear_normalize.argtypes = [vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_float,
                                            fp, fp, ci, vp]
    lib.resize_linear_normalize.restype = ci
    lib.resize_linear_roi.argtypes = [vp, vp, ci, ci, ci, ci, ci, vp, ci, ci, vp]
    lib.resize_linear_roi.restype = ci
    lib.resize_linear_border.argtypes = [vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, vp]
    lib.resize_linear_border.restype = ci
    lib.resize_nearest_mapping.argtypes = [vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, vp]
    lib.resize_nearest_mapping.restype = ci
    lib.resize_linear_grey.argtypes = [vp, vp, ci, ci, ci, ci, ci, ci, ci, vp]
    lib.resize_linear_grey.restype = ci
    if lib.resize_abi_version() != _ABI_VERSION:
        raise RuntimeError("libmi_resize.so ABI version %d, binding expects %d"
                           % (lib.resize_abi_version(), _ABI_VERSION))
    _lib = lib
    return lib


def resize_status_string(status: int) -> str:
    return _load().resize_status_string(int(status)).decode()


def resize_abi_version() -> int:
    return int(_load().resize_abi_version())


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nhwc(t, what):
    """(N, H, W, C) view of a contiguous HWC or NHWC CUDA tensor."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % what)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device, got %s" % (what, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (interleaved HWC / NHWC)" % what)
    if t.dim() == 3:
        return (1,) + tuple(t.shape)
    if t.dim() == 4:
        return tuple(t.shape)
    raise ValueError("%s must be HWC or NHWC, got shape %s" % (what, tuple(t.shape)))


def _dtype_code(t):
    import torch
    if t.dtype == torch.uint8:
        return U8
    if t.dtype == torch.float32:
        return F32
    raise TypeError("dtype must be torch.uint8 or torch.float32, got %s" % t.dtype)


def _call(name, src, dst, stream):
    N, H, W, C = _nhwc(src, "src")
    N2, dH, dW, C2 = _nhwc(dst, "dst")
    if (N2, C2) != (N, C):
        raise ValueError("src %s and dst %s differ in batch or channels"
                         % (tuple(src.shape), tuple(dst.shape)))
    if src.dim() != dst.dim():
        raise ValueError("src and dst must both be HWC or both NHWC")
    if src.dtype != dst.dtype:
        raise TypeError("src and dst dtypes differ")
    if src.device != dst.device:
        raise ValueError("src and dst are on different devices")
    fn = getattr(_load(), name)
    rc = fn(src.data_ptr(), dst.data_ptr(), N, H, W, C, _dtype_code(src), dH, dW,
            _stream_handle(stream, src.device))
    if rc != 0:
        raise ResizeError(rc, name)
    return dst


def resize_linear(src, dst, stream=None):
    """Linear resize of ``src`` into the caller-owned ``dst`` (same dtype and
    layout; the output size is dst's H x W).  Enqueued on ``stream`` (a
    torch.cuda.Stream or raw hipStream_t int; default: the current stream)."""
    return _call("resize_linear", src, dst, stream)


def resize_nearest(src, dst, stream=None):
    """Nearest-neighbour resize of ``src`` into ``dst``; see resize_linear."""
    return _call("resize_nearest", src, dst, stream)


LAYOUTS = {"NHWC": 0, "NCHW": 1}


def resize_linear_normalize(src, dst, mean, std, alpha=1.0 / 255.0, layout="NCHW", stream=None):
    """Linear resize of a uint8 HWC / NHWC tensor fused with normalisation
    into a caller-owned float32 ``dst``:  dst = (v * alpha - mean[c]) / std[c],
    v being exactly resize_linear's uint8 result.  ``layout`` "NCHW" (dst is
    (N,) C x dst_H x dst_W) or "NHWC" (dst is (N,) dst_H x dst_W x C)."""
    import torch
    N, H, W, C = _nhwc(src, "src")
    if src.dtype != torch.uint8:
        raise TypeError("src must be uint8")
    if not isinstance(dst, torch.Tensor) or dst.dtype != torch.float32:
        raise TypeError("dst must be a float32 tensor")
    if dst.device != src.device or not dst.is_contiguous():
        raise ValueError("dst must be contiguous and on src's device")
    if layout not in LAYOUTS:
        raise ValueError("layout must be 'NCHW' or 'NHWC'")
    shape = tuple(dst.shape) if dst.dim() == 4 else (1,) + tuple(dst.shape)
    if dst.dim() != src.dim() or len(shape) != 4:
        raise ValueError("dst must be batched exactly when src is")
    if layout == "NHWC":
        N2, dH, dW, C2 = shape
    else:
        N2, C2, dH, dW = shape
    if (N2, C2) != (N, C):
        raise ValueError("dst shape %s does not match src %s" % (tuple(dst.shape), tuple(src.shape)))
    mean = [float(v) for v in mean]
    std = [float(v) for v in std]
    if len(mean) != C or len(std) != C:
        raise ValueError("mean and std need one value per channel")
    fa = ctypes.c_float * C
    rc = _load().resize_linear_normalize(src.data_ptr(), dst.data_ptr(), N, H, W, C, dH, dW,
                                         float(alpha), fa(*mean), fa(*std), LAYOUTS[layout],
                                         _stream_handle(stream, src.device))
    if rc != 0:
        raise ResizeError(rc, "resize_linear_normalize")
    return dst


def resize_linear_roi(src, dst, rois, stream=None):
    """Batched crop-then-resize: image n's region ``rois[n] = (x, y, w, h)``
    (an int32 CUDA tensor of shape (N, 4), read on the device and clamped into
    the image) is resized linearly into ``dst[n]`` (same dtype, (N,) dst_H x
    dst_W x C)."""
    import torch
    N, H, W, C = _nhwc(src, "src")
    N2, dH, dW, C2 = _nhwc(dst, "dst")
    if (N2, C2) != (N, C) or src.dim() != dst.dim() or src.dtype != dst.dtype:
        raise ValueError("src %s / dst %s mismatch" % (tuple(src.shape), tuple(dst.shape)))
    if (not isinstance(rois, torch.Tensor) or rois.dtype != torch.int32 or rois.device != src.device
            or not rois.is_contiguous() or tuple(rois.shape) != (N, 4)):
        raise ValueError("rois must be a contiguous int32 tensor of shape (%d, 4) on %s" % (N, src.device))
    rc = _load().resize_linear_roi(src.data_ptr(), dst.data_ptr(), N, H, W, C, _dtype_code(src),
                                   rois.data_ptr(), dH, dW, _stream_handle(stream, src.device))
    if rc != 0:
        raise ResizeError(rc, "resize_linear_roi")
    return dst


BORDERS = {"clamp": 0, "mirror": 1, "wrap": 2}


def resize_linear_border(src, dst, border="mirror", stream=None):
    """Linear resize with a border rule for coordinates beyond the outermost
    pixel centres: "clamp" (as resize_linear), "mirror" (reflect about the
    edge pixel centres) or "wrap" (periodic image)."""
    if border not in BORDERS:
        raise ValueError("border must be one of %s" % sorted(BORDERS))
    N, H, W, C = _nhwc(src, "src")
    N2, dH, dW, C2 = _nhwc(dst, "dst")
    if (N2, C2) != (N, C) or src.dim() != dst.dim() or src.dtype != dst.dtype:
        raise ValueError("src %s / dst %s mismatch" % (tuple(src.shape), tuple(dst.shape)))
    rc = _load().resize_linear_border(src.data_ptr(), dst.data_ptr(), N, H, W, C, _dtype_code(src),
                                      dH, dW, BORDERS[border], _stream_handle(stream, src.device))
    if rc != 0:
        raise ResizeError(rc, "resize_linear_border")
    return dst


NEAREST_MAPPINGS = {"half_pixel": 0, "floor": 1, "round": 2}


def resize_nearest_mapping(src, dst, mapping="floor", stream=None):
    """Nearest-neighbour resize with a coordinate mapping: "half_pixel" (as
    resize_nearest), "floor" (floor(d * in / out), the legacy nearest) or
    "round" (floor(d * in / out + 1/2)); see include/mi_resize.h."""
    if mapping not in NEAREST_MAPPINGS:
        raise ValueError("mapping must be one of %s" % sorted(NEAREST_MAPPINGS))
    N, H, W, C = _nhwc(src, "src")
    N2, dH, dW, C2 = _nhwc(dst, "dst")
    if (N2, C2) != (N, C) or src.dim() != dst.dim() or src.dtype != dst.dtype:
        raise ValueError("src %s / dst %s mismatch" % (tuple(src.shape), tuple(dst.shape)))
    rc = _load().resize_nearest_mapping(src.data_ptr(), dst.data_ptr(), N, H, W, C, _dtype_code(src),
                                        dH, dW, NEAREST_MAPPINGS[mapping],
                                        _stream_handle(stream, src.device))
    if rc != 0:
        raise ResizeError(rc, "resize_nearest_mapping")
    return dst


def resize_linear_grey(src, dst, stream=None):
    """RGB(A) -> grey (BT.601 luma weights) fused with the linear resize:
    ``src`` (N,) H x W x 3|4, ``dst`` (N,) dst_H x dst_W x 1, same dtype."""
    N, H, W, C = _nhwc(src, "src")
    N2, dH, dW, C2 = _nhwc(dst, "dst")
    if N2 != N or C2 != 1 or src.dim() != dst.dim() or src.dtype != dst.dtype:
        raise ValueError("src %s / dst %s mismatch (dst needs one channel)"
                         % (tuple(src.shape), tuple(dst.shape)))
    if src.device != dst.device:
        raise ValueError("src and dst are on different devices")
    rc = _load().resize_linear_grey(src.data_ptr(), dst.data_ptr(), N, H, W, C, _dtype_code(src),
                                    dH, dW, _stream_handle(stream, src.device))
    if rc != 0:
        raise ResizeError(rc, "resize_linear_grey")
    return dst


def resize(src, size=None, mode: str = "linear", scale=None, stream=None):
    """Allocate the output and resize.  ``size=(dst_H, dst_W)`` or ``scale``."""
    import torch
    N, H, W, C = _nhwc(src, "src")
    if (size is None) == (scale is None):
        raise ValueError("give exactly one of size=(H, W) or scale=")
    if size is None:
        size = (int(H * scale), int(W * scale))
    dH, dW = int(size[0]), int(size[1])
    shape = (dH, dW, C) if src.dim() == 3 else (N, dH, dW, C)
    dst = torch.empty(shape, dtype=src.dtype, device=src.device)
    if mode == "linear":
        return resize_linear(src, dst, stream)
    if mode == "nearest":
        return resize_nearest(src, dst, stream)
    raise ValueError("mode must be 'linear' or 'nearest'")


def resize_copy_bytes(src, dst, nbytes=None, stream=None):
    """Plain device copy of ``nbytes`` (default: all of src) with 16-byte
    accesses: the bandwidth calibration kernel."""
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    if nbytes > src.numel() * src.element_size() or nbytes > dst.numel() * dst.element_size():
        raise ValueError("nbytes exceeds a buffer")
    rc = _load().resize_copy_bytes(src.data_ptr(), dst.data_ptr(), int(nbytes),
                                   _stream_handle(stream, src.device))
    if rc != 0:
        raise ResizeError(rc, "resize_copy_bytes")
    return dst
