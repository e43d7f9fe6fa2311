"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no resize arithmetic: only the workload shapes and the
random-number recipes that fill the source images.  Both the HIP path's tests
and the CPU oracle's tests draw their inputs from here.

Workloads (all interleaved HWC, contiguous batch):

=====  ===============================  ============  =======  ==========
name   source N x H x W x C, dtype      destination   mode(s)  seed
=====  ===============================  ============  =======  ==========
small  1 x 48 x 64 x 1, uint8           72 x 96       linear   1001
4k     1 x 2160 x 3840 x 3, uint8       1080 x 1920   linear   1002
up2x   1 x 1080 x 1920 x 1, uint8       2160 x 3840   both     1003
thumb  256 x 480 x 640 x 3, uint8       224 x 224     linear   1004
rgbaf  1 x 4320 x 7680 x 4, float32     5927 x 3153   linear   1005
up15   1 x 1080 x 1920 x 3, uint8       1620 x 2880   both     1006
=====  ===============================  ============  =======  ==========

The "4k" frame (the 4K video frame of the pages' timing table, downscaled to
1080p) is smooth per-channel gradients plus uniform noise; the others are
uniform random bytes or uniform floats in [0, 1).  "up15" (a 1.5x
enlargement of a camera frame) is not one of the pages' timed
configurations; it measures the general enlargement path.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    H: int
    W: int
    C: int
    dtype: str          # "u8" or "f32"
    dH: int
    dW: int
    modes: tuple        # ("linear",) or ("linear", "nearest")
    seed: int
    content: str        # "uniform" or "gradient+noise"

    @property
    def src_shape(self):
        return (self.batch, self.H, self.W, self.C)

    @property
    def dst_shape(self):
        return (self.batch, self.dH, self.dW, self.C)

    @property
    def np_dtype(self):
        return np.uint8 if self.dtype == "u8" else np.float32

    @property
    def itemsize(self):
        return 1 if self.dtype == "u8" else 4

    @property
    def src_bytes(self):
        return self.batch * self.H * self.W * self.C * self.itemsize

    @property
    def dst_bytes(self):
        return self.batch * self.dH * self.dW * self.C * self.itemsize

    @property
    def dst_pixels(self):
        return self.batch * self.dH * self.dW


WORKLOADS = {
    w.name: w
    for w in (
        Workload("small", 1, 48, 64, 1, "u8", 72, 96, ("linear",), 1001, "uniform"),
        Workload("4k", 1, 2160, 3840, 3, "u8", 1080, 1920, ("linear",), 1002, "gradient+noise"),
        Workload("up2x", 1, 1080, 1920, 1, "u8", 2160, 3840, ("linear", "nearest"), 1003, "uniform"),
        Workload("thumb", 256, 480, 640, 3, "u8", 224, 224, ("linear",), 1004, "uniform"),
        Workload("rgbaf", 1, 4320, 7680, 4, "f32", 5927, 3153, ("linear",), 1005, "uniform"),
        Workload("up15", 1, 1080, 1920, 3, "u8", 1620, 2880, ("linear", "nearest"), 1006, "uniform"),
    )
}


def uniform_u8(shape, seed):
    """Independent uniform bytes in [0, 255]."""
    return np.random.default_rng(seed).integers(0, 256, size=shape, dtype=np.uint8)


def uniform_f32(shape, seed):
    """Independent uniform float32 values in [0, 1)."""
    return np.random.default_rng(seed).random(size=shape, dtype=np.float32)


def gradient_noise_u8(shape, seed):
    """Smooth per-channel gradients plus uniform noise, clipped to [0, 255].

    Channel k of every image is 255 * (a_k * x / (W-1) + (1 - a_k) * y / (H-1))
    with a_k uniform in [0, 1), plus independent integer noise in [-32, 32].
    """
    N, H, W, C = shape
    rng = np.random.default_rng(seed)
    a = rng.random(C)
    xs = np.linspace(0.0, 1.0, W) if W > 1 else np.zeros(1)
    ys = np.linspace(0.0, 1.0, H) if H > 1 else np.zeros(1)
    out = np.empty(shape, dtype=np.uint8)
    for n in range(N):
        noise = rng.integers(-32, 33, size=(H, W, C), dtype=np.int16)
        for k in range(C):
            g = np.rint(255.0 * (a[k] * xs[None, :] + (1.0 - a[k]) * ys[:, None]))
            out[n, :, :, k] = np.clip(g.astype(np.int16) + noise[:, :, k], 0, 255)
    return out


def make_source(w: Workload) -> np.ndarray:
    if w.dtype == "f32":
        return uniform_f32(w.src_shape, w.seed)
    if w.content == "gradient+noise":
        return gradient_noise_u8(w.src_shape, w.seed)
    return uniform_u8(w.src_shape, w.seed)


def random_image(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """Random image of the given NHWC shape for randomised parity cases."""
    if dtype == "u8":
        return rng.integers(0, 256, size=shape, dtype=np.uint8)
    return rng.random(size=shape, dtype=np.float32)
