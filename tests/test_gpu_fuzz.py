"""GPU parity over a seeded random mix of every entry point.

Each case draws an operation (linear, nearest under its three mappings,
mirror / wrap borders, fused grey, fused normalisation, crop-then-resize), a
kernel family (MI_RESIZE_PATH auto / rowseg / direct), a dtype, a shape
(sizes 1-259, scale 0.08x-9x, some exact 2x and 2:1 cases; or wide, short
images up to 3199 wide) and sometimes a
misaligned source, and compares the result with the oracle: uint8 and
nearest bit-exact, float32 within 1e-5, normalised output within
1e-5 * max(1, |v|).  Every case prints its name before its GPU work.
"""
import os

import numpy as np
import pytest
import torch

import bilinear_image_resize_amd as R
import oracle
from bilinear_image_resize_amd.workloads import random_image

pytestmark = pytest.mark.gpu

OPS = ["linear", "nearest", "near_floor", "near_round", "mirror", "wrap", "grey", "norm", "roi"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R._load()
    yield
    torch.cuda.synchronize()


def _shape_wide(r):
    """Wide, short images (widths up to 3199, scale 0.3x-3x): rows of
    several wave segments, where the row-segment kernel's pixels-per-lane
    choice and its fill thresholds decide the launch."""
    N = int(r.choice([1, 2, 3, 5]))
    H, W = int(r.integers(1, 24)), int(r.integers(1, 3200))
    sy, sx = np.exp(r.uniform(np.log(0.3), np.log(3.0), size=2))
    return N, H, W, int(min(max(1, round(H * sy)), 40)), int(min(max(1, round(W * sx)), 3200))


def _shape(r):
    N = int(r.choice([1, 2, 3, 5]))
    H, W = (int(v) for v in r.integers(1, 260, size=2))
    sy, sx = np.exp(r.uniform(np.log(0.08), np.log(9.0), size=2))
    dH = int(min(max(1, round(H * sy)), 700))
    dW = int(min(max(1, round(W * sx)), 700))
    if r.random() < 0.15:
        dH, dW = (2 * H, 2 * W) if r.random() < 0.5 else (max(1, H // 2), max(1, W // 2))
    return N, H, W, dH, dW


def _run(r, op, path, monkeypatch, i, shape=_shape):
    monkeypatch.setenv("MI_RESIZE_PATH", path)
    N, H, W, dH, dW = shape(r)
    C = int(r.choice([3, 4])) if op == "grey" else int(r.choice([1, 3, 4]))
    dt = "u8" if op == "norm" else str(r.choice(["u8", "f32"]))
    s = random_image(r, (N, H, W, C), dt)
    print("case fuzz %d %s %s %s %s" % (i, op, path, dt, (N, H, W, C, dH, dW)), flush=True)
    tdt = torch.uint8 if dt == "u8" else torch.float32
    off = int(r.choice([0, 0, 1, 3]))              # elements: bytes for uint8, 4 B steps for float
    big = torch.empty(s.size + 64, dtype=tdt, device="cuda")
    src = big[off:off + s.size].view(s.shape)
    src.copy_(torch.from_numpy(s))
    if op == "grey":
        dst = torch.empty((N, dH, dW, 1), dtype=tdt, device="cuda")
        R.resize_linear_grey(src, dst)
        want = oracle.resize_linear_grey(s, dH, dW)
    elif op == "norm":
        dst = torch.empty((N, C, dH, dW), dtype=torch.float32, device="cuda")
        mean, std = [0.4, 0.5, 0.6, 0.5][:C], [0.2, 0.25, 0.3, 0.5][:C]
        R.resize_linear_normalize(src, dst, mean, std, layout="NCHW")
        want = oracle.resize_linear_normalize(s, dH, dW, 1 / 255.0, mean, std, "NCHW")
    elif op == "roi":
        rois = np.stack([r.integers(-5, W + 5, N), r.integers(-5, H + 5, N),
                         r.integers(-3, W + 8, N), r.integers(-3, H + 8, N)], 1).astype(np.int32)
        dst = torch.empty((N, dH, dW, C), dtype=tdt, device="cuda")
        R.resize_linear_roi(src, dst, torch.from_numpy(rois).cuda())
        want = oracle.resize_linear_roi(s, rois, dH, dW)
    else:
        dst = torch.empty((N, dH, dW, C), dtype=tdt, device="cuda")
        if op == "linear":
            R.resize_linear(src, dst)
            want = oracle.resize_linear(s, dH, dW)
        elif op == "nearest":
            R.resize_nearest(src, dst)
            want = oracle.resize_nearest(s, dH, dW)
        elif op in ("near_floor", "near_round"):
            m = op[5:]
            R.resize_nearest_mapping(src, dst, m)
            want = oracle.resize_nearest(s, dH, dW, mapping=m)
        else:
            R.resize_linear_border(src, dst, op)
            want = oracle.resize_linear(s, dH, dW, border=op)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    what = "fuzz %d %s %s %s %s" % (i, op, path, dt, (N, H, W, C, dH, dW))
    if op == "norm":
        assert (np.abs(got - want) <= 1e-5 * np.maximum(1, np.abs(want))).all(), what
    elif dt == "u8" or op.startswith("near"):
        assert np.array_equal(got, want), what
    else:
        assert float(np.abs(got.astype(np.float64) - want).max()) <= 1e-5, what


@pytest.mark.parametrize("block", range(3))
def test_random_mix(block, monkeypatch):
    r = np.random.default_rng(20251 + block)
    for i in range(300):
        _run(r, OPS[i % len(OPS)], ["auto", "rowseg", "direct"][int(r.integers(0, 3))],
             monkeypatch, 300 * block + i)


def test_random_mix_wide_rows(monkeypatch):
    r = np.random.default_rng(31337)
    for i in range(300):
        _run(r, OPS[i % len(OPS)], ["auto", "rowseg", "direct"][int(r.integers(0, 3))],
             monkeypatch, 900 + i, shape=_shape_wide)
