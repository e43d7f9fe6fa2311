"""GPU parity: the HIP path against the CPU oracle, element by element.

uint8 results must be bit-exact; float32 results within 1e-5 absolute for
inputs in [0, 1] (the tolerance the resize is specified to).  Every call goes
through the C ABI (via the ctypes binding).  Each case prints its name before
its GPU work so a failing run names the case.
"""
import os
import sys

import numpy as np
import pytest
import torch

import bilinear_image_resize_amd as R
import oracle
from bilinear_image_resize_amd.workloads import WORKLOADS, make_source, random_image

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R._load()
    yield
    torch.cuda.synchronize()


def run_gpu(src_np, dH, dW, mode="linear", stream=None):
    src = torch.from_numpy(src_np).cuda()
    N, H, W, C = src.shape
    dst = torch.empty((N, dH, dW, C), dtype=src.dtype, device="cuda")
    if mode == "linear":
        R.resize_linear(src, dst, stream=stream)
    else:
        R.resize_nearest(src, dst, stream=stream)
    torch.cuda.synchronize()
    return dst.cpu().numpy()


def run_oracle(src_np, dH, dW, mode="linear"):
    if mode == "linear":
        return oracle.resize_linear(src_np, dH, dW)
    return oracle.resize_nearest(src_np, dH, dW)


def assert_parity(got, want, what):
    assert got.shape == want.shape, what
    if want.dtype == np.uint8 or want.dtype != np.float32:
        bad = np.argwhere(got != want)
        assert bad.size == 0, "%s: %d mismatches, first at %s (got %s want %s)" % (
            what, len(bad), tuple(bad[0]), got[tuple(bad[0])], want[tuple(bad[0])])
    else:
        err = np.abs(got.astype(np.float64) - want.astype(np.float64))
        assert np.isfinite(got).all(), what
        assert err.max() <= F32_TOL, "%s: max abs err %g at %s" % (
            what, err.max(), np.unravel_index(err.argmax(), err.shape))


# --------------------------------------------------------------------------
# the five workloads at their full sizes, in the launch configuration the
# benchmark times (default dispatch), and again forced onto the generic kernel
# --------------------------------------------------------------------------
CASES = [(w.name, m) for w in WORKLOADS.values() for m in w.modes]


@pytest.mark.parametrize("name,mode", CASES)
def test_workload_full_size(name, mode):
    w = WORKLOADS[name]
    say("case workload=%s mode=%s src=%s dst=%s" % (name, mode, w.src_shape, w.dst_shape))
    s = make_source(w)
    assert_parity(run_gpu(s, w.dH, w.dW, mode), run_oracle(s, w.dH, w.dW, mode),
                  "%s/%s" % (name, mode))


PATHS = ["rowseg", "direct", "tile"]   # MI_RESIZE_PATH: force one kernel family


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name,mode", CASES)
def test_workload_forced_path(name, mode, path, monkeypatch):
    w = WORKLOADS[name]
    monkeypatch.setenv("MI_RESIZE_PATH", path)
    say("case workload=%s mode=%s path=%s" % (name, mode, path))
    s = make_source(w)
    assert_parity(run_gpu(s, w.dH, w.dW, mode), run_oracle(s, w.dH, w.dW, mode),
                  "%s/%s/%s" % (name, mode, path))


# --------------------------------------------------------------------------
# randomised shapes: dims 1..300, scales ~0.1..8, C in {1,3,4}, N in {1,3}
# --------------------------------------------------------------------------
def random_case(r):
    N = int(r.choice([1, 3]))
    C = int(r.choice([1, 3, 4]))
    H, W = (int(v) for v in r.integers(1, 301, size=2))
    sy, sx = np.exp(r.uniform(np.log(0.1), np.log(8.0), size=2))
    dH = int(min(max(1, round(H * sy)), 600))
    dW = int(min(max(1, round(W * sx)), 600))
    return N, H, W, C, dH, dW


@pytest.mark.parametrize("path", ["auto"] + PATHS)
@pytest.mark.parametrize("dtype", ["u8", "f32"])
@pytest.mark.parametrize("mode", ["linear", "nearest"])
def test_random_shapes(dtype, mode, path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("MI_RESIZE_PATH", path)
    r = np.random.default_rng(2024 + (dtype == "f32") + 2 * (mode == "nearest") + 4 * (["auto"] + PATHS).index(path))
    for i in range(60):
        N, H, W, C, dH, dW = random_case(r)
        say("case random %s %s %s #%d N=%d H=%d W=%d C=%d -> %dx%d" % (dtype, mode, path, i, N, H, W, C, dH, dW))
        s = random_image(r, (N, H, W, C), dtype)
        assert_parity(run_gpu(s, dH, dW, mode), run_oracle(s, dH, dW, mode),
                      "random #%d %s" % (i, (N, H, W, C, dH, dW)))


@pytest.mark.parametrize("path", ["auto"] + PATHS)
@pytest.mark.parametrize("op", ["grey", "roi", "mirror", "wrap"])
def test_random_shapes_other_entry_points(op, path, monkeypatch):
    """The fused grey output, per-image regions (some partly or wholly
    outside the image, clamped by both sides) and the mirror / wrap borders
    on random shapes, uint8 and float32, on every kernel family."""
    if path != "auto":
        monkeypatch.setenv("MI_RESIZE_PATH", path)
    r = np.random.default_rng(4242 + 8 * ["grey", "roi", "mirror", "wrap"].index(op) +
                              (["auto"] + PATHS).index(path))
    for i in range(30):
        N, H, W, C, dH, dW = random_case(r)
        if op == "grey" and C == 1:
            C = 3
        dtype = "u8" if r.random() < 0.7 else "f32"
        s = random_image(r, (N, H, W, C), dtype)
        src = torch.from_numpy(s).cuda()
        dC = 1 if op == "grey" else C
        dst = torch.empty((N, dH, dW, dC), dtype=src.dtype, device="cuda")
        say("case random %s %s %s #%d N=%d H=%d W=%d C=%d -> %dx%d" % (op, dtype, path, i, N, H, W, C, dH, dW))
        if op == "grey":
            R.resize_linear_grey(src, dst)
            want = oracle.resize_linear_grey(s, dH, dW)
        elif op == "roi":
            rois = np.array([(int(r.integers(-3, W)), int(r.integers(-3, H)),
                              int(r.integers(0, W + 4)), int(r.integers(0, H + 4)))
                             for _ in range(N)], dtype=np.int32)
            R.resize_linear_roi(src, dst, torch.from_numpy(rois).cuda())
            want = oracle.resize_linear_roi(s, rois, dH, dW)
        else:
            R.resize_linear_border(src, dst, border=op)
            want = oracle.resize_linear(s, dH, dW, border=op)
        torch.cuda.synchronize()
        assert_parity(dst.cpu().numpy().reshape(want.shape), want,
                      "random %s #%d %s" % (op, i, (N, H, W, C, dH, dW, dtype)))


# --------------------------------------------------------------------------
# exact 2:1 downscale (its own kernel) for every channel count, ragged batch,
# and the shapes just off its conditions (which take the generic kernel)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("C", [1, 3, 4])
def test_half_downscale_shapes(C):
    r = np.random.default_rng(77 + C)
    for (N, dH, dW) in ((1, 1, 16), (3, 5, 32), (2, 17, 48), (1, 64, 1920), (5, 3, 16 * 37),
                        (1, 9, 15), (2, 4, 17), (1, 1, 1), (1, 7, 31)):
        say("case half C=%d N=%d dst=%dx%d" % (C, N, dH, dW))
        s = random_image(r, (N, 2 * dH, 2 * dW, C), "u8")
        assert_parity(run_gpu(s, dH, dW), run_oracle(s, dH, dW), "half %s" % ((C, N, dH, dW),))


@pytest.mark.parametrize("C", [1, 3, 4])
def test_half_downscale_random_shapes(C):
    """Seeded random shapes that the exact 2:1 kernel takes (output widths a
    multiple of 16, 8 or 4 for 1, 3 or 4 channels): several 256- or
    1024-pixel segments per row with a partial last one, odd row counts and
    batches; for 3 and 4 channels also the grey output."""
    q = {1: 16, 3: 8, 4: 4}[C]
    r = np.random.default_rng(5050 + C)
    for i in range(40):
        N = int(r.integers(1, 4))
        dH = int(r.integers(1, 40))
        dW = q * int(r.integers(1, 2200 // q))
        s = random_image(r, (N, 2 * dH, 2 * dW, C), "u8")
        say("case half random %d C=%d N=%d dst=%dx%d" % (i, C, N, dH, dW))
        assert_parity(run_gpu(s, dH, dW), run_oracle(s, dH, dW), "half random %s" % ((C, N, dH, dW),))
        if C >= 3:
            src = torch.from_numpy(s).cuda()
            dst = torch.empty((N, dH, dW, 1), dtype=src.dtype, device="cuda")
            R.resize_linear_grey(src, dst)
            torch.cuda.synchronize()
            assert_parity(dst.cpu().numpy(), oracle.resize_linear_grey(s, dH, dW),
                          "half grey random %s" % ((C, N, dH, dW),))


# --------------------------------------------------------------------------
# exact 2x upscale (its own kernel): channel counts, batches, one-row and
# one-chunk images, and widths that fall back to the generic kernels
# --------------------------------------------------------------------------
@pytest.mark.parametrize("C", [1, 3, 4])
def test_double_upscale_shapes(C):
    r = np.random.default_rng(91 + C)
    # (1, 3, 4) and (2, 2, 4): for 4 channels a row of a single chunk, which
    # the linear 2x kernel loads without its one-load window; W = 2 chunks
    # (16 px for 1 and 3 channels, 8 for 4) has only a start and an end lane
    for (N, H, W) in ((1, 1, 16), (2, 3, 32), (3, 17, 48), (1, 64, 1920), (1, 2, 8), (1, 1, 1),
                      (2, 5, 24), (1, 9, 17), (4, 1, 160), (1, 3, 4), (2, 2, 4)):
        s = random_image(r, (N, H, W, C), "u8")
        for mode in ("linear", "nearest"):
            say("case up2 %s C=%d N=%d src=%dx%d" % (mode, C, N, H, W))
            assert_parity(run_gpu(s, 2 * H, 2 * W, mode), run_oracle(s, 2 * H, 2 * W, mode),
                          "up2 %s %s" % (mode, (C, N, H, W)))


@pytest.mark.parametrize("dtype", ["u8", "f32"])
def test_rowseg_rgb_enlargements(dtype, monkeypatch):
    """RGB enlargements forced onto the row-segment kernel (float ones
    take the direct kernel by default): output widths with rows on 16-byte
    boundaries and others, several segments per row with a partial last
    one, batches, and shapes that only just enlarge."""
    monkeypatch.setenv("MI_RESIZE_PATH", "rowseg")
    q = 16 if dtype == "u8" else 4
    r = np.random.default_rng(6060 + (dtype == "f32"))
    shapes = [(1, 37, 50, 80, 32 * q), (2, 9, 11, 20, 5 * q), (1, 100, 100, 101, 25 * q),
              (3, 20, 30, 45, 45), (1, 64, 300, 70, 81 * q), (1, 5, 7, 9, 3 * q + 1)]
    for _ in range(12):
        N, H, W = int(r.integers(1, 3)), int(r.integers(1, 60)), int(r.integers(1, 300))
        dH, dW = H + int(r.integers(0, 60)), q * max(1, (W + int(r.integers(1, 200))) // q)
        shapes.append((N, H, W, dH, dW))
    for mode in ("linear", "nearest"):
        for i, (N, H, W, dH, dW) in enumerate(shapes):
            say("case rowseg rgb enlarge %s %s #%d %s" % (dtype, mode, i, (N, H, W, dH, dW)))
            s = random_image(r, (N, H, W, 3), dtype)
            assert_parity(run_gpu(s, dH, dW, mode), run_oracle(s, dH, dW, mode),
                          "rowseg rgb enlarge %s %s %s" % (dtype, mode, (N, H, W, dH, dW)))


def test_rowseg_lane_widths(monkeypatch):
    """The row-segment kernel's output pixels per lane follow the output
    width: 16, 8 or 4 for one-channel uint8 (by how full the row leaves its
    wave segments), 8 instead of 4 for wide uint8 RGB / RGBA and
    one-channel float rows that shrink little or grow, and for float RGB
    nearest rows that shrink by at most 2.1 (the last three float RGB cases:
    8, 8 and, shrinking 2.7, 4 under nearest; 4 under linear).  Each shape below
    lands on one of those choices, with full, ragged and nearly full last
    segments; linear and nearest."""
    monkeypatch.setenv("MI_RESIZE_PATH", "rowseg")
    r = np.random.default_rng(8181)
    cases = [  # (dtype, C, N, H, W, dH, dW)
        ("u8", 1, 2, 11, 640, 7, 224), ("u8", 1, 1, 9, 2100, 5, 700),
        ("u8", 1, 1, 8, 3000, 6, 1900), ("u8", 1, 2, 9, 1920, 6, 1280),
        ("u8", 1, 1, 7, 200, 5, 96), ("u8", 1, 1, 5, 1500, 9, 2047),
        ("u8", 3, 1, 9, 3840, 6, 2560), ("u8", 3, 1, 6, 1920, 11, 3000),
        ("u8", 3, 2, 7, 1500, 5, 1030), ("u8", 3, 1, 8, 3825, 5, 2550),
        ("u8", 3, 1, 6, 2560, 4, 2040), ("u8", 4, 1, 6, 2560, 4, 2040),
        ("u8", 4, 1, 9, 3000, 6, 2048), ("u8", 4, 1, 5, 1500, 8, 2000),
        ("f32", 1, 1, 9, 1920, 6, 1280), ("f32", 1, 1, 5, 2000, 9, 2560),
        ("f32", 1, 2, 7, 1600, 5, 1021),
        ("f32", 3, 1, 7, 3840, 5, 1900), ("f32", 3, 2, 6, 1500, 4, 1270),
        ("f32", 3, 1, 5, 3000, 4, 1100),
    ]
    for mode in ("linear", "nearest"):
        for (dt, C, N, H, W, dH, dW) in cases:
            say("case rowseg lanes %s %s %s" % (mode, dt, (C, N, H, W, dH, dW)))
            s = random_image(r, (N, H, W, C), dt)
            assert_parity(run_gpu(s, dH, dW, mode), run_oracle(s, dH, dW, mode),
                          "rowseg lanes %s %s %s" % (mode, dt, (C, N, H, W, dH, dW)))


@pytest.mark.parametrize("C", [3, 4])
def test_direct_float_enlargements(C):
    """Float RGB / RGBA enlargements take the direct kernels: whole 16-byte
    pixels (RGBA) stored with the non-temporal hint, and RGB rows that start
    on 16-byte boundaries (widths a multiple of 4) written through LDS as
    16-byte pieces; other RGB widths store three floats per lane.  Widths
    leave partial last waves and workgroups; linear and nearest."""
    r = np.random.default_rng(7070 + C)
    shapes = [(1, 30, 40, 45, 64), (1, 30, 40, 45, 68), (2, 17, 33, 40, 100), (1, 9, 50, 13, 257),
              (3, 5, 7, 11, 12), (1, 64, 64, 96, 256), (1, 2, 3, 3, 4)]
    for _ in range(10):
        N, H, W = int(r.integers(1, 3)), int(r.integers(1, 50)), int(r.integers(1, 300))
        shapes.append((N, H, W, H + int(r.integers(0, 50)), W + int(r.integers(1, 300))))
    for mode in ("linear", "nearest"):
        for i, (N, H, W, dH, dW) in enumerate(shapes):
            say("case direct float enlarge C=%d %s #%d %s" % (C, mode, i, (N, H, W, dH, dW)))
            s = random_image(r, (N, H, W, C), "f32")
            assert_parity(run_gpu(s, dH, dW, mode), run_oracle(s, dH, dW, mode),
                          "direct float enlarge C=%d %s %s" % (C, mode, (N, H, W, dH, dW)))


@pytest.mark.parametrize("C", [1, 3, 4])
def test_double_upscale_random_shapes(C):
    """Seeded random shapes that the exact 2x kernels take (widths a multiple
    of 16): row counts around the waves per workgroup, several 64-chunk
    segments per row with a partial last one, and batches."""
    r = np.random.default_rng(4040 + C)
    for i in range(40):
        N = int(r.integers(1, 4))
        H = int(r.integers(1, 70))
        W = 16 * int(r.integers(1, 21))
        s = random_image(r, (N, H, W, C), "u8")
        for mode in ("linear", "nearest"):
            say("case up2 random %d %s C=%d N=%d src=%dx%d" % (i, mode, C, N, H, W))
            assert_parity(run_gpu(s, 2 * H, 2 * W, mode), run_oracle(s, 2 * H, 2 * W, mode),
                          "up2 random %s %s" % (mode, (C, N, H, W)))


# --------------------------------------------------------------------------
# degenerate and extreme shapes
# --------------------------------------------------------------------------
EDGE = [
    (1, 1, 1, 1, 1, 1), (1, 1, 1, 3, 7, 9), (1, 5, 7, 4, 1, 1), (1, 1, 300, 3, 1, 41),
    (1, 300, 1, 1, 53, 1), (2, 1, 1, 4, 33, 65), (1, 3, 3, 1, 600, 600), (1, 600, 600, 3, 2, 3),
    (1, 2, 65535, 1, 3, 40000), (1, 40000, 2, 1, 65535, 3), (1, 1, 65535, 4, 1, 65535),
    (4, 13, 17, 3, 13, 17), (1, 8, 8, 3, 8, 16), (1, 8, 8, 3, 16, 8),
    (7, 31, 33, 3, 61, 67), (1, 1000, 10, 1, 3, 999),
    (1, 4, 4000, 3, 2, 37), (1, 3, 5000, 4, 3, 7), (2, 9, 1025, 1, 5, 1023), (1, 5, 1024, 1, 7, 1025),
    (1, 6, 257, 3, 4, 255), (3, 17, 129, 4, 9, 131),
    # the widest rows of the exact 2x and 2:1 kernels (uint8) and of the
    # float RGB rows staged through LDS on the direct kernels
    (1, 2, 32760, 1, 4, 65520), (1, 4, 65504, 3, 2, 32752), (1, 2, 20000, 3, 3, 65532),
    # coprime near-maximum lengths: coordinate quotients near 2^16 over
    # denominators near 2^17, where the division's estimate is least precise
    (1, 2, 65521, 3, 3, 65519), (1, 65519, 2, 1, 65521, 3),
]


@pytest.mark.parametrize("path", ["auto"] + PATHS)
@pytest.mark.parametrize("dtype", ["u8", "f32"])
@pytest.mark.parametrize("mode", ["linear", "nearest"])
def test_edge_shapes(dtype, mode, path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("MI_RESIZE_PATH", path)
    r = np.random.default_rng(99)
    for (N, H, W, C, dH, dW) in EDGE:
        say("case edge %s %s %s %s" % (dtype, mode, path, (N, H, W, C, dH, dW)))
        s = random_image(r, (N, H, W, C), dtype)
        assert_parity(run_gpu(s, dH, dW, mode), run_oracle(s, dH, dW, mode),
                      "edge %s" % ((N, H, W, C, dH, dW),))


# --------------------------------------------------------------------------
# 11-bit weight ties: an odd source length resized to a multiple of 2048
# (or an even one with the right residue, 6 -> 4096) puts 2048 u exactly on
# k + 1/2, which the resize rounds half up.  Every kernel family that takes
# general scales must round those the same way as the oracle.
# --------------------------------------------------------------------------
TIE_SHAPES = [
    (1, 3, 5, 2048, 2048),       # ties on both axes at almost every sample
    (1, 2, 6, 4, 4096),          # 6 -> 4096: ties along x at every interior sample
    (3, 7, 2049, 6, 2048),       # ties along x only, a slight downscale
    (1, 2047, 9, 2048, 16),      # ties along y only
]


@pytest.mark.parametrize("C", [1, 3, 4])
@pytest.mark.parametrize("dtype", ["u8", "f32"])
def test_weight_tie_shapes(dtype, C, monkeypatch):
    r = np.random.default_rng(4242 + C)
    shapes = TIE_SHAPES + ([(1, 1081, 1921, 2048, 2048)] if (dtype, C) == ("u8", 3) else [])
    for (N, H, W, dH, dW) in shapes:
        s = random_image(r, (N, H, W, C), dtype)
        want = run_oracle(s, dH, dW)
        for path in ["auto"] + PATHS:
            if path == "auto":
                monkeypatch.delenv("MI_RESIZE_PATH", raising=False)
            else:
                monkeypatch.setenv("MI_RESIZE_PATH", path)
            say("case tie %s C=%d %s %s" % (dtype, C, path, (N, H, W, dH, dW)))
            assert_parity(run_gpu(s, dH, dW), want,
                          "tie %s C=%d %s %s" % (dtype, C, path, (N, H, W, dH, dW)))


def test_golden_hand_cases():
    import json
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")
    for c in json.load(open(path))["cases"]:
        say("case golden %s" % c["name"])
        a = np.array(c["src"], dtype=np.uint8)
        s = a[None, :, :, None] if a.ndim == 2 else a[None]
        dH, dW = c["dst_hw"]
        m = c["mode"]
        if m in ("linear", "nearest"):
            got = run_gpu(s, dH, dW, m)[0, :, :, 0]
        else:
            src = torch.from_numpy(s).cuda()
            C = 1 if m == "grey" else s.shape[3]
            dst = torch.empty((1, dH, dW, C), dtype=torch.uint8, device="cuda")
            if m == "grey":
                R.resize_linear_grey(src, dst)
            else:
                R.resize_nearest_mapping(src, dst, mapping=m[len("nearest_"):])
            torch.cuda.synchronize()
            got = dst.cpu().numpy()[0, :, :, 0]
        assert got.tolist() == c["expected"], c["name"]


def test_batch_of_tiny_images():
    r = np.random.default_rng(5)
    s = random_image(r, (1000, 3, 2, 3), "u8")
    say("case tiny batch 1000x3x2x3 -> 5x7")
    assert_parity(run_gpu(s, 5, 7), run_oracle(s, 5, 7), "tiny batch")


# --------------------------------------------------------------------------
# uint8 row enlargements large enough for the tiled kernel under the default
# path: 16-row tiles (about 700 or more) and 8-row tiles, batches, ragged
# last tiles in both directions, one, three and four channels
# --------------------------------------------------------------------------
TILE_SHAPES = [
    (4, 300, 500, 3, 800, 1201),     # 16-row tiles
    (2, 300, 500, 3, 701, 1100),     # 8-row tiles
    (1, 500, 900, 4, 1000, 1803),
    (3, 400, 600, 1, 1003, 1500),
    (2, 600, 800, 1, 1500, 2000),    # 16-row tiles, one channel
    (2, 123, 1000, 3, 1300, 1001),   # rows enlarge, columns nearly the same
    (1, 700, 97, 3, 2100, 291),      # narrow rows, a single column segment
]


@pytest.mark.parametrize("shape", TILE_SHAPES)
def test_tile_enlargements(shape, monkeypatch):
    monkeypatch.delenv("MI_RESIZE_PATH", raising=False)
    N, H, W, C, dH, dW = shape
    say("case tile %s" % (shape,))
    r = np.random.default_rng(7 + sum(shape))
    s = random_image(r, (N, H, W, C), "u8")
    assert_parity(run_gpu(s, dH, dW, "linear"), run_oracle(s, dH, dW, "linear"),
                  "tile %s" % (shape,))


# one-channel and RGBA float32 row enlargements: the float tiles (8 and 16 rows)
@pytest.mark.parametrize("shape", [(2, 300, 500, 1, 800, 1300), (4, 300, 600, 1, 900, 1601),
                                   (1, 300, 400, 4, 700, 901), (2, 400, 400, 4, 900, 900)])
def test_tile_enlargements_f32(shape, monkeypatch):
    monkeypatch.delenv("MI_RESIZE_PATH", raising=False)
    N, H, W, C, dH, dW = shape
    say("case tile f32 %s" % (shape,))
    s = random_image(np.random.default_rng(3 + sum(shape)), (N, H, W, C), "f32")
    assert_parity(run_gpu(s, dH, dW, "linear"), run_oracle(s, dH, dW, "linear"),
                  "tile f32 %s" % (shape,))


@pytest.mark.parametrize("shape", [(1, 540, 960, 3, 1080, 1700),     # 8-row tiles
                                   (2, 600, 800, 4, 1200, 1601)])   # 16-row tiles
def test_tile_grey_enlargements(shape, monkeypatch):
    monkeypatch.delenv("MI_RESIZE_PATH", raising=False)
    N, H, W, C, dH, dW = shape
    say("case tile grey %s" % (shape,))
    s = random_image(np.random.default_rng(5 + sum(shape)), (N, H, W, C), "u8")
    src = torch.from_numpy(s).cuda()
    dst = torch.empty((N, dH, dW, 1), dtype=src.dtype, device="cuda")
    R.resize_linear_grey(src, dst)
    torch.cuda.synchronize()
    assert_parity(dst.cpu().numpy(), oracle.resize_linear_grey(s, dH, dW), "tile grey %s" % (shape,))


# --------------------------------------------------------------------------
# misaligned buffers take the scalar paths; results must not change
# --------------------------------------------------------------------------
@pytest.mark.parametrize("path", ["auto"] + PATHS)
@pytest.mark.parametrize("dtype", ["u8", "f32"])
@pytest.mark.parametrize("mode", ["linear", "nearest"])
def test_misaligned_buffers(dtype, mode, path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("MI_RESIZE_PATH", path)
    r = np.random.default_rng(11)
    es = 1 if dtype == "u8" else 4
    for (N, H, W, C, dH, dW) in ((1, 64, 64, 4, 32, 32), (2, 40, 64, 3, 20, 32), (1, 33, 47, 1, 70, 20),
                                 (1, 400, 700, 3, 800, 1400)):   # the last: a tiled enlargement
        for off in ((1, 3) if dtype == "u8" else (1, 2)):
            say("case misaligned %s %s off=%d %s" % (dtype, mode, off, (N, H, W, C, dH, dW)))
            s_np = random_image(r, (N, H, W, C), dtype)
            tdt = torch.uint8 if dtype == "u8" else torch.float32
            n_src, n_dst = s_np.size, N * dH * dW * C
            src_buf = torch.empty(n_src + 8, dtype=tdt, device="cuda")
            dst_buf = torch.empty(n_dst + 8, dtype=tdt, device="cuda")
            src = src_buf[off:off + n_src].view(N, H, W, C)
            dst = dst_buf[off:off + n_dst].view(N, dH, dW, C)
            assert src.data_ptr() % 16 == off * es
            src.copy_(torch.from_numpy(s_np))
            (R.resize_linear if mode == "linear" else R.resize_nearest)(src, dst)
            torch.cuda.synchronize()
            assert_parity(dst.cpu().numpy(), run_oracle(s_np, dH, dW, mode), "misaligned")


# --------------------------------------------------------------------------
# nothing is written outside dst: canary bytes on both sides
# --------------------------------------------------------------------------
@pytest.mark.parametrize("path", ["auto"] + PATHS)
@pytest.mark.parametrize("dtype", ["u8", "f32"])
def test_guard_bands(dtype, path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("MI_RESIZE_PATH", path)
    r = np.random.default_rng(12)
    tdt = torch.uint8 if dtype == "u8" else torch.float32
    pad = 4096
    for (N, H, W, C, dH, dW) in ((1, 100, 64, 3, 50, 32), (2, 37, 53, 4, 71, 29),
                                 (1, 64, 96, 1, 32, 48), (3, 16, 16, 3, 8, 8)):
        for mode in ("linear", "nearest"):
            say("case guard %s %s %s" % (dtype, mode, (N, H, W, C, dH, dW)))
            s_np = random_image(r, (N, H, W, C), dtype)
            n = N * dH * dW * C
            buf = torch.full((n + 2 * pad,), 77, dtype=tdt, device="cuda")
            dst = buf[pad:pad + n].view(N, dH, dW, C)
            (R.resize_linear if mode == "linear" else R.resize_nearest)(
                torch.from_numpy(s_np).cuda(), dst)
            torch.cuda.synchronize()
            host = buf.cpu().numpy()
            assert (host[:pad] == 77).all() and (host[pad + n:] == 77).all()
            assert_parity(host[pad:pad + n].reshape(N, dH, dW, C),
                          run_oracle(s_np, dH, dW, mode), "guard")


# --------------------------------------------------------------------------
# a non-default stream, and HWC (unbatched) tensors through resize()
# --------------------------------------------------------------------------
def test_side_stream_and_hwc():
    r = np.random.default_rng(13)
    s_np = random_image(r, (1, 480, 640, 3), "u8")
    st = torch.cuda.Stream()
    src = torch.from_numpy(s_np[0]).cuda()
    torch.cuda.synchronize()
    say("case side stream")
    with torch.cuda.stream(st):
        out = R.resize(src, (224, 224))
    st.synchronize()
    assert out.shape == (224, 224, 3)
    assert_parity(out.cpu().numpy()[None], oracle.resize_linear(s_np, 224, 224), "stream")
    out2 = R.resize(src, scale=0.5, mode="nearest")
    torch.cuda.synchronize()
    assert out2.shape == (240, 320, 3)
    assert_parity(out2.cpu().numpy()[None], oracle.resize_nearest(s_np, 240, 320), "scale")


def test_frames_round_robin_over_streams():
    """Frames issued round-robin on three streams, so that consecutive
    launches overlap on the GPU (the sustained configuration the benchmark
    times): every frame's output must still equal the oracle's.  Distinct
    seeded 4K-shaped frames (2:1 kernel) and 1080p grey frames (2x kernel),
    each into its own output buffer."""
    r = np.random.default_rng(3131)
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(2)]
    for (H, W, C, dH, dW) in ((2160, 3840, 3, 1080, 1920), (540, 960, 1, 1080, 1920)):
        frames = [random_image(r, (1, H, W, C), "u8") for _ in range(6)]
        srcs = [torch.from_numpy(f).cuda() for f in frames]
        outs = [torch.empty((1, dH, dW, C), dtype=torch.uint8, device="cuda") for _ in frames]
        torch.cuda.synchronize()
        say("case round-robin streams %s -> %s" % ((H, W, C), (dH, dW)))
        for i, (sv, ov) in enumerate(zip(srcs, outs)):
            R.resize_linear(sv, ov, stream=streams[i % 3])
        torch.cuda.synchronize()
        for i, f in enumerate(frames):
            assert_parity(outs[i].cpu().numpy(), oracle.resize_linear(f, dH, dW),
                          "round-robin frame %d %s" % (i, (H, W, C)))


def test_binding_rejects_bad_tensors():
    with pytest.raises(ValueError):
        R.resize(torch.zeros(4, 4, 3, dtype=torch.uint8), (2, 2))          # host tensor
    with pytest.raises(TypeError):
        R.resize(torch.zeros(4, 4, 3, dtype=torch.int32, device="cuda"), (2, 2))
    with pytest.raises(R.ResizeError):
        R.resize(torch.zeros(4, 4, 2, dtype=torch.uint8, device="cuda"), (2, 2))  # C=2
    with pytest.raises(ValueError):
        R.resize(torch.zeros(4, 4, 3, dtype=torch.uint8, device="cuda")[:, ::2], (2, 2))


def test_copy_bytes():
    for n in (16, 1000, 4096 * 16 + 5, 3 << 20):
        say("case copy %d" % n)
        a = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
        b = torch.zeros(n, dtype=torch.uint8, device="cuda")
        R.resize_copy_bytes(a, b)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


# --------------------------------------------------------------------------
# fused resize + normalisation (uint8 -> float32, NHWC / NCHW)
# --------------------------------------------------------------------------
IMAGENET = ((0.485, 0.456, 0.406, 0.5), (0.229, 0.224, 0.225, 0.25))


def run_normalize(s, dH, dW, layout, alpha=1 / 255):
    N, H, W, C = s.shape
    mean, std = IMAGENET[0][:C], IMAGENET[1][:C]
    src = torch.from_numpy(s).cuda()
    shape = (N, dH, dW, C) if layout == "NHWC" else (N, C, dH, dW)
    dst = torch.empty(shape, dtype=torch.float32, device="cuda")
    R.resize_linear_normalize(src, dst, mean, std, alpha=alpha, layout=layout)
    torch.cuda.synchronize()
    return dst.cpu().numpy(), oracle.resize_linear_normalize(s, dH, dW, alpha, mean, std, layout)


def assert_norm_parity(got, want, what):
    """The uint8 resize inside is exact; the float32 affine step (one FMA with
    scale and bias rounded to float) is within 3 * 2^-24 relative of the
    float64 value, so 1e-5 * max(1, |value|) bounds it with margin."""
    assert got.shape == want.shape, what
    assert np.isfinite(got).all(), what
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    tol = 1e-5 * np.maximum(1.0, np.abs(want.astype(np.float64)))
    bad = err > tol
    assert not bad.any(), "%s: %d elements off, worst %g" % (what, bad.sum(), (err / tol).max())


@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_normalize_thumb_batch(layout):
    w = WORKLOADS["thumb"]
    say("case normalize thumb %s" % layout)
    got, want = run_normalize(make_source(w), w.dH, w.dW, layout)
    assert_norm_parity(got, want, "normalize thumb " + layout)


@pytest.mark.parametrize("path", ["auto"] + PATHS)
@pytest.mark.parametrize("layout", ["NCHW", "NHWC"])
def test_normalize_random_shapes(layout, path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("MI_RESIZE_PATH", path)
    r = np.random.default_rng(333 + (layout == "NHWC"))
    for i in range(40):
        N, H, W, C, dH, dW = random_case(r)
        say("case normalize %s %s #%d %s" % (layout, path, i, (N, H, W, C, dH, dW)))
        s = random_image(r, (N, H, W, C), "u8")
        got, want = run_normalize(s, dH, dW, layout, alpha=float(r.choice([1 / 255, 1.0])))
        assert_norm_parity(got, want, "normalize #%d" % i)
    for (N, H, W, C, dH, dW) in EDGE[:12]:
        say("case normalize edge %s %s %s" % (layout, path, (N, H, W, C, dH, dW)))
        s = random_image(r, (N, H, W, C), "u8")
        got, want = run_normalize(s, dH, dW, layout)
        assert_norm_parity(got, want, "normalize edge %s" % ((N, H, W, C, dH, dW),))


# --------------------------------------------------------------------------
# HIP graph capture: the entry points allocate, synchronise and memset
# nothing, so a sequence of calls can be captured once and replayed (the
# small-image latency path).  Every replay, with eager work and
# synchronisation in between, must match the eager results.
# --------------------------------------------------------------------------
def test_graph_capture_replay():
    r = np.random.default_rng(404)
    cases = [((1, 48, 64, 1), (72, 96), "u8", "linear"), ((2, 30, 40, 3), (15, 20), "u8", "linear"),
             ((1, 33, 17, 4), (50, 9), "f32", "linear"), ((3, 16, 16, 3), (32, 32), "u8", "nearest"),
             ((1, 64, 96, 1), (32, 48), "u8", "linear")]
    srcs, dsts, eager = [], [], []
    for shape, (dH, dW), dt, mode in cases:
        s = random_image(r, shape, dt)
        srcs.append(torch.from_numpy(s).cuda())
        dsts.append(torch.empty((shape[0], dH, dW, shape[3]), dtype=srcs[-1].dtype, device="cuda"))
        eager.append(run_oracle(s, dH, dW, mode))
    say("case graph capture of %d resizes" % len(cases))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the binding up outside the capture
        for (shape, _, _, mode), a, b in zip(cases, srcs, dsts):
            (R.resize_linear if mode == "linear" else R.resize_nearest)(a, b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for (shape, _, _, mode), a, b in zip(cases, srcs, dsts):
            (R.resize_linear if mode == "linear" else R.resize_nearest)(a, b)
    for rep in range(4):
        for b in dsts:
            b.fill_(0)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (b, want) in enumerate(zip(dsts, eager)):
            assert_parity(b.cpu().numpy(), want, "graph replay %d case %d" % (rep, i))


# --------------------------------------------------------------------------
# batched crop-then-resize with per-image regions
# --------------------------------------------------------------------------
def random_crops(r, N, H, W, bad=False):
    """Random-resized-crop style regions (area 8-100 %, aspect 3/4-4/3); with
    bad=True some are partly or wholly outside the image (clamped)."""
    out = []
    for _ in range(N):
        area = H * W * r.uniform(0.08, 1.0)
        ar = np.exp(r.uniform(np.log(3 / 4), np.log(4 / 3)))
        w = int(min(W, max(1, round(np.sqrt(area * ar)))))
        h = int(min(H, max(1, round(np.sqrt(area / ar)))))
        x = int(r.integers(0, W - w + 1))
        y = int(r.integers(0, H - h + 1))
        if bad and r.random() < 0.5:
            x, y = x + int(r.integers(-W, W)), y + int(r.integers(-H, H))
            w, h = w + int(r.integers(-W, W)), h + int(r.integers(-H, H))
        out.append((x, y, w, h))
    return np.array(out, dtype=np.int32)


def run_roi(s, rois, dH, dW):
    src = torch.from_numpy(s).cuda()
    N, H, W, C = s.shape
    dst = torch.empty((N, dH, dW, C), dtype=src.dtype, device="cuda")
    R.resize_linear_roi(src, dst, torch.from_numpy(rois).cuda())
    torch.cuda.synchronize()
    return dst.cpu().numpy()


def test_roi_thumb_batch():
    w = WORKLOADS["thumb"]
    r = np.random.default_rng(515)
    s = make_source(w)
    rois = random_crops(r, w.batch, w.H, w.W)
    say("case roi thumb batch")
    assert_parity(run_roi(s, rois, w.dH, w.dW), oracle.resize_linear_roi(s, rois, w.dH, w.dW), "roi thumb")


@pytest.mark.parametrize("path", ["auto"] + PATHS)
@pytest.mark.parametrize("dtype", ["u8", "f32"])
def test_roi_random(dtype, path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("MI_RESIZE_PATH", path)
    r = np.random.default_rng(616 + (dtype == "f32"))
    for i in range(25):
        N = int(r.integers(1, 9))
        C = int(r.choice([1, 3, 4]))
        H, W = (int(v) for v in r.integers(1, 200, size=2))
        dH, dW = (int(v) for v in r.integers(1, 300, size=2))
        s = random_image(r, (N, H, W, C), dtype)
        rois = random_crops(r, N, H, W, bad=(i % 3 == 0))
        say("case roi %s %s #%d %s" % (dtype, path, i, (N, H, W, C, dH, dW)))
        assert_parity(run_roi(s, rois, dH, dW), oracle.resize_linear_roi(s, rois, dH, dW),
                      "roi #%d" % i)


# --------------------------------------------------------------------------
# border rules (mirror, wrap)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("path", ["auto"] + PATHS)
@pytest.mark.parametrize("border", ["mirror", "wrap"])
@pytest.mark.parametrize("dtype", ["u8", "f32"])
def test_border_modes(border, dtype, path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("MI_RESIZE_PATH", path)
    r = np.random.default_rng(717 + (dtype == "f32") + 2 * (border == "wrap"))
    shapes = [random_case(r) for _ in range(40)] + EDGE[:14] + [(1, 3, 3, 1, 6144, 6144 // 2048 * 3)]
    for i, (N, H, W, C, dH, dW) in enumerate(shapes):
        say("case border %s %s %s #%d %s" % (border, dtype, path, i, (N, H, W, C, dH, dW)))
        s = random_image(r, (N, H, W, C), dtype)
        src = torch.from_numpy(s).cuda()
        dst = torch.empty((N, dH, dW, C), dtype=src.dtype, device="cuda")
        R.resize_linear_border(src, dst, border=border)
        torch.cuda.synchronize()
        assert_parity(dst.cpu().numpy(), oracle.resize_linear(s, dH, dW, border=border),
                      "border %s #%d %s" % (border, i, (N, H, W, C, dH, dW)))


@pytest.mark.parametrize("border", ["mirror", "wrap"])
def test_border_thumb_full_size(border):
    """The thumbnail batch (256 x 480x640x3 -> 224x224) under each border rule,
    in the launch configuration the benchmark times; every image compared."""
    w = WORKLOADS["thumb"]
    say("case border full size %s %s -> %s" % (border, w.src_shape, w.dst_shape))
    s = make_source(w)
    src = torch.from_numpy(s).cuda()
    dst = torch.empty(w.dst_shape, dtype=src.dtype, device="cuda")
    R.resize_linear_border(src, dst, border=border)
    torch.cuda.synchronize()
    assert_parity(dst.cpu().numpy(), oracle.resize_linear(s, w.dH, w.dW, border=border),
                  "border %s thumb" % border)


# --------------------------------------------------------------------------
# nearest coordinate mappings (half_pixel, floor, round)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("path", ["auto"] + PATHS)
@pytest.mark.parametrize("mapping", ["half_pixel", "floor", "round"])
@pytest.mark.parametrize("dtype", ["u8", "f32"])
def test_nearest_mappings(mapping, dtype, path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("MI_RESIZE_PATH", path)
    r = np.random.default_rng(818 + 3 * (dtype == "f32") + ["half_pixel", "floor", "round"].index(mapping))
    shapes = [random_case(r) for _ in range(30)] + EDGE[:14] + [(1, 540, 960, 1, 1080, 1920),
                                                                (2, 64, 96, 3, 128, 192)]
    for i, (N, H, W, C, dH, dW) in enumerate(shapes):
        say("case nearest %s %s %s #%d %s" % (mapping, dtype, path, i, (N, H, W, C, dH, dW)))
        s = random_image(r, (N, H, W, C), dtype)
        src = torch.from_numpy(s).cuda()
        dst = torch.empty((N, dH, dW, C), dtype=src.dtype, device="cuda")
        R.resize_nearest_mapping(src, dst, mapping=mapping)
        torch.cuda.synchronize()
        assert_parity(dst.cpu().numpy(), oracle.resize_nearest(s, dH, dW, mapping=mapping),
                      "nearest %s #%d %s" % (mapping, i, (N, H, W, C, dH, dW)))


# --------------------------------------------------------------------------
# fused RGB(A) -> grey + linear resize
# --------------------------------------------------------------------------
@pytest.mark.parametrize("path", ["auto"] + PATHS)
@pytest.mark.parametrize("dtype", ["u8", "f32"])
def test_grey_random_shapes(dtype, path, monkeypatch):
    if path != "auto":
        monkeypatch.setenv("MI_RESIZE_PATH", path)
    r = np.random.default_rng(919 + (dtype == "f32"))
    shapes = []
    for _ in range(30):
        N, H, W, C, dH, dW = random_case(r)
        shapes.append((N, H, W, 3 + (C == 4), dH, dW))
    shapes += [(1, 1, 1, 3, 1, 1), (1, 1, 7, 4, 5, 1), (2, 33, 65, 3, 17, 129), (1, 600, 600, 4, 2, 3),
               (2, 64, 128, 3, 32, 64), (1, 48, 96, 4, 24, 48), (3, 20, 1040, 3, 10, 520),   # exact 2:1
               # row enlargements in batches: source rows repeat within an
               # image, never across an image boundary
               (3, 17, 230, 3, 40, 310), (2, 30, 500, 4, 45, 700), (4, 9, 300, 3, 25, 280),
               (2, 40, 600, 3, 50, 400)]
    for i, (N, H, W, C, dH, dW) in enumerate(shapes):
        say("case grey %s %s #%d %s" % (dtype, path, i, (N, H, W, C, dH, dW)))
        s = random_image(r, (N, H, W, C), dtype)
        src = torch.from_numpy(s).cuda()
        dst = torch.empty((N, dH, dW, 1), dtype=src.dtype, device="cuda")
        R.resize_linear_grey(src, dst)
        torch.cuda.synchronize()
        assert_parity(dst.cpu().numpy(), oracle.resize_linear_grey(s, dH, dW),
                      "grey %s #%d %s" % (dtype, i, (N, H, W, C, dH, dW)))


def test_grey_thumb_full_size():
    """The thumbnail batch (256 x 480x640x3 -> 224x224) to grey, in the launch
    configuration the benchmark times; every image compared."""
    w = WORKLOADS["thumb"]
    say("case grey full size %s -> %dx%d" % (w.src_shape, w.dH, w.dW))
    s = make_source(w)
    src = torch.from_numpy(s).cuda()
    dst = torch.empty((w.batch, w.dH, w.dW, 1), dtype=src.dtype, device="cuda")
    R.resize_linear_grey(src, dst)
    torch.cuda.synchronize()
    assert_parity(dst.cpu().numpy(), oracle.resize_linear_grey(s, w.dH, w.dW), "grey thumb")


def test_grey_4k_full_size():
    """The 4K RGB frame to grey 1080p (exact 2:1: the rounded mean of the four
    source greys), in the launch configuration a benchmark of it times."""
    w = WORKLOADS["4k"]
    say("case grey full size %s -> %dx%d" % (w.src_shape, w.dH, w.dW))
    s = make_source(w)
    src = torch.from_numpy(s).cuda()
    dst = torch.empty((w.batch, w.dH, w.dW, 1), dtype=src.dtype, device="cuda")
    R.resize_linear_grey(src, dst)
    torch.cuda.synchronize()
    assert_parity(dst.cpu().numpy(), oracle.resize_linear_grey(s, w.dH, w.dW), "grey 4k")


# --------------------------------------------------------------------------
# batches beyond the 65535 grid extent: the exact 2x, exact 2:1, nearest and
# direct kernels stride over images or rows past one grid's reach
# --------------------------------------------------------------------------
def _sampled_parity(s, dH, dW, mode, what, picks):
    """Full-batch GPU run, compared with the oracle image by image on the
    picked images (batches too large for the oracle as a whole)."""
    got = run_gpu(s, dH, dW, mode)
    for i in picks:
        assert_parity(got[i:i + 1], run_oracle(s[i:i + 1], dH, dW, mode), "%s image %d" % (what, i))


@pytest.mark.parametrize("case", ["wide", "tall"])
def test_half_grid_row_loops(case):
    """The exact 2:1 kernel past its grids' row reach.  wide: three
    segments per row (520 RGB pixels: 256 + 256 + 8) take the row-major
    grid with XCD-contiguous numbering, capped at 65535 rows, over 68000
    output rows.  tall: one segment per row takes the segment-major grid,
    rows along x capped at 2^24, over 2^24 + 1000 one-row images.
    Sampled images cover the first and last rows, rows on both sides of
    each cap and a spread between."""
    r = np.random.default_rng(1313 + (case == "tall"))
    if case == "wide":
        N, H, W, C = 17000, 8, 1040, 3
        picks = [0, 1, 16383, 16384, 16999] + [int(v) for v in r.integers(0, N, 20)]
    else:
        N, H, W, C = (1 << 24) + 1000, 2, 32, 1   # 16 output pixels: one segment
        picks = [0, (1 << 24) - 1, 1 << 24, N - 1] + [int(v) for v in r.integers(0, N, 20)]
    s = random_image(r, (N, H, W, C), "u8")
    say("case half grid row loop %s %s" % (case, (N, H, W, C)))
    _sampled_parity(s, H // 2, W // 2, "linear", "half row loop %s" % case, sorted(set(picks)))


@pytest.mark.parametrize("case", ["up2", "half", "generic", "rowseg"])
def test_batches_beyond_grid_extent(case, monkeypatch):
    r = np.random.default_rng(1212)
    N = 70000
    if case == "up2":          # grid z = images (linear) or y = rows / 2 (nearest), capped at 65535
        shape, dst = (2 * N, 1, 16, 1), (2, 32)
    elif case == "half":       # grid y = output rows, capped at 65535
        shape, dst = (N, 2, 32, 1), (1, 16)
    elif case == "generic":    # direct kernels, many rows per band
        monkeypatch.setenv("MI_RESIZE_PATH", "direct")
        shape, dst = (N, 3, 5, 3), (2, 7)
    else:                      # row-segment kernel, 2-row bands
        monkeypatch.setenv("MI_RESIZE_PATH", "rowseg")
        shape, dst = (N, 3, 5, 3), (2, 7)
    s = random_image(r, shape, "u8")
    for mode in ("linear", "nearest"):
        say("case big batch %s %s %s -> %s" % (case, mode, shape, dst))
        assert_parity(run_gpu(s, dst[0], dst[1], mode), run_oracle(s, dst[0], dst[1], mode),
                      "big batch %s %s" % (case, mode))
