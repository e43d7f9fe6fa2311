"""Pins for the CPU oracle: facts the pages and the mathematics fix.

None of these re-types the oracle's arithmetic.  Each checks the oracle
against something independent of it: a closed form, an invariant, exact
rational arithmetic in a different (separable) form, or torch's float64
``interpolate``, which is the textbook half-pixel bilinear / nearest-exact
resize and serves as a library special case.

Sources: "From Prototype to Performance: Optimizing OpenCV Resize on Volcanic
GPUs" ("Naive resize with linear sampling": centre + 0.5 scaled into the
input, linear filter), and hnwysp.cn news/129086 (s2.1 nearest, s2.2
bilinear formula, s6.1 clamping, s6.2 fixed point).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from bilinear_image_resize_amd.workloads import WORKLOADS, make_source


def rng(seed):
    return np.random.default_rng(seed)


def rand_img(r, shape, dtype):
    if dtype == np.uint8:
        return r.integers(0, 256, size=shape, dtype=np.uint8)
    return r.random(size=shape, dtype=np.float32)


# --------------------------------------------------------------------------
# identity: scale 1 maps every pixel centre onto itself
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [np.uint8, np.float32])
def test_identity(dtype):
    r = rng(1)
    for _ in range(40):
        N, H, W = r.integers(1, 3), r.integers(1, 40), r.integers(1, 40)
        C = int(r.choice([1, 3, 4]))
        s = rand_img(r, (N, H, W, C), dtype)
        assert np.array_equal(oracle.resize_linear(s, H, W), s)
        assert np.array_equal(oracle.resize_nearest(s, H, W), s)


# --------------------------------------------------------------------------
# constant images stay constant (weights sum to one, any scale, any border)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [np.uint8, np.float32])
def test_constant(dtype):
    r = rng(2)
    for _ in range(60):
        H, W = r.integers(1, 30, size=2)
        dH, dW = r.integers(1, 70, size=2)
        C = int(r.choice([1, 3, 4]))
        vals = rand_img(r, (C,), dtype)
        s = np.broadcast_to(vals, (1, H, W, C)).copy()
        out = oracle.resize_linear(s, dH, dW)
        assert np.array_equal(out, np.broadcast_to(vals, out.shape))


# --------------------------------------------------------------------------
# an exact 2:1 downscale is the 2x2 block average (half-pixel centres put the
# sample exactly between four pixels).  A corner-aligned map would return the
# top-left pixel of each block instead, and truncation instead of
# round-half-up would turn {0,0,0,2} into 0 instead of 1.
# --------------------------------------------------------------------------
def test_half_down_u8_block_average():
    r = rng(3)
    for _ in range(30):
        N, h, w = r.integers(1, 3), r.integers(1, 20), r.integers(1, 20)
        C = int(r.choice([1, 3, 4]))
        s = rand_img(r, (N, 2 * h, 2 * w, C), np.uint8)
        blocks = s.reshape(N, h, 2, w, 2, C).astype(np.int64).sum(axis=(2, 4))
        expect = ((blocks + 2) // 4).astype(np.uint8)
        assert np.array_equal(oracle.resize_linear(s, h, w), expect)
    tie = np.array([[0, 0], [0, 2]], dtype=np.uint8)
    assert oracle.resize_linear(tie, 1, 1).item() == 1
    tie = np.array([[0, 0], [0, 1]], dtype=np.uint8)   # 0.25 rounds down
    assert oracle.resize_linear(tie, 1, 1).item() == 0


def test_half_down_f32_block_mean():
    r = rng(4)
    for _ in range(30):
        N, h, w = r.integers(1, 3), r.integers(1, 20), r.integers(1, 20)
        C = int(r.choice([1, 3, 4]))
        s = rand_img(r, (N, 2 * h, 2 * w, C), np.float32)
        mean = s.reshape(N, h, 2, w, 2, C).astype(np.float64).mean(axis=(2, 4))
        out = oracle.resize_linear(s, h, w)
        assert np.max(np.abs(out - mean)) <= 6e-8


def test_full_4k_frame_is_block_average():
    """The 4K RGB frame -> 1080p at its real size: every output is a 2x2 mean."""
    w = WORKLOADS["4k"]
    s = make_source(w)
    blocks = s.reshape(1, w.dH, 2, w.dW, 2, 3).astype(np.int32).sum(axis=(2, 4))
    expect = ((blocks + 2) // 4).astype(np.uint8)
    assert np.array_equal(oracle.resize_linear(s, w.dH, w.dW), expect)


# --------------------------------------------------------------------------
# linear ramps are reproduced: bilinear interpolation of p = a + bx*x + by*y
# sampled at the clamped source coordinate gives the ramp there.
# --------------------------------------------------------------------------
def src_coord(d, n_in, n_out):
    """Half-pixel source coordinate, clamped to [0, n_in - 1], as a Fraction."""
    x = (Fraction(d) + Fraction(1, 2)) * Fraction(n_in, n_out) - Fraction(1, 2)
    return min(max(x, Fraction(0)), Fraction(n_in - 1))


def test_ramp_f32_any_scale():
    r = rng(5)
    for _ in range(40):
        H, W = r.integers(1, 24, size=2)
        dH, dW = r.integers(1, 50, size=2)
        a, bx, by = (int(v) / 64.0 for v in r.integers(-64, 64, size=3))
        ys, xs = np.mgrid[0:H, 0:W]
        s = (a + bx * xs + by * ys).astype(np.float32)[None, :, :, None]
        out = oracle.resize_linear(s, dH, dW)[0, :, :, 0]
        for dy in range(dH):
            sy = float(src_coord(dy, H, dH))
            for dx in range(dW):
                sx = float(src_coord(dx, W, dW))
                assert abs(out[dy, dx] - (a + bx * sx + by * sy)) <= 2e-6


@pytest.mark.parametrize("shape", [((6, 5), (12, 10)), ((5, 7), (20, 28)),
                                   ((16, 12), (8, 6)), ((12, 16), (3, 4)),
                                   ((3, 9), (24, 18))])
def test_ramp_u8_dyadic_scales(shape):
    """At scales whose weights are exact 11-bit fractions the u8 result is the
    ramp at the source coordinate, rounded half up."""
    (H, W), (dH, dW) = shape
    checked = 0
    for a, bx, by in ((3, 7, 11), (200, -9, -4), (0, 20, 1), (0, 3, 5), (255, -4, -7)):
        ys, xs = np.mgrid[0:H, 0:W]
        vals = a + bx * xs + by * ys
        if vals.min() < 0 or vals.max() > 255:
            continue
        checked += 1
        s = vals.astype(np.uint8)[None, :, :, None]
        out = oracle.resize_linear(s, dH, dW)[0, :, :, 0]
        for dy in range(dH):
            sy = src_coord(dy, H, dH)
            for dx in range(dW):
                sx = src_coord(dx, W, dW)
                v = a + bx * sx + by * sy
                assert out[dy, dx] == int(np.floor(v + Fraction(1, 2)))
    assert checked >= 2


# --------------------------------------------------------------------------
# uint8 weights at any scale.  The 11-bit weight of an axis is 2048 u rounded
# half up (hnwysp.cn news/129086 s6.2, fixed point; the reading taken: one
# rounding per axis, halves up), where u is the exact fractional part of the
# half-pixel coordinate.  The four weights then sum to 2048^2 and blend a
# linear ramp to the ramp's value at the *quantised* coordinate
# i + U/2048, j + V/2048 (s2.2's four-term sum of a linear function), which
# the final rounding takes half up.  Here U and V come from Fractions, never
# from the oracle's integer code, so a wrong weight anywhere fails.
# --------------------------------------------------------------------------
def weight11_fraction(u):
    """round-half-up(2048 u) for a Fraction u in [0, 1)."""
    return math.floor(2048 * u + Fraction(1, 2))


def quantised_coord(d, n_in, n_out):
    """Clamped half-pixel coordinate with its fraction quantised to 11 bits."""
    x = src_coord(d, n_in, n_out)
    i = math.floor(x)
    return i + Fraction(weight11_fraction(x - i), 2048)


def ramp_expectation(a, bx, by, H, W, dH, dW):
    ys = [quantised_coord(dy, H, dH) for dy in range(dH)]
    xs = [quantised_coord(dx, W, dW) for dx in range(dW)]
    return np.array([[math.floor(a + bx * x + by * y + Fraction(1, 2)) for x in xs]
                     for y in ys], dtype=np.int64)


def ramp_image(a, bx, by, H, W):
    ys, xs = np.mgrid[0:H, 0:W]
    vals = a + bx * xs + by * ys
    assert vals.min() >= 0 and vals.max() <= 255
    return vals.astype(np.uint8)[None, :, :, None]


# Non-dyadic scales: the small image's scale 2/3 (64 -> 96), the thumbnail
# batch's 15/7 and 20/7 (480 -> 224, 640 -> 224), and a few others.
@pytest.mark.parametrize("shape,ramp", [
    (((8, 12), (12, 18)), (5, 13, 11)),        # 1.5x both axes
    (((6, 10), (9, 15)), (200, -9, -17)),
    (((15, 20), (7, 7)), (3, 7, 8)),           # 480/224 and 640/224 ratios
    (((30, 40), (14, 14)), (250, -3, -4)),
    (((7, 5), (11, 13)), (1, 31, 19)),         # 7/11, 5/13
    (((9, 4), (5, 7)), (17, 29, 13)),          # 9/5 down, 4/7 up
])
def test_ramp_u8_quantised_any_scale(shape, ramp):
    (H, W), (dH, dW) = shape
    a, bx, by = ramp
    out = oracle.resize_linear(ramp_image(a, bx, by, H, W), dH, dW)[0, :, :, 0]
    assert np.array_equal(out.astype(np.int64), ramp_expectation(a, bx, by, H, W, dH, dW))


@pytest.mark.parametrize("axis", ["x", "y"])
def test_weight_ties_round_half_up(axis):
    """An odd source length resized to 2048 samples puts 2048 u on k + 1/2 at
    every interior sample (u = r / 4096 with r odd), the only way a weight tie
    arises; 6 -> 4096 does it too (2048 u = r / 4 with r = 2 mod 4).  The
    ramp pins which way those ties go: half up."""
    for n_in, n_out, a, b in ((3, 2048, 20, 101), (5, 2048, 2, 59), (6, 4096, 3, 48)):
        ties = sum((2048 * (src_coord(d, n_in, n_out) - math.floor(src_coord(d, n_in, n_out)))).denominator == 2
                   for d in range(n_out))
        assert ties > n_out // 2
        if axis == "x":
            H, W, dH, dW, bx, by = 2, n_in, 3, n_out, b, 7
        else:
            H, W, dH, dW, bx, by = n_in, 2, n_out, 3, 7, b
        out = oracle.resize_linear(ramp_image(a, bx, by, H, W), dH, dW)[0, :, :, 0]
        assert np.array_equal(out.astype(np.int64), ramp_expectation(a, bx, by, H, W, dH, dW))


def test_four_by_four_tables_by_hand():
    """S = 16 (4y + x).  The tables below were worked by hand from the
    definition (the pages print no worked example): 4 -> 3 puts the centres
    at 1/6, 3/2, 17/6, so the 11-bit weights are 341, 1024, 1707 (341.33 and
    1706.67 rounded), and an output is 16 (4 y_q + x_q) rounded half up at
    the quantised coordinates, e.g. 80 * 341 / 2048 = 13.32 -> 13 at (0, 0).
    4 -> 8 puts the centres at d/2 - 1/4, clamped at 0 and 3."""
    S = (16 * (4 * np.arange(4)[:, None] + np.arange(4)[None, :])).astype(np.uint8)
    assert [weight11_fraction(src_coord(d, 4, 3) % 1) for d in range(3)] == [341, 1024, 1707]
    out3 = oracle.resize_linear(S, 3, 3)[0, :, :, 0]
    assert out3.tolist() == [[13, 35, 56], [99, 120, 141], [184, 205, 227]]
    out8 = oracle.resize_linear(S, 8, 8)[0, :, :, 0]
    assert out8[0].tolist() == [0, 4, 12, 20, 28, 36, 44, 48]
    assert out8[7].tolist() == [192, 196, 204, 212, 220, 228, 236, 240]
    assert out8[:, 0].tolist() == [0, 16, 48, 80, 112, 144, 176, 192]
    assert np.array_equal(out3.astype(np.int64), ramp_expectation(0, 16, 64, 4, 4, 3, 3))
    assert np.array_equal(out8.astype(np.int64), ramp_expectation(0, 16, 64, 4, 4, 8, 8))


# --------------------------------------------------------------------------
# exact rational bilinear (separable form: lerp along x on both rows, then
# along y) - the u8 result is within the fixed-point bound of it:
# two 11-bit weight roundings (255/4096 each) plus the final rounding 1/2.
# --------------------------------------------------------------------------
def exact_bilinear(img, dH, dW):
    H, W = img.shape
    out = np.empty((dH, dW), dtype=object)
    for dy in range(dH):
        y = src_coord(dy, H, dH)
        j = int(np.floor(y)); v = y - j; j1 = min(j + 1, H - 1)
        for dx in range(dW):
            x = src_coord(dx, W, dW)
            i = int(np.floor(x)); u = x - i; i1 = min(i + 1, W - 1)
            top = int(img[j, i]) + u * (int(img[j, i1]) - int(img[j, i]))
            bot = int(img[j1, i]) + u * (int(img[j1, i1]) - int(img[j1, i]))
            out[dy, dx] = top + v * (bot - top)
    return out


def test_u8_within_fixed_point_bound_of_exact():
    r = rng(6)
    worst = Fraction(0)
    for _ in range(150):
        H, W = r.integers(1, 8, size=2)
        dH, dW = r.integers(1, 10, size=2)
        img = r.integers(0, 256, size=(H, W), dtype=np.uint8)
        ex = exact_bilinear(img, dH, dW)
        out = oracle.resize_linear(img, dH, dW)[0, :, :, 0]
        for dy in range(dH):
            for dx in range(dW):
                d = abs(Fraction(int(out[dy, dx])) - ex[dy, dx])
                worst = max(worst, d)
    assert worst <= Fraction(1, 2) + Fraction(2 * 255, 4096)


# --------------------------------------------------------------------------
# library special case: torch float64 interpolate (half-pixel centres,
# align_corners=False, no antialias) is the real-valued bilinear resize.
# --------------------------------------------------------------------------
def torch_bilinear(s, dH, dW):
    t = torch.from_numpy(s.astype(np.float64)).permute(0, 3, 1, 2)
    o = torch.nn.functional.interpolate(t, size=(dH, dW), mode="bilinear",
                                        align_corners=False, antialias=False)
    return o.permute(0, 2, 3, 1).numpy()


def test_f32_matches_torch_float64():
    r = rng(7)
    for _ in range(200):
        N = int(r.integers(1, 3)); C = int(r.choice([1, 3, 4]))
        H, W = r.integers(1, 40, size=2)
        dH, dW = r.integers(1, 60, size=2)
        s = rand_img(r, (N, H, W, C), np.float32)
        ref = torch_bilinear(s, dH, dW)
        out = oracle.resize_linear(s, dH, dW)
        # the oracle rounds a double result to float once: <= 1/2 ulp(1)
        assert np.max(np.abs(out.astype(np.float64) - ref)) <= 6e-8


def test_u8_matches_torch_at_dyadic_scales():
    """Weights 0, 1/4, 1/2, 3/4 are exact in 11 bits: u8 = round-half-up of the
    float64 value (which is exact for these weights)."""
    r = rng(8)
    for (H, W, dH, dW) in ((7, 9, 14, 18), (8, 12, 4, 6), (5, 6, 20, 24), (30, 17, 60, 34)):
        s = rand_img(r, (2, H, W, 3), np.uint8)
        ref = torch_bilinear(s, dH, dW)
        assert np.array_equal(oracle.resize_linear(s, dH, dW),
                              np.floor(ref + 0.5).astype(np.uint8))


def test_u8_within_bound_of_torch_random_scales():
    r = rng(9)
    for _ in range(100):
        H, W = r.integers(1, 40, size=2)
        dH, dW = r.integers(1, 60, size=2)
        s = rand_img(r, (1, H, W, 3), np.uint8)
        ref = torch_bilinear(s, dH, dW)
        out = oracle.resize_linear(s, dH, dW).astype(np.float64)
        assert np.max(np.abs(out - ref)) <= 0.5 + 2 * 255 / 4096 + 1e-9


def test_full_up2x_matches_torch():
    """1080p grey -> 2160x3840 at its real size: weights 1/4, 3/4 are exact."""
    w = WORKLOADS["up2x"]
    s = make_source(w)
    ref = torch_bilinear(s, w.dH, w.dW)
    assert np.array_equal(oracle.resize_linear(s, w.dH, w.dW),
                          np.floor(ref + 0.5).astype(np.uint8))


# --------------------------------------------------------------------------
# nearest: closed forms and torch's nearest-exact
# --------------------------------------------------------------------------
def test_nearest_integer_upscale_replicates():
    r = rng(10)
    for k in (2, 3, 4, 5):
        s = rand_img(r, (2, 7, 5, 3), np.uint8)
        out = oracle.resize_nearest(s, 7 * k, 5 * k)
        assert np.array_equal(out, s.repeat(k, axis=1).repeat(k, axis=2))


def test_nearest_integer_downscale_picks_centre():
    """W = k*dW: the centre of output pixel d lands at k*d + (k-1)/2; rounding
    half up picks k*d + k//2 (4 -> 2 picks columns 1 and 3)."""
    r = rng(11)
    for k in (2, 3, 4):
        s = rand_img(r, (1, 4 * k, 6 * k, 1), np.float32)
        out = oracle.resize_nearest(s, 4, 6)
        assert np.array_equal(out, s[:, k // 2::k, k // 2::k])


def test_full_up2x_nearest_replicates():
    w = WORKLOADS["up2x"]
    s = make_source(w)
    out = oracle.resize_nearest(s, w.dH, w.dW)
    assert np.array_equal(out, s.repeat(2, axis=1).repeat(2, axis=2))


def test_nearest_matches_torch_nearest_exact():
    """torch computes floor((d + 0.5) * in / out) in floating point; where the
    exact value is an integer its rounding may land one pixel low, so those
    rows and columns are left to the closed-form tests above."""
    r = rng(12)
    compared = 0
    for _ in range(200):
        H, W = (int(v) for v in r.integers(1, 40, size=2))
        dH, dW = (int(v) for v in r.integers(1, 60, size=2))
        s = rand_img(r, (1, H, W, 2), np.float32)
        t = torch.from_numpy(s.astype(np.float64)).permute(0, 3, 1, 2)
        ref = torch.nn.functional.interpolate(t, size=(dH, dW), mode="nearest-exact")
        ref = ref.permute(0, 2, 3, 1).numpy().astype(np.float32)
        out = oracle.resize_nearest(s, dH, dW)
        rows = [d for d in range(dH) if ((Fraction(d) + Fraction(1, 2)) * Fraction(H, dH)).denominator != 1]
        cols = [d for d in range(dW) if ((Fraction(d) + Fraction(1, 2)) * Fraction(W, dW)).denominator != 1]
        sub = np.ix_([0], rows, cols, [0, 1])
        assert np.array_equal(out[sub], ref[sub])
        compared += len(rows) * len(cols)
    assert compared > 100000


# --------------------------------------------------------------------------
# nearest, corner-aligned mappings: "floor" (legacy) and "round" (the CUDA
# kernel of hnwysp.cn news/129086 s3.2: x = d / scale, floor(x + 0.5))
# --------------------------------------------------------------------------
def test_nearest_mappings_by_hand():
    """S = 16 (4y + x), resized 4x4 -> 3x3: the source coordinate of output d
    is 4d/3 = 0, 1.33, 2.67 (corner-aligned) or (d + 1/2) 4/3 - 1/2 =
    0.17, 1.5, 2.83 (half-pixel); floor gives columns 0, 1, 2, round half up
    0, 1, 3, and the half-pixel map rounded half up 0, 2, 3.  4x4 -> 2x2:
    corner-aligned 0, 2 for both floor and round, half-pixel 1, 3."""
    S = (16 * (4 * np.arange(4)[:, None] + np.arange(4)[None, :])).astype(np.uint8)
    idx = {"floor": [0, 1, 2], "round": [0, 1, 3], "half_pixel": [0, 2, 3]}
    for m, cols in idx.items():
        out = oracle.resize_nearest(S, 3, 3, mapping=m)[0, :, :, 0]
        assert out.tolist() == [[16 * (4 * y + x) for x in cols] for y in cols], m
    half = {"floor": [0, 2], "round": [0, 2], "half_pixel": [1, 3]}
    for m, cols in half.items():
        out = oracle.resize_nearest(S, 2, 2, mapping=m)[0, :, :, 0]
        assert out.tolist() == [[16 * (4 * y + x) for x in cols] for y in cols], m


def test_nearest_mappings_identity_and_upscale():
    """At scale 1 every mapping is the identity.  For an integer upscale k,
    floor picks d // k (replication, like the half-pixel map), and round
    picks floor(d / k + 1/2), clamped to the last pixel."""
    r = rng(13)
    s = rand_img(r, (2, 9, 7, 3), np.uint8)
    for m in ("floor", "round"):
        assert np.array_equal(oracle.resize_nearest(s, 9, 7, mapping=m), s)
    for k in (2, 3, 5):
        out = oracle.resize_nearest(s, 9 * k, 7 * k, mapping="floor")
        assert np.array_equal(out, s.repeat(k, axis=1).repeat(k, axis=2))
        out = oracle.resize_nearest(s, 9 * k, 7 * k, mapping="round")
        ys = np.minimum((2 * np.arange(9 * k) + k) // (2 * k), 8)
        xs = np.minimum((2 * np.arange(7 * k) + k) // (2 * k), 6)
        assert np.array_equal(out, s[:, ys][:, :, xs])


def test_nearest_floor_matches_torch_nearest():
    """torch's legacy "nearest" takes floor(d * in / out) in floating point;
    where the exact value is an integer its rounding may land one pixel low,
    so those rows and columns are left out (the cases above cover them)."""
    r = rng(14)
    compared = 0
    for _ in range(200):
        H, W = (int(v) for v in r.integers(1, 40, size=2))
        dH, dW = (int(v) for v in r.integers(1, 60, size=2))
        s = rand_img(r, (1, H, W, 2), np.float32)
        t = torch.from_numpy(s.astype(np.float64)).permute(0, 3, 1, 2)
        ref = torch.nn.functional.interpolate(t, size=(dH, dW), mode="nearest")
        ref = ref.permute(0, 2, 3, 1).numpy().astype(np.float32)
        out = oracle.resize_nearest(s, dH, dW, mapping="floor")
        rows = [d for d in range(dH) if (Fraction(d) * Fraction(H, dH)).denominator != 1]
        cols = [d for d in range(dW) if (Fraction(d) * Fraction(W, dW)).denominator != 1]
        sub = np.ix_([0], rows, cols, [0, 1])
        assert np.array_equal(out[sub], ref[sub])
        compared += len(rows) * len(cols)
    assert compared > 50000


def test_nearest_round_brute_force():
    """round: the exact coordinate d * in / out as a Fraction, rounded half up
    and clamped, on small shapes."""
    r = rng(15)
    for _ in range(60):
        H, W = (int(v) for v in r.integers(1, 12, size=2))
        dH, dW = (int(v) for v in r.integers(1, 20, size=2))
        s = rand_img(r, (1, H, W, 1), np.uint8)
        out = oracle.resize_nearest(s, dH, dW, mapping="round")
        for y in range(dH):
            sy = min(int(Fraction(y * H, dH) + Fraction(1, 2)), H - 1)
            for x in range(dW):
                sx = min(int(Fraction(x * W, dW) + Fraction(1, 2)), W - 1)
                assert out[0, y, x, 0] == s[0, sy, sx, 0]


# --------------------------------------------------------------------------
# fused RGB -> grey (BT.601 luma weights), then resize
# --------------------------------------------------------------------------
def test_grey_closed_forms():
    """0.299 R + 0.587 G + 0.114 B, rounded half up: pure red 255 -> 76.245
    -> 76, green -> 149.685 -> 150, blue -> 29.07 -> 29, white -> 255, any
    grey v stays v, and the tie 114 * 250 / 1000 = 28.5 rounds up to 29."""
    px = [((255, 0, 0), 76), ((0, 255, 0), 150), ((0, 0, 255), 29), ((255, 255, 255), 255),
          ((0, 0, 250), 29), ((0, 0, 0), 0), ((1, 0, 0), 0), ((2, 0, 0), 1)]
    src = np.array([[[p for p, _ in px]]], dtype=np.uint8)
    assert oracle.rgb_to_grey(src)[0, 0, :, 0].tolist() == [v for _, v in px]
    vals = np.arange(256, dtype=np.uint8)
    greys = np.stack([vals, vals, vals], axis=-1)[None, None]
    assert np.array_equal(oracle.rgb_to_grey(greys)[0, 0, :, 0], vals)
    f = np.array([[[[1, 0, 0, 7], [0, 1, 0, 7], [0, 0, 1, 7], [0.5, 0.5, 0.5, 0]]]], np.float32)
    assert np.allclose(oracle.rgb_to_grey(f)[0, 0, :, 0], [0.299, 0.587, 0.114, 0.5], atol=1e-7, rtol=0)


def test_grey_ignores_alpha_and_resizes_as_grey_image():
    """A fourth channel does not matter; at scale 1 the result is the grey
    image itself; an exact 2:1 downscale is the rounded mean of the greys."""
    r = rng(16)
    s = rand_img(r, (2, 10, 12, 4), np.uint8)
    s2 = s.copy()
    s2[..., 3] = 255 - s2[..., 3]
    assert np.array_equal(oracle.resize_linear_grey(s, 5, 6), oracle.resize_linear_grey(s2, 5, 6))
    g = oracle.rgb_to_grey(s).astype(np.int64)
    assert np.array_equal(oracle.resize_linear_grey(s, 10, 12), g.astype(np.uint8))
    mean = (g[:, 0::2, 0::2] + g[:, 0::2, 1::2] + g[:, 1::2, 0::2] + g[:, 1::2, 1::2] + 2) >> 2
    assert np.array_equal(oracle.resize_linear_grey(s, 5, 6), mean.astype(np.uint8))


# --------------------------------------------------------------------------
# layout invariants: transpose, horizontal flip, channels, batch
# --------------------------------------------------------------------------
def test_transpose_equivariance():
    r = rng(13)
    for dtype in (np.uint8, np.float32):
        for _ in range(30):
            H, W = r.integers(1, 30, size=2)
            dH, dW = r.integers(1, 50, size=2)
            s = rand_img(r, (1, H, W, 3), dtype)
            a = oracle.resize_linear(s, dH, dW)
            b = oracle.resize_linear(s.transpose(0, 2, 1, 3), dW, dH).transpose(0, 2, 1, 3)
            if dtype == np.uint8:   # weight product is symmetric, exact integers
                assert np.array_equal(a, b)
            else:
                assert np.max(np.abs(a - b)) <= 1.2e-7
            na = oracle.resize_nearest(s, dH, dW)
            nb = oracle.resize_nearest(s.transpose(0, 2, 1, 3), dW, dH).transpose(0, 2, 1, 3)
            assert np.array_equal(na, nb)


def test_flip_equivariance():
    """Mirroring input and output together: the half-pixel map is symmetric.
    f32 exactly up to rounding; u8 at scales whose weights are not 11-bit
    half-way ties (a tie rounds up on one side and down on the other)."""
    r = rng(14)
    for _ in range(30):
        H, W = r.integers(1, 30, size=2)
        dH, dW = r.integers(1, 50, size=2)
        s = rand_img(r, (1, H, W, 1), np.float32)
        a = oracle.resize_linear(s, dH, dW)[:, :, ::-1]
        b = oracle.resize_linear(s[:, :, ::-1], dH, dW)
        assert np.max(np.abs(a - b)) <= 1.2e-7
    for (H, W, dH, dW) in ((48, 64, 72, 96), (20, 30, 10, 15), (9, 11, 36, 44)):
        s = rand_img(r, (1, H, W, 3), np.uint8)
        a = oracle.resize_linear(s, dH, dW)[:, ::-1, ::-1]
        b = oracle.resize_linear(s[:, ::-1, ::-1], dH, dW)
        assert np.array_equal(a, b)


def test_channel_and_batch_independence():
    r = rng(15)
    for dtype in (np.uint8, np.float32):
        s = rand_img(r, (3, 13, 17, 4), dtype)
        full = oracle.resize_linear(s, 29, 11)
        for n in range(3):
            for c in range(4):
                one = oracle.resize_linear(s[n:n + 1, :, :, c:c + 1], 29, 11)
                assert np.array_equal(one, full[n:n + 1, :, :, c:c + 1])


def test_row_ranges_compose():
    r = rng(16)
    s = rand_img(r, (2, 11, 13, 3), np.uint8)
    full = oracle.resize_linear(s, 7, 19).reshape(14, 19, 3)
    parts = [oracle.resize_linear(s, 7, 19, rows=(a, b)) for a, b in ((0, 5), (5, 6), (6, 14))]
    assert np.array_equal(np.concatenate(parts), full)


def test_output_within_source_range():
    r = rng(17)
    for _ in range(30):
        s = rand_img(r, (1, 9, 9, 1), np.uint8) // 2 + 40
        out = oracle.resize_linear(s, int(r.integers(1, 30)), int(r.integers(1, 30)))
        assert out.min() >= s.min() and out.max() <= s.max()


# --------------------------------------------------------------------------
# fused resize + normalisation: the resize part is the pinned uint8 oracle;
# these pin the affine map and the layouts
# --------------------------------------------------------------------------
def test_normalize_identity_scale_is_plain_normalisation():
    r = rng(18)
    s = rand_img(r, (2, 9, 11, 3), np.uint8)
    mean, std = (0.485, 0.456, 0.406), (0.229, 0.224, 0.225)
    out = oracle.resize_linear_normalize(s, 9, 11, 1 / 255, mean, std, "NHWC")
    ref = (s.astype(np.float64) / 255 - np.array(mean)) / np.array(std)
    assert np.max(np.abs(out - ref)) <= 3e-7


def test_normalize_layouts_and_constant():
    r = rng(19)
    s = rand_img(r, (3, 13, 7, 4), np.uint8)
    a = oracle.resize_linear_normalize(s, 5, 17, 1.0, (1, 2, 3, 4), (2, 4, 8, 16), "NHWC")
    b = oracle.resize_linear_normalize(s, 5, 17, 1.0, (1, 2, 3, 4), (2, 4, 8, 16), "NCHW")
    assert b.shape == (3, 4, 5, 17) and np.array_equal(a.transpose(0, 3, 1, 2), b)
    # powers-of-two std and integer mean: exact in float32
    v = oracle.resize_linear(s, 5, 17).astype(np.float64)
    assert np.array_equal(a, ((v - np.array([1, 2, 3, 4])) / np.array([2, 4, 8, 16])).astype(np.float32))
    c = np.full((1, 6, 6, 1), 200, dtype=np.uint8)
    out = oracle.resize_linear_normalize(c, 10, 3, 1 / 255, (0.5,), (0.25,), "NCHW")
    assert np.allclose(out, (200 / 255 - 0.5) / 0.25, atol=1e-6, rtol=0)


# --------------------------------------------------------------------------
# crop then resize: a crop of a ramp is a ramp (offset by the crop corner),
# so the result is the ramp at crop corner + the crop's half-pixel coordinate
# --------------------------------------------------------------------------
def test_roi_of_ramp_is_shifted_ramp():
    H, W = 40, 50
    ys, xs = np.mgrid[0:H, 0:W]
    img = (xs / 64.0 + ys / 128.0).astype(np.float32)[None, :, :, None]
    rois = [(3, 5, 20, 17), (0, 0, 50, 40), (49, 39, 7, 9), (-4, 10, 30, 100)]
    src = np.repeat(img, len(rois), axis=0)
    out = oracle.resize_linear_roi(src, rois, 11, 13)
    for n, roi in enumerate(rois):
        x0, y0, w, h = oracle.clamp_roi(roi, H, W)
        for dy in range(11):
            sy = float(src_coord(dy, h, 11)) + y0
            for dx in range(13):
                sx = float(src_coord(dx, w, 13)) + x0
                assert abs(out[n, dy, dx, 0] - (sx / 64.0 + sy / 128.0)) <= 1e-6


def test_roi_full_image_is_plain_resize():
    r = rng(20)
    s = rand_img(r, (3, 17, 23, 3), np.uint8)
    full = [(0, 0, 23, 17)] * 3
    assert np.array_equal(oracle.resize_linear_roi(s, full, 9, 31), oracle.resize_linear(s, 9, 31))


# --------------------------------------------------------------------------
# border rules: wrap = the centre tile of the clamp resize of the image tiled
# 3 x 3 (same scale, coordinates shifted by one image); mirror = the centre of
# the clamp resize of the image padded by reflection about its edge pixels
# (numpy's "reflect" padding).  In both, the centre never reaches the padded
# image's own border, so the (pinned) clamp resize decides it.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [np.uint8, np.float32])
def test_border_wrap_and_mirror_by_extension(dtype):
    r = rng(21)
    for _ in range(25):
        H, W = (int(v) for v in r.integers(2, 14, size=2))
        dH, dW = (int(v) for v in r.integers(1, 40, size=2))
        s = rand_img(r, (1, H, W, 2), dtype)
        # uint8: bit-exact (same integer weights); float32: the two evaluate
        # the same weighted sum in a different order before one rounding
        tol = 0 if dtype == np.uint8 else 1.2e-7
        tiled = np.tile(s, (1, 3, 3, 1))
        big = oracle.resize_linear(tiled, 3 * dH, 3 * dW)
        got = oracle.resize_linear(s, dH, dW, border="wrap")
        assert np.max(np.abs(got.astype(np.float64) - big[:, dH:2 * dH, dW:2 * dW])) <= tol
        padded = np.pad(s, ((0, 0), (H, H), (W, W), (0, 0)), mode="reflect")
        big = oracle.resize_linear(np.ascontiguousarray(padded), 3 * dH, 3 * dW)
        got = oracle.resize_linear(s, dH, dW, border="mirror")
        assert np.max(np.abs(got.astype(np.float64) - big[:, dH:2 * dH, dW:2 * dW])) <= tol


def test_border_rules_agree_inside():
    """Downscales by 2 never leave the image: all three rules agree; an
    enlargement differs only in the outermost output pixels."""
    r = rng(22)
    s = rand_img(r, (1, 16, 20, 3), np.uint8)
    for b in ("mirror", "wrap"):
        assert np.array_equal(oracle.resize_linear(s, 8, 10, border=b), oracle.resize_linear(s, 8, 10))
        up = oracle.resize_linear(s, 64, 80, border=b)
        ref = oracle.resize_linear(s, 64, 80)
        assert np.array_equal(up[:, 2:-2, 2:-2], ref[:, 2:-2, 2:-2])
        assert not np.array_equal(up, ref)
