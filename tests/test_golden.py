"""Stored hand cases: the oracle reproduces them and each satisfies a closed
form computed here (the cases come from tests/golden/make_golden.py)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")
CASES = json.load(open(GOLDEN))["cases"]


def arr(c):
    a = np.array(c["src"], dtype=np.uint8)
    return a[None, :, :, None] if a.ndim == 2 else a[None]


def oracle_run(c):
    dH, dW = c["dst_hw"]
    m = c["mode"]
    if m == "linear":
        return oracle.resize_linear(arr(c), dH, dW)
    if m == "grey":
        return oracle.resize_linear_grey(arr(c), dH, dW)
    if m.startswith("nearest_"):
        return oracle.resize_nearest(arr(c), dH, dW, mapping=m[len("nearest_"):])
    return oracle.resize_nearest(arr(c), dH, dW)


@pytest.mark.parametrize("c", CASES, ids=[c["name"] for c in CASES])
def test_oracle_reproduces(c):
    assert oracle_run(c)[0, :, :, 0].tolist() == c["expected"]


def by_name(n):
    return next(c for c in CASES if c["name"] == n)


def test_closed_forms():
    s = np.array(by_name("ramp4_to_2x2")["src"], dtype=np.int64)
    means = (s.reshape(2, 2, 2, 2).sum(axis=(1, 3)) + 2) // 4
    assert by_name("ramp4_to_2x2")["expected"] == means.tolist()
    # ramp value 16 (4y + x) at the clamped half-pixel coordinate, rounded half up
    for name, n_out in (("ramp4_to_8x8", 8),):
        exp = by_name(name)["expected"]
        for dy in range(n_out):
            y = min(max((Fraction(dy) + Fraction(1, 2)) * Fraction(4, n_out) - Fraction(1, 2), 0), 3)
            for dx in range(n_out):
                x = min(max((Fraction(dx) + Fraction(1, 2)) * Fraction(4, n_out) - Fraction(1, 2), 0), 3)
                assert exp[dy][dx] == int(np.floor(16 * (4 * y + x) + Fraction(1, 2)))
    assert by_name("ramp4_nearest_2x2")["expected"] == s[1::2, 1::2].tolist()
    assert by_name("ramp4_nearest_8x8")["expected"] == s.repeat(2, 0).repeat(2, 1).tolist()
    assert by_name("tie_2x2_to_1")["expected"] == [[1]]
    # corner-aligned nearest: source index floor(4d/3) or floor(4d/3 + 1/2)
    fl = [int(Fraction(4 * d, 3)) for d in range(3)]
    ro = [min(int(Fraction(4 * d, 3) + Fraction(1, 2)), 3) for d in range(3)]
    assert by_name("ramp4_nearest_floor_3x3")["expected"] == s[np.ix_(fl, fl)].tolist()
    assert by_name("ramp4_nearest_round_3x3")["expected"] == s[np.ix_(ro, ro)].tolist()
    # grey: the BT.601 weighted sum as an exact fraction, rounded half up
    def grey(px):
        r, g, b = (Fraction(v) for v in px[:3])
        return int(Fraction(299, 1000) * r + Fraction(587, 1000) * g + Fraction(114, 1000) * b
                   + Fraction(1, 2))
    prim = by_name("grey_primaries")
    assert prim["expected"] == [[grey(px) for px in prim["src"][0]]]
    gt = by_name("grey_2x2_to_1")
    greys = [grey(px) for row in gt["src"] for px in row]
    assert gt["expected"] == [[(sum(greys) + 2) // 4]]
