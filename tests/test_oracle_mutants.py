"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a private copy of the oracle's C source (on
the CPU, in a temporary directory), builds it, points the oracle module at it
and checks that at least one pin in ``test_oracle_pins`` now fails.  The real
oracle is restored afterwards.
"""
import inspect
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

_SRC = open(os.path.join(os.path.dirname(oracle.__file__), "resize_oracle.c")).read()

_MAP = ("int64_t num = (2 * d + 1) * in_len - out_len;\n    int64_t den = 2 * out_len;\n    *u_den")
MUTANTS = {
    # corner-aligned map (no half-pixel offset), as in the CUDA listing
    "corner_aligned": (_MAP, _MAP.replace("(2 * d + 1) * in_len - out_len", "(2 * d) * in_len")),
    "offset_sign": (_MAP, _MAP.replace("- out_len", "+ out_len")),
    "swap_taps": ("+ U * (2048 - V) * s_i1j\n                            + (2048 - U) * V * s_ij1",
                  "+ U * (2048 - V) * s_ij1\n                            + (2048 - U) * V * s_i1j"),
    "truncate_result": ("(sum + ((int64_t)1 << 21)) >> 22", "sum >> 22"),
    "truncate_weight": ("floor_div(4096 * u_num + u_den, 2 * u_den)", "floor_div(4096 * u_num, 2 * u_den)"),
    # weight ties (2048 u = k + 1/2) rounded half to even, or half down
    "weight_round_half_even": ("return floor_div(4096 * u_num + u_den, 2 * u_den);",
                               "int64_t q = floor_div(4096 * u_num + u_den, 2 * u_den);\n"
                               "    if ((4096 * u_num + u_den) % (2 * u_den) == 0 && (q & 1))\n"
                               "        q -= 1;\n    return q;"),
    "weight_round_half_down": ("return floor_div(4096 * u_num + u_den, 2 * u_den);",
                               "return floor_div(4096 * u_num + u_den - 1, 2 * u_den);"),
    "half_weight_v": ("int64_t V = quantise_11(v_num, v_den);", "int64_t V = quantise_11(v_num, v_den) / 2;"),
    "nearest_floor": ("floor_div(num + den / 2, den)", "floor_div(num, den)"),
    "f32_transposed": ("+ (1.0 - u) * v * s_ij1", "+ (1.0 - v) * u * s_ij1"),
    "f32_dropped_term": ("+ u * v * s_i1j1;", ";"),
    "f32_same_row": ("double v = (double)v_num / (double)v_den;",
                     "double v = (double)v_num / (double)v_den; j1 = j;"),
    "mirror_about_edge": ("            num = 2 * (in_len - 1) * den - num;",
                          "            num = 2 * (in_len - 1) * den - num - den;"),
    "wrap_neighbour_clamped": ("        return (i + 1 < len) ? (i + 1) : 0;",
                               "        return (i + 1 < len) ? (i + 1) : (len - 1);"),
    # the corner-aligned floor mapping rounding instead of flooring
    "corner_floor_rounds": ("k = floor_div(d * in_len, out_len);",
                            "k = floor_div(2 * d * in_len + out_len, 2 * out_len);"),
    # the corner-aligned round mapping rounding halves down
    "corner_round_half_down": ("k = floor_div(2 * d * in_len + out_len, 2 * out_len);   /* floor(x + 1/2) */",
                               "k = floor_div(2 * d * in_len + out_len - 1, 2 * out_len);"),
}
# (truncating instead of flooring the division is an equivalent mutant: the
# coordinate is clamped to be non-negative before it is divided.)


def _pin_calls():
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        argsets = [()]
        for mark in getattr(fn, "pytestmark", []):
            if mark.name == "parametrize":
                multi = "," in mark.args[0]
                argsets = [tuple(v) if multi else (v,) for v in mark.args[1]]
        for args in argsets:
            yield name, fn, args


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, monkeypatch):
    before, after = MUTANTS[mutant]
    assert _SRC.count(before) == 1, "mutation site not found"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "m.c")
        so = os.path.join(d, "m.so")
        open(c, "w").write(_SRC.replace(before, after))
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", c, "-o", so])
        monkeypatch.setattr(oracle, "_SRC", c)
        monkeypatch.setattr(oracle, "_LIB", so)
        monkeypatch.setattr(oracle, "_lib", None)
        caught = None
        for name, fn, args in _pin_calls():
            try:
                fn(*args)
            except AssertionError:
                caught = name
                break
        monkeypatch.setattr(oracle, "_lib", None)
    assert caught is not None, "no pin fails for mutant %s" % mutant


def _grey_swapped_rb(src):
    src = oracle._as_nhwc(src)
    r, g, b = (src[..., k:k + 1].astype(np.int64) for k in range(3))
    return ((114 * r + 587 * g + 299 * b + 500) // 1000).astype(np.uint8)


def _grey_truncated(src):
    src = oracle._as_nhwc(src)
    r, g, b = (src[..., k:k + 1].astype(np.int64) for k in range(3))
    return ((299 * r + 587 * g + 114 * b) // 1000).astype(np.uint8)


@pytest.mark.parametrize("mutant", [_grey_swapped_rb, _grey_truncated])
def test_grey_pins_catch_mutant(mutant, monkeypatch):
    """The grey conversion lives in the Python half of the oracle: swap its
    red and blue weights, or truncate instead of rounding, and its pins fail."""
    monkeypatch.setattr(oracle, "rgb_to_grey", mutant)
    with pytest.raises(AssertionError):
        pins.test_grey_closed_forms()
