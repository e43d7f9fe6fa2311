"""Write tests/golden/hand_cases.json from the oracle (and nothing else).

The pages print no worked resize example, so the stored cases are small
hand-checkable inputs whose expected outputs come from the oracle; the test
that reads them also checks each against a closed form it computes on its
own (block means, replication, ramps), so a stored value cannot drift
silently.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_cases.json")


def run(mode, src, dH, dW):
    """The oracle call a case's mode names."""
    if mode == "linear":
        return oracle.resize_linear(src, dH, dW)
    if mode == "grey":
        return oracle.resize_linear_grey(src, dH, dW)
    if mode.startswith("nearest_"):
        return oracle.resize_nearest(src, dH, dW, mapping=mode[len("nearest_"):])
    return oracle.resize_nearest(src, dH, dW)


def case(name, src, dH, dW, mode, note):
    out = run(mode, src, dH, dW)
    # one-channel sources are stored as H x W, others as H x W x C
    stored = src[0, :, :, 0] if src.shape[3] == 1 else src[0]
    return {"name": name, "mode": mode, "dtype": str(src.dtype), "src": stored.tolist(),
            "dst_hw": [dH, dW], "expected": out[0, :, :, 0].tolist(), "note": note}


def main():
    ramp = (16 * np.arange(16, dtype=np.uint8)).reshape(1, 4, 4, 1)   # S[y][x] = 16 (4y + x)
    tie = np.array([[0, 0], [0, 2]], dtype=np.uint8).reshape(1, 2, 2, 1)
    prim = np.array([[[255, 0, 0], [0, 255, 0], [0, 0, 255], [0, 0, 250], [255, 255, 255]]],
                    dtype=np.uint8).reshape(1, 1, 5, 3)
    grey_tie = np.array([[[255, 0, 0], [0, 255, 0]], [[0, 0, 255], [0, 0, 0]]],
                        dtype=np.uint8).reshape(1, 2, 2, 3)
    cases = [
        case("ramp4_to_2x2", ramp, 2, 2, "linear", "exact 2:1: each output is the mean of a 2x2 block"),
        case("ramp4_to_3x3", ramp, 3, 3, "linear", "weights 341/1024/1707 of 2048 per axis"),
        case("ramp4_to_8x8", ramp, 8, 8, "linear", "weights 1/4, 3/4; borders clamp"),
        case("ramp4_nearest_2x2", ramp, 2, 2, "nearest", "centres land on pixels 1 and 3"),
        case("ramp4_nearest_3x3", ramp, 3, 3, "nearest", "half-pixel map rounded half up"),
        case("ramp4_nearest_8x8", ramp, 8, 8, "nearest", "integer upscale replicates"),
        case("tie_2x2_to_1", tie, 1, 1, "linear", "mean 0.5 rounds half up to 1"),
        case("ramp4_nearest_floor_3x3", ramp, 3, 3, "nearest_floor",
             "corner-aligned 4d/3 = 0, 1.33, 2.67 floored: pixels 0, 1, 2"),
        case("ramp4_nearest_round_3x3", ramp, 3, 3, "nearest_round",
             "corner-aligned 4d/3 rounded half up: pixels 0, 1, 3"),
        case("grey_primaries", prim, 1, 5, "grey",
             "0.299 R + 0.587 G + 0.114 B rounded half up: 76.245, 149.685, 29.07, 28.5, 255"),
        case("grey_2x2_to_1", grey_tie, 1, 1, "grey",
             "greys 76, 150, 29, 0 average to 63.75 -> 64"),
    ]
    with open(OUT, "w") as fh:
        json.dump({"generated_by": "tests/golden/make_golden.py (oracle only)", "cases": cases}, fh, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
