"""Build libmi_resize.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmi_resize.so")
SOURCES = [os.path.join(CSRC, "resize_abi.hip")]
# measurement program (launch and bandwidth ceilings), linked against the
# library; bench.py --ceiling runs it
CEILING_SRC = os.path.join(CSRC, "ceiling.hip")
CEILING = os.path.join(PKG, "mi_resize_ceiling")
DEPENDS = SOURCES + [os.path.join(CSRC, "resize_kernels.hpp"),
                     os.path.join(ROOT, "include", "mi_resize.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # No packed fp32 instructions (v_pk_add/mul/fma_f32) in the gfx950 code:
    # the device pass honours this feature.  The host (x86) pass does not
    # know it and prints that it ignores it; that warning is harmless.
    # tests/test_code_object.py checks the built code object for them.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def _compile(cmd, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = cmd + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        subprocess.check_call(cmd)
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)


def build(verbose: bool = False) -> str:
    """Compile the HIP sources into bilinear_image_resize_amd/libmi_resize.so,
    then the ceiling measurement program linked against it."""
    _compile([HIPCC] + FLAGS + SOURCES, LIB, verbose)
    exe_flags = [f for f in FLAGS if f not in ("-fPIC", "-shared")]
    _compile([HIPCC] + exe_flags + [CEILING_SRC, "-L", PKG, "-lmi_resize",
                                    "-Wl,-rpath,$ORIGIN"], CEILING, verbose)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPENDS)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
