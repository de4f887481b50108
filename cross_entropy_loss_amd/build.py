"""Builds the HIP library libce_mi355x.so in-tree with hipcc for gfx950.

    python -m cross_entropy_loss_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "ce_api.hip")
SRCS = [SRC] + [os.path.join(HERE, "csrc", f) for f in ("ce_linear.hip", "rmsnorm.hip", "rope.hip")]
HEADERS = ("ce_kernels.h", "ce_buffer.h", "row_formats.h", "lin_gemm.h")
DEPS = SRCS + [os.path.join(HERE, "csrc", h) for h in HEADERS] + [os.path.join(ROOT, "include", "ce_mi355x.h")]
LIBS: list = []  # no libraries beyond the HIP runtime
LIB = os.path.join(HERE, "libce_mi355x.so")
CALIB_SRC = os.path.join(HERE, "csrc", "calib_copy.hip")
CALIB_LIB = os.path.join(HERE, "libce_calib.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU ops anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def up_to_date() -> bool:
    if not os.path.exists(LIB):
        return False
    t = os.path.getmtime(LIB)
    return all(os.path.getmtime(d) <= t for d in DEPS)


def _compile(srcs, out: str, verbose: bool, libs=()) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-o", tmp] + list(srcs) + list(libs)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile the library and the counter-calibration copy (always when force=True)."""
    if not force and up_to_date() and os.path.exists(CALIB_LIB):
        return LIB
    _compile(SRCS, LIB, verbose, LIBS)
    _compile([CALIB_SRC], CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose="-v" in sys.argv))
