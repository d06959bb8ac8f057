"""Build libdgc.so for gfx950 with hipcc, in-tree.

    python -m sparsified_gradient_compression_amd.build

Floating-point flags: no FMA contraction, IEEE denormals kept, and packed
FP32 instructions disabled, so every binary32 operation rounds once, as the
method's arithmetic is defined.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libdgc.so")
SOURCES = [os.path.join(CSRC, "dgc_api.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, f) for f in
                     ("dgc_device.hpp", "kernel_fused.hpp", "kernels_binlocal.hpp", "kernels_sampled.hpp",
                      "kernels_compress.hpp", "kernels_codec.hpp", "kernels_shared.hpp", "kernels_tensor.hpp")] + [os.path.join(ROOT, "include", "dgc.h")]

ARCH = os.environ.get("DGC_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return exe


def build(verbose=True):
    """Compile libdgc.so (always recompiles)."""
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def is_stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in DEPENDS)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
