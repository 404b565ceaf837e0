"""Build libdpnorm.so in-tree with hipcc for gfx950.

The library is one shared object holding the HIP kernels and the C-ABI host
layer. It is built next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libdpnorm.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = [
    "kernels_hutch.hip",
    "kernels_hutchpp.hip",
    "kernels_exact.hip",
    "kernels_calib.hip",
    "dpnorm.cpp",
]

# Packed-fp32 VALU forms are disabled for all device code (-packed-fp32-ops);
# the host pass warns that it does not know the feature, which is harmless.
HIP_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libdpnorm needs the ROCm toolchain to build")


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source into LIB_PATH (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=HERE, prefix=".libdpnorm.")
    os.close(fd)
    cmd = [hipcc(), *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        os.unlink(tmp)
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {LIB_NAME} (exit {res.returncode})")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
