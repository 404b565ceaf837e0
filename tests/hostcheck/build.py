"""Build libdpnorm's host layer for the CPU under AddressSanitizer and
UndefinedBehaviorSanitizer (test infrastructure).

The library's sources are compiled host-only (no device code), the HIP
runtime functions they import come from fake_hip.cpp, and the per-file device
code objects a host-only build leaves undefined are pointed at a dummy. The
results are the sanitized library (for tests/test_abi.py through ctypes, with
the sanitizer runtime preloaded into Python) and the fuzz_plan driver (the
runtime linked in).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "sample_grad_norms_amd", "csrc")
SOURCES = ["dpnorm.cpp", "kernels_hutch.hip", "kernels_hutchpp.hip", "kernels_exact.hip", "kernels_calib.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
COMMON = ["-O1", "-g", "-std=c++17", "-fPIC", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm clang (to preload)."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return found[-1]


def run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
        raise RuntimeError(f"build step failed: {cmd[0]} (exit {res.returncode})")
    return res.stdout


def build(out_dir: str) -> dict:
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src + ".o")
        run([HIPCC, *COMMON, "--offload-arch=gfx950", "--offload-host-only", *SAN, "-I", CSRC, "-x", "hip", "-c",
             os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    fake = os.path.join(out_dir, "fake_hip.o")
    run([HIPCC, *COMMON, *SAN, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-c",
         os.path.join(HERE, "fake_hip.cpp"), "-o", fake])
    fatbins = set()
    for line in run(["nm", "--undefined-only", *objs]).splitlines():
        parts = line.split()
        if parts and parts[-1].startswith("__hip_fatbin"):
            fatbins.add(parts[-1])
    defsyms = [f"-Wl,--defsym,{s}=dpnorm_fake_fatbin" for s in sorted(fatbins)]
    lib = os.path.join(out_dir, "libdpnorm_hostcheck.so")
    run([HIPCC, "-shared", *SAN, *objs, fake, *defsyms, "-nogpulib", "-o", lib])
    fuzz = os.path.join(out_dir, "fuzz_plan")
    fobj = os.path.join(out_dir, "fuzz_plan.o")
    run([HIPCC, *COMMON, *SAN, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-c",
         os.path.join(HERE, "fuzz_plan.cpp"), "-o", fobj])
    run([HIPCC, *SAN, fobj, *objs, fake, *defsyms, "-nogpulib", "-o", fuzz])
    return {"lib": lib, "fuzz": fuzz, "asan_runtime": asan_runtime()}


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "_build", "hostcheck")))
