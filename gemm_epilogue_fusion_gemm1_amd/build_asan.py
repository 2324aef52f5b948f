"""A copy of libcoda.so whose C-ABI host code (api.cpp: argument checks,
workspace carving, launch order) is built with AddressSanitizer, for the
CPU-side ABI tests.  The kernels' object is the one build.py makes (device
code is never sanitized); only the host code of the boundary is.

Usage: python -m gemm_epilogue_fusion_gemm1_amd.build_asan  (prints the path).
The sanitized library must be loaded into a process that has the matching
runtime preloaded: asan_runtime() names it (LD_PRELOAD), and leak detection is
switched off for Python (ASAN_OPTIONS=detect_leaks=0).
"""
from __future__ import annotations

import glob
import os

from . import build as _b

OUT = os.path.join(_b.BUILD, "asan")
LIB = os.path.join(OUT, "libcoda_asan.so")
CLANG = "/opt/rocm/llvm/bin/clang++"


def asan_runtime() -> str:
    """The shared ASan runtime of the ROCm clang that compiles the library."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("the ROCm clang ASan runtime (libclang_rt.asan-x86_64.so) is missing")
    return hits[-1]


def build_asan(verbose: bool = True) -> str:
    hipcc = _b._hipcc()
    kernels_o = os.path.join(_b.BUILD, "kernels.o")
    if not os.path.exists(kernels_o):
        _b.build(verbose)
    os.makedirs(OUT, exist_ok=True)
    api_o = os.path.join(OUT, "api_asan.o")
    # host-only sanitizer flags: each -fsanitize= sits right after -Xarch_host
    _b._run([hipcc, *_b.HIP_FLAGS, "-O1", "-g",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fno-omit-frame-pointer",
             "-c", os.path.join(_b.CSRC, "api.cpp"), "-o", api_o], verbose)
    rt_dir = os.path.dirname(asan_runtime())
    tmp = LIB + ".tmp"
    # host link of the two objects (no .hip source on this line)
    _b._run([CLANG, "-shared", "-fPIC", "-fsanitize=address", "-shared-libsan", "-o", tmp, api_o,
             kernels_o, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
             f"-Wl,-rpath,{rt_dir}"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_asan())
