"""Builds libfia.so, the gfx950 C-ABI library, in-tree with hipcc.

The library leaves the HIP runtime symbols to the process: it is linked
against the libamdhip64 that torch ships (so one HIP runtime serves both
torch's allocations/streams and this library's launches), found through an
rpath; a C program links its own libamdhip64 first.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfia.so")
SOURCES = [os.path.join(CSRC, "fia_plan.cpp"), os.path.join(CSRC, "fia_kernels.hip")]
HEADERS = [os.path.join(CSRC, "fia_internal.h"), os.path.join(INCLUDE, "fia.h")]

ARCH = "gfx950"


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _torch_lib_dir() -> str | None:
    try:
        import torch  # noqa: F401
    except Exception:
        return None
    d = os.path.join(os.path.dirname(sys.modules["torch"].__file__), "lib")
    return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None


def compile_flags() -> list[str]:
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # no packed-fp32 instructions in generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libfia.so (always rebuilds
    unless ``force`` is False and the library is newer than its sources)."""
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in SOURCES + HEADERS)
        if os.path.getmtime(LIB) >= newest:
            return LIB
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [_hipcc()] + compile_flags() + lang + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        subprocess.check_call(cmd)
        objs.append(obj)
    link = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", LIB + ".tmp"] + objs
    tl = _torch_lib_dir()
    if tl:
        link += ["-L", tl, "-Wl,-rpath," + tl]
    if verbose:
        print(" ".join(link))
    subprocess.check_call(link)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
