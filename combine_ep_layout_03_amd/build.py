"""Build libep.so (the HIP / C-ABI library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libep.so")

SOURCES = ["ep_api.cpp", "ep_layout.hip", "ep_dispatch.hip", "ep_combine.hip", "ep_fused.hip",
           "ep_expert.hip", "ep_router.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources() -> list[str]:
    return [os.path.join(CSRC, s) for s in SOURCES]


# HIP test kernels under tests/hip/ (each its own small shared library, loaded
# only by the tests): built with the library's flags and its device headers.
TEST_HIP = os.path.join(ROOT, "tests", "hip")
TEST_KERNELS = ["cvt_e4m3"]


def test_kernel_path(name: str) -> str:
    return os.path.join(TEST_HIP, "lib%s.so" % name)


def build_test_kernels(verbose: bool = False) -> list[str]:
    out = []
    for name in TEST_KERNELS:
        lib = test_kernel_path(name)
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-shared",
               os.path.join(TEST_HIP, name + ".hip"), "-o", tmp]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
        out.append(lib)
    return out


EXAMPLE_SRC = os.path.join(ROOT, "examples", "ep_c_example.c")
EXAMPLE = os.path.join(ROOT, "examples", "ep_c_example")


def build(verbose: bool = False) -> str:
    """Compile every source into libep.so (always rebuilds), then the plain-C
    example program against it and the HIP test kernels.  Returns the
    library's path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-shared", *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_example(verbose)
    build_test_kernels(verbose)
    return LIB


def build_example(verbose: bool = False) -> str:
    """The C example (examples/ep_c_example.c): gcc, C11, linked to libep.so
    and the HIP runtime, found at run time through rpath."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cc = os.environ.get("CC") or shutil.which("gcc") or "cc"
    tmp = EXAMPLE + ".tmp%d" % os.getpid()
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
           "-I", os.path.join(rocm, "include"), EXAMPLE_SRC, "-L", PKG, "-lep",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../combine_ep_layout_03_amd", "-Wl,-rpath," + os.path.join(rocm, "lib"),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXAMPLE)
    return EXAMPLE


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + [os.path.join(CSRC, "ep_internal.h"), os.path.join(CSRC, "ep_device.h"),
                        os.path.join(INCLUDE, "ep.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build(verbose=True))
