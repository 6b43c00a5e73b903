"""Build libfp8fg.so (HIP, gfx950) in-tree.

    python -m fp8_fine_grained_x1_amd.build

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file.  Every call recompiles.

``build_host_sanitized()`` compiles the same sources with AddressSanitizer
and UndefinedBehaviorSanitizer on the host code only (argument validation,
launch planning; the GPU code is built as usual) into ``_build/hostsan/``,
for the CPU test that runs the C-ABI argument matrix under the sanitizers.
The sanitizer runtime is not linked in: the process that loads the library
preloads it (``asan_runtime()``).
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp8fg.so")

SOURCES = ["abi.cpp", "quant.hip", "gemm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I" + INCLUDE, "-I" + CSRC,
    "-ffp-contract=off",
    "-fvisibility=hidden", "-DFP8FG_BUILDING_LIBRARY",
]
DEVICE = [
    "--offload-arch=gfx950",
    # no packed-FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in architectural VGPRs: the GEMMs scale and promote
    # them with VALU instructions every K group, which cannot read AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


# host-only sanitizers: each option applies to the host compilation alone
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address,undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-g",
]
HOSTSAN_BUILD = os.path.join(BUILD, "hostsan")
HOSTSAN_LIB = os.path.join(HOSTSAN_BUILD, "libfp8fg_hostsan.so")


def _compile(src, outdir=BUILD, extra=()):
    obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + DEVICE + list(extra) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose=True):
    if not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found at %s" % HIPCC)
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    shutil.move(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def asan_runtime():
    """The clang AddressSanitizer runtime (with its UBSan handlers) that a
    process loading the host-sanitized library must preload."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib",
                                         "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found under the ROCm tree")
    return hits[-1]


def build_host_sanitized():
    """Objects and library with the host code under ASan + UBSan; returns
    (library path, object paths)."""
    if not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found at %s" % HIPCC)
    os.makedirs(HOSTSAN_BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, HOSTSAN_BUILD, HOST_SANITIZE), SOURCES))
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", "-o", HOSTSAN_LIB] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return HOSTSAN_LIB, objs


if __name__ == "__main__":
    build()
    sys.exit(0)
