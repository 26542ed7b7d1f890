"""Build the MATE mixer shared library (liblingen_mate.so) for gfx950 in-tree.

    python -m linear_complexity_video_mate_amd.build [-v]

Compiles every HIP/C++ source under csrc/ with hipcc and links them into
``linear_complexity_video_mate_amd/liblingen_mate.so``.  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "liblingen_mate.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = os.environ.get("LINGEN_OFFLOAD_ARCH", "gfx950")

SOURCES = ["lingen_host.cpp", "lingen_kernels.hip", "dense_attn.hip", "tesa_bwd.hip", "block_steps.hip",
           "lingen_block.cpp", "ma_bwd.hip", "tesa_window.hip", "lingen_noalloc.hip"]
# The block's projections are plain GEMMs, left to rocBLAS.
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
LINK_FLAGS = [f"-L{ROCM}/lib", "-lrocblas", f"-Wl,-rpath,{ROCM}/lib"]

COMMON_FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # never let the backend form packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
    "-Wall",
    "-Wno-unused-function",
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build the library")
    return path


# Per-source additions.  The dense and windowed attention kernels never
# produce or consume NaN (masked scores are -inf, exp2(-inf) = 0), so they
# are built without NaN semantics: their maxima then need no NaN-quieting
# instructions around v_max.
SOURCE_FLAGS = {"dense_attn.hip": ["-fno-honor-nans"], "tesa_window.hip": ["-fno-honor-nans"]}


# AddressSanitizer on the host code only (the device code is built as
# usual): the variant that tests/test_abi_cpu.py runs against on the CPU.
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_LIB_PATH = os.path.join(BUILD_DIR, "asan", "liblingen_mate_asan.so")


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm clang that builds the
    variant (to be preloaded into an uninstrumented Python)."""
    import glob

    found = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("the ROCm clang AddressSanitizer runtime was not found")
    return found[-1]


def _compile(src: str, verbose: bool, asan: bool = False) -> str:
    out_dir = os.path.join(BUILD_DIR, "asan") if asan else BUILD_DIR
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), *(ASAN_FLAGS if asan else []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build(verbose: bool = False, asan: bool = False) -> str:
    """Compile and link the library; with asan, the host-ASan variant at
    ASAN_LIB_PATH instead of the library at LIB_PATH."""
    out = ASAN_LIB_PATH if asan else LIB_PATH
    os.makedirs(os.path.dirname(out) if asan else BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, asan), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *(["-shared-libasan", *ASAN_FLAGS] if asan else []),
           "-o", tmp, *objs, *LINK_FLAGS]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(out)} failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
