"""Build libbcjr.so (HIP kernels + C-ABI) for gfx950, in-tree.

Usage: ``python -m differentiable_bcjr_amd.build [--incremental]`` or ``build()`` from Python.  Every translation unit is compiled
with hipcc for gfx950 only, then linked into ``differentiable_bcjr_amd/libbcjr.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbcjr.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["soft.hip", "grad.hip", "viterbi.hip", "tail_biting.hip", "general.hip", "bcjr_abi.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # a multiply and an add are fused only where one expression holds both (or fmaf says so), never across statements:
    # the rounding of every result is then fixed by the source alone, so kernels that share code (the full-tape and the
    # checkpoint forms, the codebook-gradient forms) give bit-identical shared outputs
    "-ffp-contract=on",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbcjr.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _stale(src: str) -> bool:
    """The object of src is missing or older than src or any header it may include."""
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(d, f) for d in (CSRC, INCLUDE) for f in os.listdir(d)
                                        if f.endswith((".hpp", ".h"))]
    return os.path.getmtime(obj) < max(os.path.getmtime(d) for d in deps)


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every HIP source for gfx950 (with ``incremental``, only those whose object is out of date) and link
    libbcjr.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    todo = [s for s in SOURCES if not incremental or _stale(s)]
    jobs = min(max(len(todo), 1), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# The host side of the C-ABI (argument checks, workspace planning, dispatch) built with AddressSanitizer and
# UndefinedBehaviorSanitizer: host code only, each -fsanitize behind -Xarch_host so no GPU code is instrumented.  Load it
# with clang's ASan runtime preloaded (libclang_rt.asan) and BCJR_LIB pointing at it.
SANITIZE_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """clang's AddressSanitizer runtime, which the sanitized library needs preloaded."""
    llvm = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "lib", "clang")
    for root, _, files in os.walk(os.path.realpath(llvm)):
        if "libclang_rt.asan-x86_64.so" in files:
            return os.path.join(root, "libclang_rt.asan-x86_64.so")
    raise RuntimeError("libclang_rt.asan-x86_64.so not found")


def build_sanitized(path: str) -> str:
    """libbcjr.so with its C-ABI translation unit (every check and workspace plan) rebuilt with the host sanitizers,
    linked with the kernels' objects of the last build into `path`; returns path."""
    obj = path + ".abi.o"
    cmd = [hipcc(), "-x", "hip", *HIPCC_FLAGS, *SANITIZE_HOST_FLAGS, "-c", os.path.join(CSRC, "bcjr_abi.cpp"), "-o",
           obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on bcjr_abi.cpp:\n{r.stdout}\n{r.stderr}")
    objs = [obj if s == "bcjr_abi.cpp" else os.path.join(BUILD_DIR, s + ".o") for s in SOURCES]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build() first: missing {missing}")
    r = subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", *objs, "-o", path], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.remove(obj)
    return path


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
