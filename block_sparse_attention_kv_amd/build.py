"""Build libssa.so (the C-ABI HIP library) in-tree for gfx950 with hipcc.

Usage:  python -m block_sparse_attention_kv_amd.build  [--jobs N]
Each source is compiled to an object under ``_build/`` (in parallel), then
linked into ``block_sparse_attention_kv_amd/libssa.so``.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libssa.so")
SOURCES = ["ssa_api.cpp", "ssa_scores.hip", "ssa_topk.hip", "ssa_decode_select.hip", "ssa_attn.hip", "ssa_decode.hip",
           "ssa_bwd.hip", "ssa_route.hip"]
# measurement aid (include/ssa_peaks.h), a library of its own beside libssa
PEAKS_LIB = os.path.join(PKG, "libssa_peaks.so")
PEAKS_SOURCES = ["ssa_peaks.hip"]
ARCH = os.environ.get("SSA_OFFLOAD_ARCH", "gfx950")

CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libssa")
    return exe


def _compile(src: str, verbose: bool, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CXXFLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, jobs: int | None = None, out: str = LIB, build_dir: str = BUILD,
          defines=(), peaks: bool = True) -> str:
    """Compile every source and link the library (default: in-tree libssa.so),
    and the measurement library libssa_peaks.so beside it (``peaks``);
    ``defines`` are extra NAME=VALUE preprocessor definitions (tuning knobs)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = SOURCES + (PEAKS_SOURCES if peaks else [])
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2) // 2))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines), srcs))
    _link(objs[:len(SOURCES)], out, verbose)
    if peaks:
        _link(objs[len(SOURCES):], PEAKS_LIB, verbose)
    return out


ASAN_BUILD = os.path.join(PKG, "_build_asan")
ASAN_LIB = os.path.join(ASAN_BUILD, "libssa_asan.so")


def asan_runtime() -> str | None:
    """The compiler's AddressSanitizer runtime, preloaded into the (not
    instrumented) Python process that loads the instrumented library."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "..",
                                         "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    hits += sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return os.path.realpath(hits[0]) if hits else None


def build_asan(verbose: bool = False, jobs: int | None = None) -> str:
    """libssa with its host code built under AddressSanitizer (device code as
    usual), for running the host-layer tests under ASan on a CPU machine."""
    os.makedirs(ASAN_BUILD, exist_ok=True)
    flags = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer")
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2) // 2))

    def comp(src):
        obj = os.path.join(ASAN_BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *CXXFLAGS, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(comp, SOURCES))
    tmp = ASAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-fsanitize=address", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--asan", action="store_true", help="also build the host-ASan library (_build_asan/)")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose, jobs=args.jobs))
    if args.asan:
        print(build_asan(verbose=args.verbose, jobs=args.jobs))


if __name__ == "__main__":
    main(sys.argv[1:])
