"""Build libspmm.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libspmm.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["api.cpp", "pack.cpp", "bcsr_bf16.hip", "wcsr_f32.hip", "sp24.hip", "sddmm_csr.hip", "sddmm_bcsr.hip"]
ARCH = "gfx950"

# Every HIP object is built with packed fp32 arithmetic disabled.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _compile(src: str, verbose: bool, extra=(), build_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc()] + COMMON + list(extra) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def build(verbose: bool = False, out: str = LIB, build_dir: str = BUILD_DIR) -> str:
    """Compile every source and link `out`."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir=build_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU
# tests: the packers, the ABI and the host side of every .hip file (the device
# code is built as usual, without sanitizers).  The process that loads it must
# preload the clang ASan runtime (asan_runtime()).
SANITIZE = ["-O1", "-g",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZED_LIB = os.path.join(BUILD_DIR, "sanitize", "libspmm.so")


def asan_runtime() -> str:
    """Path of the clang ASan runtime that matches hipcc."""
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang ASan runtime not found under /opt/rocm/llvm")
    return found[-1]


def build_sanitized(verbose: bool = False) -> str:
    """Compile every source's host code with ASan + UBSan into SANITIZED_LIB."""
    d = os.path.dirname(SANITIZED_LIB)
    os.makedirs(d, exist_ok=True)
    common = [c for c in COMMON if c != "-O3"] + SANITIZE

    def comp(src):
        obj = os.path.join(d, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [_hipcc()] + common + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (sanitized) failed on {src}:\n{r.stderr[-4000:]}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(comp, SOURCES))
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", SANITIZED_LIB] + objs
    subprocess.run(cmd, check=True)
    return SANITIZED_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
