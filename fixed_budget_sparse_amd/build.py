"""Build libkvpop.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m fixed_budget_sparse_amd.build   (or build_library() from Python)

Every source is compiled for gfx950 only, with packed-FP32 instructions
disabled, and linked into fixed_budget_sparse_amd/libkvpop.so.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvpop.so")
SOURCES = ["thresholds.hip", "masked_fwd.hip", "future_target.hip", "decode.hip", "handoff.hip",
           "labels.hip", "backward.hip", "api.hip"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libkvpop)")


COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [_hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build_library(extra=(), verbose: bool = True) -> str:
    """Compile every source and link libkvpop.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the whole
# library (device code unchanged): every sanitizer flag applies to the host
# pass only, so the C ABI's validation, workspace sizing and launch set-up are
# checked.  Used by tests/test_abi.py with a C driver that exercises the error
# paths on the CPU.
SANITIZE_HOST = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=undefined "
                 "-Xarch_host -fno-omit-frame-pointer").split()


def _llvm_bin(tool: str) -> str:
    return os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib", "llvm", "bin",
                        tool)


def asan_runtime_dir() -> str:
    """Directory of clang's shared sanitizer runtimes (empty if not found)."""
    r = subprocess.run([_llvm_bin("clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return os.path.dirname(path) if r.returncode == 0 and os.path.isabs(path) else ""


def build_sanitized(out_dir: str) -> str:
    """Compile every source with host-side ASan/UBSan into
    out_dir/libkvpop_san.so; returns its path."""
    os.makedirs(out_dir, exist_ok=True)

    def comp(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        cmd = [_hipcc(), *COMMON, "-O1", "-g", *SANITIZE_HOST, "-c", os.path.join(CSRC, src),
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitized hipcc failed for {src}:\n{r.stderr}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(comp, SOURCES))
    lib = os.path.join(out_dir, "libkvpop_san.so")
    rocm_lib = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib")
    cmd = [_llvm_bin("clang++"), "-shared", "-fPIC", "-fsanitize=address,undefined",
           "-shared-libsan", "-o", lib, *objs, "-L", rocm_lib, "-lamdhip64",
           "-Wl,-rpath," + rocm_lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return lib


if __name__ == "__main__":
    build_library()
