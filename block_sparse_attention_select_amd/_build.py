"""Builds libmsa.so (the HIP library behind include/msa.h) in-tree for gfx950."""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmsa.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["select.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dkdv.hip", "qk_norm.hip", "qsa_attn.hip",
           "noalloc.hip", "msa_api.cpp",
           "timing.cpp"]

# -packed-fp32-ops keeps the compiler from emitting packed fp32 VALU forms.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MSA library needs ROCm's hipcc to build")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or r.returncode != 0:
        print(" ".join(cmd))
        print(r.stdout + r.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libmsa.so; always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or r.returncode != 0:
        print(" ".join(cmd))
        print(r.stdout + r.stderr)
    if r.returncode != 0:
        raise RuntimeError("linking libmsa.so failed")
    os.replace(tmp, LIB)
    return LIB


# Host-code sanitizers for the CPU checks of the ABI: address and undefined
# behaviour instrumentation of the host side of every source (each
# -fsanitize= applies to the host pass only; device code is built as usual).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_DIR = os.path.join(PKG, "_build_asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libmsa_asan.so")


def build_sanitized(verbose: bool = False) -> str:
    """libmsa_asan.so: the library with sanitized host code (for tests/abi_host_check.cpp)."""
    os.makedirs(ASAN_DIR, exist_ok=True)

    def one(src: str) -> str:
        obj = os.path.join(ASAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *FLAGS, *SANITIZE, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if verbose or r.returncode != 0:
            print(" ".join(cmd))
            print(r.stdout + r.stderr)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} (sanitized) failed")
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(one, SOURCES))
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *SANITIZE, "-o", ASAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or r.returncode != 0:
        print(" ".join(cmd))
        print(r.stdout + r.stderr)
    if r.returncode != 0:
        raise RuntimeError("linking libmsa_asan.so failed")
    return ASAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
