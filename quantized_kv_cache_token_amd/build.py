"""Build the HIP library liblkv.so for gfx950 with hipcc (in-tree).

    python -m quantized_kv_cache_token_amd.build

Kernels that compute quantisation codes (append, tier update) are compiled
with -ffp-contract=off so that their fp32 arithmetic is exactly the stated
sequence of IEEE operations.  Packed-fp32 instructions are disabled for all
device code.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblkv.so")

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]
SOURCES = [
    ("append.hip", ["-ffp-contract=off"]),
    ("tier.hip", ["-ffp-contract=off"]),
    ("decode.hip", []),
    ("decode_mfma.hip", []),
    ("decode_f16.hip", []),
    ("probe.hip", []),
    ("api.cpp", ["-x", "hip"]),
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    for src, extra in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
        cmd = [cc, *COMMON, *extra, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


ASAN_LIB = os.path.join(BUILD, "liblkv_asan.so")


def asan_runtime() -> str | None:
    """The compiler's shared AddressSanitizer runtime, if present."""
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm", "lib", "clang")
    for cand in sorted(glob.glob(os.path.join(root, "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))):
        return cand
    return None


def build_asan(verbose: bool = False) -> str:
    """The library with its host code (the C ABI's validation, planning and
    launch set-up in api.cpp) built with AddressSanitizer; device code as in
    build().  Written to _build/liblkv_asan.so, for CPU tests that load it
    with the sanitizer runtime preloaded."""
    cc = hipcc()
    objs = []
    for src, _ in SOURCES:
        if src == "api.cpp":
            continue
        obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
        if not os.path.exists(obj):
            build(verbose)
        objs.append(obj)
    api = os.path.join(BUILD, "api_cpp_asan.o")
    cmd = [cc, *COMMON, "-x", "hip", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           "-c", os.path.join(CSRC, "api.cpp"), "-o", api]
    for c in (cmd, [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, api, "-Xarch_host",
                    "-fsanitize=address", "-shared-libsan", "-o", ASAN_LIB]):
        if verbose:
            print(" ".join(c), flush=True)
        r = subprocess.run(c, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("ASan build failed")
    return ASAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
