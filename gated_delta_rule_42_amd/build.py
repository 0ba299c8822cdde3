"""Build libkda.so (the C-ABI library of HIP kernels for gfx950) in-tree.

    python -m gated_delta_rule_42_amd.build

Each .hip source compiles to an object under _build/, then hipcc links the
shared library next to this file, where the binding loads it from.
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
BUILD = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.hip", "decode.hip", "prefill.hip", "norm.hip", "conv.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # Keep the compiler from forming packed-fp32 instructions.
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # Export only the entry points that kda.h marks KDA_API.
         "-fvisibility=hidden",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


# Host AddressSanitizer + UndefinedBehaviorSanitizer for kda_api.hip (the
# entry points' argument checks; device code is unchanged).  A process that
# loads the result must preload clang's ASan runtime.
HOST_SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()
HOST_SANITIZED = os.path.join(BUILD, "libkda_hostsan.so")


def asan_runtime() -> str:
    """clang's ASan runtime for the host compiler hipcc drives."""
    res = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang ASan runtime not found")
    return found[-1]


def build_host_sanitized() -> str:
    """libkda_hostsan.so: kda_api.hip compiled with HOST_SANITIZE, linked with
    the other sources' objects from the last build() (built first if
    missing).  Returns the library path."""
    others = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "kda_api.hip"]
    if not all(os.path.exists(o) for o in others):
        build()
    obj = os.path.join(BUILD, "kda_api_hostsan.o")
    cmd = [_hipcc(), *FLAGS, *HOST_SANITIZE, "-c", os.path.join(CSRC, "kda_api.hip"), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    tmp = HOST_SANITIZED + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", obj, *others, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, HOST_SANITIZED)
    return HOST_SANITIZED


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print("built", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
