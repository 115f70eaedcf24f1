"""Build libpa.so (the gfx950 paged-attention library) in place with hipcc.

    python -m paged_kv_cache_396_amd.build [--no-sanitized]

Every ``csrc/*.hip`` file (and host-only ``csrc/*.cpp``) is compiled to an
object in parallel, then linked
into ``paged_kv_cache_396_amd/libpa.so``.  Only the C-ABI symbols declared in
``include/pa.h`` are exported.

A second library, ``libpa_sanitized.so``, has the same exports with the
host code that runs without a GPU (argument validation in ``pa_api.hip``,
the block pool in ``block_pool.cpp``) built with AddressSanitizer and
UndefinedBehaviorSanitizer; its kernels are the objects of the main build.
The CPU test ``tests/test_sanitized_host.py`` loads it (with the sanitizer
runtime preloaded) under the ABI and block-pool tests.  GPU code is never
built with a sanitizer.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
SAN_LIB = os.path.join(PKG, "libpa_sanitized.so")
SAN_BUILD = os.path.join(BUILD, "sanitized")
# host-only sanitizer flags; for hipcc each one is scoped to the host pass
SAN_HOST = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer", "-g"]
SAN_CXX = os.environ.get("PA_SAN_CXX", "/opt/rocm/llvm/bin/clang++")
# the host files the sanitized library rebuilds
SAN_SOURCES = ("pa_api.hip", "block_pool.cpp")


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime of the compiler that built
    libpa_sanitized.so (preload it before loading that library)."""
    out = subprocess.run([SAN_CXX, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    return out.stdout.strip()
# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx feature flag; drop that notice only
    err = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False, sanitized: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]
    extra = os.environ.get("PA_EXTRA_FLAGS", "").split()

    def compile_one(pair):
        src, obj = pair
        if src.endswith(".cpp"):  # host-only code
            cmd = [CXX, "-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"-I{INCLUDE}",
                   f"-I{CSRC}", "-c", src, "-o", obj]
        else:
            cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if sanitized:
        build_sanitized(srcs, objs, verbose)
    return LIB


def build_sanitized(srcs, objs, verbose=False):
    """libpa_sanitized.so: the host files rebuilt with ASan + UBSan, linked
    with the main build's other objects.  The sanitizer runtime is left
    unresolved; it is preloaded by whoever loads the library."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    linked = []
    for src, obj in zip(srcs, objs):
        name = os.path.basename(src)
        if name not in SAN_SOURCES:
            linked.append(obj)
            continue
        sobj = os.path.join(SAN_BUILD, name + ".o")
        if src.endswith(".cpp"):
            cmd = [SAN_CXX, "-O1", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"-I{INCLUDE}",
                   f"-I{CSRC}", *SAN_HOST, "-c", src, "-o", sobj]
        else:
            host_only = [f for flag in SAN_HOST for f in ("-Xarch_host", flag)]
            cmd = [HIPCC, *COMMON, *host_only, "-c", src, "-o", sobj]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        linked.append(sobj)
    tmp = SAN_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *linked])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitized="--no-sanitized" not in sys.argv))
