"""Build libpa.so (the gfx950 paged-attention library) in place with hipcc.

    python -m paged_kv_cache_396_amd.build

Every ``csrc/*.hip`` file (and host-only ``csrc/*.cpp``) is compiled to an
object in parallel, then linked
into ``paged_kv_cache_396_amd/libpa.so``.  Only the C-ABI symbols declared in
``include/pa.h`` are exported.
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


def build(verbose: bool = False) -> str:
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
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
