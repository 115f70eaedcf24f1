"""The host code that runs without a GPU (argument validation in
pa_api.hip, the block pool in block_pool.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer.

build() also makes libpa_sanitized.so: the same exports, with those host
files rebuilt with both sanitizers.  Here the ABI and block-pool tests run in
a child process against it, with the sanitizer runtime preloaded; the child
must pass and print no sanitizer report.
"""

import os
import subprocess
import sys

import pytest

from paged_kv_cache_396_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_is_clean_under_asan_and_ubsan():
    if not os.path.exists(B.SAN_LIB):
        pytest.skip("libpa_sanitized.so is not built (python -m paged_kv_cache_396_amd.build)")
    rt = B.sanitizer_runtime()
    assert os.path.exists(rt), f"sanitizer runtime not found: {rt}"
    env = dict(os.environ)
    env.update({
        "PA_LIB": B.SAN_LIB,
        "LD_PRELOAD": rt,
        # Python itself is not instrumented and keeps its allocations to exit
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "tests/test_abi.py", "tests/test_block_pool.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in ("AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in out, out[-4000:]
    assert " passed" in r.stdout
