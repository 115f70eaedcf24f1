"""Host-only checks of the C ABI: the library loads, exports every entry point
that include/pa.h declares, and rejects bad arguments before touching a GPU."""

import ctypes
import os
import re

import pytest

import paged_kv_cache_396_amd as pa
from paged_kv_cache_396_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    L = pa.lib()
    names = declared_functions()
    assert "pa_decode" in names and "pa_reshape_and_cache" in names and "pa_prefill_chunk" in names
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/ but not exported"


def test_abi_version_and_status_strings():
    L = pa.lib()
    assert L.pa_abi_version() == 3
    assert L.pa_status_string(0) == b"ok"
    assert L.pa_status_string(-5) == b"workspace too small"
    assert L.pa_status_string(123) == b"unknown status"


def test_cache_bytes():
    d = pa.cache_desc(10, 8, 128, pa.PA_BF16)
    assert pa.pa_cache_bytes(d) == 10 * 8 * 16 * 128 * 2
    d = pa.cache_desc(32, 2, 64, pa.PA_F32)
    assert pa.pa_cache_bytes(d) == 32 * 2 * 16 * 64 * 4
    for bad in (pa.CacheDesc(10, 8, 8, 128, 1), pa.CacheDesc(10, 16, 8, 96, 1),
                pa.CacheDesc(0, 16, 8, 128, 1), pa.CacheDesc(10, 16, 8, 128, 7),
                pa.CacheDesc(1 << 28, 16, 1, 64, 1)):
        assert pa.pa_cache_bytes(bad) == 0


def test_fp8_cache_bytes_and_scales():
    d = pa.cache_desc(10, 8, 128, pa.PA_FP8_E4M3, 0.5, 0.25)
    assert pa.pa_cache_bytes(d) == 10 * 8 * 16 * 128
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0), (1.0, float("nan"))):
        assert pa.pa_cache_bytes(pa.cache_desc(10, 8, 128, pa.PA_FP8_E4M3, ks, vs)) == 0
    # scales of bf16 / fp32 pools are ignored
    assert pa.pa_cache_bytes(pa.cache_desc(10, 8, 128, pa.PA_BF16, 0.0, float("nan"))) > 0


def test_fp8_unsupported_variants_and_bad_scales():
    L = pa.lib()
    p = ctypes.c_void_p(1)
    bad_scale = pa.cache_desc(16, 2, 128, pa.PA_FP8_E4M3, 0.0, 1.0)
    assert L.pa_reshape_and_cache(p, p, p, 4, p, p, ctypes.byref(bad_scale), None) == -2
    assert b"k_scale" in L.pa_last_error()
    assert _decode_raw(pa.cache_desc(16, 2, 64, pa.PA_FP8_E4M3, 1.0, 1.0)) == -4   # D = 64
    assert _decode_raw(pa.cache_desc(16, 2, 128, pa.PA_FP8_E4M3, 1.0, 1.0), ws=None) == -5


def _decode_raw(desc, num_seqs=2, num_q_heads=8, partition=64, max_ctx=100, mb=8,
                ptr=1, ws=None, ws_bytes=0):
    L = pa.lib()
    p = ctypes.c_void_p(ptr) if ptr else ctypes.c_void_p(0)
    return L.pa_decode(p, p, p, p, p, mb, p, max_ctx, num_seqs, num_q_heads, 0.125, partition,
                       ws, ws_bytes, ctypes.byref(desc) if desc is not None else None,
                       ctypes.c_void_p(0))


def test_decode_argument_errors_return_codes():
    good = pa.cache_desc(16, 2, 64, pa.PA_F32)
    assert _decode_raw(None) == -1
    assert _decode_raw(pa.CacheDesc(16, 8, 2, 64, 0)) == -4          # block size
    assert _decode_raw(pa.CacheDesc(16, 16, 2, 80, 0)) == -4         # head dim
    assert _decode_raw(pa.CacheDesc(16, 16, 2, 64, 9)) == -3         # dtype
    assert _decode_raw(good, num_q_heads=7) == -2                    # Hq % Hkv
    assert _decode_raw(good, num_q_heads=32) == -4                   # G = 16 not built
    assert _decode_raw(good, partition=24) == -2                     # not a multiple of 16
    assert _decode_raw(good, num_seqs=-1) == -2
    assert _decode_raw(good, ptr=0) == -1                            # null tensors
    assert b"non-NULL" in pa.lib().pa_last_error()
    # 100 tokens in 64-token partitions needs a workspace
    assert _decode_raw(good, ws=None, ws_bytes=0) == -5
    assert _decode_raw(good, num_seqs=0) == 0                        # nothing to do


def test_workspace_size_formula():
    # 2 partitions of 64 tokens for a 100-token context
    # partial states (m, l, O) per (seq, q head, partition)
    assert pa.pa_decode_workspace_bytes(2, 8, 2, 64, 100, 64) == 2 * 8 * 2 * (64 + 2) * 4
    assert pa.pa_decode_workspace_bytes(2, 8, 2, 64, 64, 64) == 0    # one partition
    assert pa.pa_decode_workspace_bytes(2, 8, 2, 64, 100, -1) == 0   # no split
    assert pa.pa_decode_workspace_bytes(2, 8, 2, 64, 100, 24) == 0   # invalid request


def test_balanced_schedule_choice_and_workspace():
    """Automatic calls that the partition rule would split run the balanced
    schedule (partition size reported as 0) for up to 1024 sequences; its
    workspace holds 2 partial slots per (kv head, range, group head), with
    ranges = CUs * 4 / Hkv for the workspace bound (no GPU here: 256 CUs)."""
    cus = 256
    # 64 seqs x 8 kv heads = 512 units < 4 per CU, contexts up to 4096: split
    assert pa.pa_decode_partition_size(64, 8, 4096, 0) == 0
    ranges = cus * 4 // 8
    assert pa.pa_decode_workspace_bytes(64, 32, 8, 128, 4096, 0) == ranges * 2 * 32 * (128 + 2) * 4
    # explicit partitions and "no split" keep the per-partition schedule
    assert pa.pa_decode_partition_size(64, 8, 4096, 512) == 512
    assert pa.pa_decode_workspace_bytes(64, 32, 8, 128, 4096, 512) == 64 * 32 * 8 * (128 + 2) * 4
    assert pa.pa_decode_partition_size(64, 8, 4096, -1) == 4096
    # enough units for the chip: no split, no workspace
    assert pa.pa_decode_partition_size(256, 8, 2048, 0) == 2048
    assert pa.pa_decode_workspace_bytes(256, 64, 8, 128, 2048, 0) == 0
    # short contexts that the rule would not split
    assert pa.pa_decode_partition_size(4, 2, 64, 0) == 64
    # up to 1023 (sequence, kv head) units on 256 CUs: balanced; 1024 units
    # are 4 per CU, which the partition rule does not split
    assert pa.pa_decode_partition_size(1023, 1, 3000, 0) == 0
    assert pa.pa_decode_partition_size(1024, 1, 3000, 0) == 3008


def test_decode_append_argument_errors():
    L = pa.lib()
    d = pa.cache_desc(16, 2, 64, pa.PA_BF16)
    one, z = ctypes.c_void_p(1), ctypes.c_void_p(0)

    def call(k=one, v=one, slots=one, desc=d, num_seqs=2, num_q_heads=8):
        return L.pa_decode_append(one, one, k, v, slots, one, one, one, 8, one, 100, num_seqs,
                                  num_q_heads, 0.125, -1, z, 0,
                                  ctypes.byref(desc) if desc is not None else None, z)

    assert call(k=z) == -1
    assert b"slot_mapping" in L.pa_last_error()
    assert call(v=z) == -1
    assert call(slots=z) == -1
    assert call(desc=None) == -1
    assert call(num_q_heads=7) == -2
    assert call(num_seqs=0, k=z, v=z, slots=z) == 0    # nothing to do


def test_reshape_and_cache_argument_errors():
    L = pa.lib()
    d = pa.cache_desc(16, 2, 64, pa.PA_BF16)
    z = ctypes.c_void_p(0)
    assert L.pa_reshape_and_cache(z, z, z, 0, z, z, ctypes.byref(d), z) == 0   # no tokens
    assert L.pa_reshape_and_cache(z, z, z, -1, z, z, ctypes.byref(d), z) == -2
    assert L.pa_reshape_and_cache(z, z, z, 4, z, z, ctypes.byref(d), z) == -1
    assert L.pa_reshape_and_cache(z, z, z, 4, z, z, None, z) == -1


def test_prefill_argument_errors():
    L = pa.lib()
    z = ctypes.c_void_p(0)
    d32 = pa.cache_desc(16, 2, 128, pa.PA_F32)
    d16 = pa.cache_desc(16, 2, 128, pa.PA_BF16)
    one = ctypes.c_void_p(1)

    def call(desc, num_reqs=1, max_ctx=100, heads=8, part=0, ws=z, ws_bytes=0, ptr=z, max_q=8):
        return L.pa_prefill_chunk(ptr, ptr, ptr, ptr, ptr, 4, ptr, ptr, num_reqs, 8, max_q, max_ctx,
                                  heads, 0.1, part, ws, ws_bytes, ctypes.byref(desc), z)

    # fp32 prefill is not built (MFMA path is bf16)
    assert call(d32) == -4
    assert call(d16, heads=7) == -2
    assert call(d16, num_reqs=-1) == -2
    assert call(d16, max_ctx=-1) == -2
    assert call(d16, part=100) == -2           # not a multiple of 64
    assert call(d16, num_reqs=0) == 0          # nothing to do
    # a requested split needs its workspace: refused before any launch
    need = L.pa_prefill_chunk_workspace_bytes(1, 8, 8, 4096, 8, 2, 128, 512)
    assert need > 0
    assert call(d16, max_ctx=4096, part=512, ptr=one) == -5
    assert call(d16, max_ctx=4096, part=512, ptr=one, ws=one, ws_bytes=need - 4) == -5


def test_prefill_workspace_sizes():
    L = pa.lib()
    # 8 rows, 8 q heads, D 128, parts of 512 keys over 4096: 8 parts per (row, head)
    slots = 8 * 8 * 8
    assert L.pa_prefill_chunk_workspace_bytes(1, 8, 8, 4096, 8, 2, 128, 512) == \
        ((2 * slots + 3) // 4 * 4 + slots * 128) * 4
    # no split: nothing needed
    assert L.pa_prefill_chunk_workspace_bytes(1, 8, 8, 4096, 8, 2, 128, -1) == 0
    assert L.pa_prefill_chunk_workspace_bytes(1, 8, 8, 400, 8, 2, 128, 512) == 0
    # the wide variant (a 512-row chunk) is never split automatically
    assert L.pa_prefill_chunk_workspace_bytes(4, 2048, 512, 4608, 32, 8, 128, 0) == 0
    # a few rows per request, long contexts, too few requests to fill the
    # chip: the automatic rule splits; enough requests: it does not
    assert L.pa_prefill_chunk_workspace_bytes(16, 80, 5, 4096, 32, 8, 128, 0) > 0
    assert L.pa_prefill_chunk_workspace_bytes(64, 320, 5, 4096, 32, 8, 128, 0) == 0


def test_binding_raises_with_detail():
    with pytest.raises(pa.PAError) as e:
        binding._check(-2)
    assert "PA_ERR_SHAPE" in str(e.value)


def test_bw_probe_argument_errors():
    L = pa.lib()
    z = ctypes.c_void_p(0)
    one = ctypes.c_void_p(1)
    assert L.pa_bw_probe(z, 4096, z, 0, z, z) == 0          # nothing to read
    assert L.pa_bw_probe(z, 4096, z, -1, z, z) == -2
    assert L.pa_bw_probe(z, 4096, one, 4, one, z) == -1
    assert L.pa_bw_probe(one, 100, one, 4, one, z) == -2    # no whole tile


def _shared_raw(desc, num_seqs=8, num_q_heads=8, max_ctx=100, mb=8, group_size=4, max_prefix=64,
                ptr=1, ws_bytes=0):
    L = pa.lib()
    p = ctypes.c_void_p(ptr) if ptr else ctypes.c_void_p(0)
    return L.pa_decode_shared_prefix(p, p, p, p, p, mb, p, max_ctx, num_seqs, num_q_heads, 0.125,
                                     p, group_size, max_prefix, p, ws_bytes,
                                     ctypes.byref(desc) if desc is not None else None,
                                     ctypes.c_void_p(0))


def test_shared_prefix_argument_errors():
    bf = pa.cache_desc(16, 2, 128, pa.PA_BF16)
    assert _shared_raw(None) == -1
    assert _shared_raw(pa.cache_desc(16, 2, 128, pa.PA_F32)) == -4   # bf16 only
    assert _shared_raw(bf, group_size=3) == -2                      # 8 seqs not in groups of 3
    assert _shared_raw(bf, group_size=0) == -2
    assert _shared_raw(bf, max_prefix=40) == -2                     # not a multiple of 16
    assert _shared_raw(bf, max_prefix=112) == -2                    # beyond max_context_len
    assert _shared_raw(bf, num_q_heads=7) == -2                     # Hq % Hkv
    assert _shared_raw(bf, num_seqs=128, group_size=128) == -4      # 128 x G 4 > 256 columns
    assert _shared_raw(bf, ptr=0) == -1
    assert _shared_raw(bf, ws_bytes=16) == -5                       # workspace too small
    assert b"workspace" in pa.lib().pa_last_error()
    assert _shared_raw(bf, num_seqs=0, group_size=1) == 0


def test_shared_prefix_workspace_size():
    f = pa.pa_decode_shared_prefix_workspace_bytes
    assert f(8, 8, 2, 128, 100, 3, 64) == 0      # bad group size
    assert f(8, 8, 2, 128, 100, 4, 40) == 0      # prefix not a multiple of 16
    n = f(8, 8, 2, 128, 100, 4, 64)
    # m and l per slot (rounded up to 4 floats), then D floats per slot
    rows = 8 * 8
    assert n > 0 and n % 4 == 0
    slots = (n // 4) // (128 + 2)
    assert slots >= 2                             # at least one prefix and one own slot
    assert n == 4 * (((2 * rows * (slots // rows) + 3) // 4) * 4 + rows * (slots // rows) * 128)


def test_rejection_sample_argument_errors():
    L = pa.lib()
    p = ctypes.c_void_p(1)
    n = ctypes.c_void_p(0)

    def call(B=2, k=4, V=100, tp=p, dt=p, u=p, out=p, num=p, ws=p, ws_bytes=1 << 20):
        return L.pa_rejection_sample(tp, n, dt, u, B, k, V, out, num, ws, ws_bytes, None)

    assert call(B=-1) == -2
    assert call(V=0) == -2
    assert call(k=33) == -4                       # more drafts than built
    assert call(V=(1 << 21) + 1) == -4            # vocabulary too large
    assert call(tp=n) == -1
    assert call(dt=n) == -1                       # k > 0 needs draft tokens
    assert call(u=n, B=0) == 0                    # nothing to do
    assert call(B=1 << 20, k=32, V=1 << 21) == -6  # index range
    assert call(B=70000, V=10) == -4               # grid limit
    assert call(ws=n) == -5                        # workspace missing
    assert call(B=64, V=128256, ws_bytes=64 * 501 * 8 - 1) == -5
    assert L.pa_rejection_sample_workspace_bytes(64, 128256) == 64 * 501 * 8
    assert L.pa_rejection_sample_workspace_bytes(0, 10) == 0
