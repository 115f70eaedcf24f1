"""CPU fp64 oracle for paged attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the library or its binding.
"""

from .paged_attention import (  # noqa: F401
    BLOCK_SIZE,
    attend,
    decode,
    gather,
    k_pool_bytes,
    k_pool_from_bytes,
    new_pool,
    prefill_chunk,
    raw_type,
    reshape_and_cache,
    reshape_and_cache_fast,
    v_pool_bytes,
    v_pool_from_bytes,
    widen,
)
