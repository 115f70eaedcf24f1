"""MI355X (gfx950) paged KV-cache attention: cache writes (bf16, fp32 and
fp8 E4M3 pools), paged decode with split-K, shared-prefix decode, chunked
prefill, block copies, a host block pool and speculative-decoding
verification, as hand-written HIP kernels behind a C ABI
(``include/pa.h``).  This package holds the kernels' sources (``csrc/``), the
build step and a ctypes binding; torch supplies device memory and streams."""

from .binding import (  # noqa: F401
    BLOCK_SIZE,
    PA_ERR_NO_BLOCKS,
    BlockPool,
    PA_BF16,
    PA_F32,
    PA_FP8_E4M3,
    CacheDesc,
    PAError,
    cache_desc,
    lib,
    pa_bw_probe,
    pa_cache_bytes,
    pa_copy_blocks,
    pa_decode,
    pa_decode_append,
    pa_decode_append_noalloc,
    NOALLOC_SCRATCH_BYTES,
    pa_decode_partition_size,
    pa_decode_shared_prefix,
    pa_decode_shared_prefix_workspace_bytes,
    pa_decode_workspace_bytes,
    pa_prefill_chunk,
    pa_prefill_chunk_workspace_bytes,
    pa_rejection_sample,
    pa_rejection_sample_workspace_bytes,
    pa_reshape_and_cache,
)
