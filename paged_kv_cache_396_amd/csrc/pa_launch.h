// Host-side launch entry points of the kernels (C++ linkage, internal to
// libpa.so).  Argument validation happens in pa_api.hip before these run;
// each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct CacheGeom {
  int num_blocks;
  int num_kv_heads;
  int head_dim;
  int elem_bytes;  // 2 (bf16) or 4 (fp32)
};

hipError_t launch_cache_write(const void* k, const void* v, const int64_t* slots, int num_tokens,
                              void* k_cache, void* v_cache, const CacheGeom& g, hipStream_t stream);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws;  // [S][Hq][P] m, [S][Hq][P] l, [S][Hq][P][D] o (fp32); null if P == 1
  int max_blocks_per_seq;
  int num_seqs;
  int num_q_heads;
  int num_partitions;   // per sequence, grid extent
  int partition_blocks; // blocks per partition
  float scale;
};

// True if (dtype, head_dim, group) has a compiled decode kernel.
bool decode_supported(int elem_bytes, int head_dim, int group);

hipError_t launch_decode(const DecodeArgs& a, const CacheGeom& g, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* query_start_loc;
  const int32_t* context_lens;
  int max_blocks_per_seq;
  int num_reqs;
  int total_q_tokens;
  int max_q_len;
  int num_q_heads;
  float scale;
};

bool prefill_supported(int elem_bytes, int head_dim, int group);

// Query rows one prefill workgroup covers for GQA group size `group`.
int prefill_queries_per_tile(int group);

hipError_t launch_prefill(const PrefillArgs& a, const CacheGeom& g, hipStream_t stream);

// Streaming-read probe over 4 KiB tiles in the given order.
hipError_t launch_bw_probe(const void* buf, size_t bytes, const int32_t* order, int ntiles,
                           uint32_t* sink, hipStream_t stream);

}  // namespace pa
