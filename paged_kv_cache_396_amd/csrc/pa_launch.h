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
  int elem_bytes;  // of a pool element: 1 (fp8 E4M3), 2 (bf16) or 4 (fp32)
  // fp8 pools only: code c of the K (V) pool stands for value(c) * k_scale
  // (v_scale); q, out and the rows written are bf16
  float k_scale;
  float v_scale;
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
  // > 0: balanced schedule (num_partitions and partition_blocks unused) whose
  // workspace holds 2 * num_ranges * num_q_heads partial slots; the launch
  // uses num_ranges * (resident workgroups per CU) / kBalancedMaxWgPerCu
  // ranges per kv head
  int num_ranges = 0;
  int max_ctx = 0;      // host bound on every context length
  // fused append: row s of new_k / new_v ([num_seqs][Hkv][D], q dtype) is
  // sequence s's newest token, written to slot new_slots[s]; null: none
  const void* new_k = nullptr;
  const void* new_v = nullptr;
  const int64_t* new_slots = nullptr;
};

// Sequences the balanced schedule supports in one call (one workgroup scans
// all their block counts in LDS).
constexpr int kBalancedMaxSeqs = 1024;
// Resident decode workgroups per compute unit of any kernel variant (at
// most), and workgroups per resident slot of the balanced schedule.
constexpr int kBalancedMaxWgPerCu = 4;
#ifndef PA_BALANCED_ROUNDS
#define PA_BALANCED_ROUNDS 1
#endif
constexpr int kBalancedRounds = PA_BALANCED_ROUNDS;

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
  // split-K over the keys (max_parts > 1): parts of part_keys keys (a
  // multiple of 64); ws holds prefill_ws_floats(total_q_tokens *
  // num_q_heads, max_parts, head_dim) floats
  int max_parts = 1;
  int part_keys = 0;
  float* ws = nullptr;
};

// Floats of a split prefill's workspace: m and l of every (row, q head,
// part) slot, then o from a 16-byte boundary.
inline size_t prefill_ws_floats(int64_t rows, int parts, int head_dim) {
  const int64_t slots = rows * parts;
  return (size_t)((2 * slots + 3) / 4 * 4 + slots * head_dim);
}

bool prefill_supported(int elem_bytes, int head_dim, int group);

// Query rows one prefill workgroup covers for GQA group size `group`.
int prefill_queries_per_tile(int group);
// Query rows per tile of the variant a call with this max_q_len launches.
int prefill_tile_queries(int max_q_len, int group);
// True if a call with this max_q_len launches the narrow (4-wave) variant.
bool prefill_narrow(int max_q_len, int group);

hipError_t launch_prefill(const PrefillArgs& a, const CacheGeom& g, hipStream_t stream);

// Shared-prefix decode: pa_decode for groups of group_size consecutive
// sequences whose block tables begin with the same prefix_lens[group] / 16
// blocks.  The prefix kernel reads each shared block once per group and
// leaves partial states; the decode kernel covers each sequence's own blocks;
// the merge combines them.
struct SharedPrefixArgs {
  DecodeArgs d;               // num_partitions / partition_blocks: own blocks
  const int32_t* prefix_lens; // [num_seqs / group_size] tokens, multiples of 16
  int group_size;
  int prefix_partition;       // tokens per prefix partition (multiple of 64)
  int prefix_parts;           // prefix partitions of the longest prefix
  int ws_stride;              // partial slots per row: prefix_parts + d.num_partitions
};

// Floats of the shared-prefix workspace: m and l of every slot, then o,
// starting on a 16-byte boundary.
inline size_t shared_prefix_ws_floats(int64_t rows, int stride, int head_dim) {
  const int64_t ml = (2 * rows * stride + 3) / 4 * 4;
  return (size_t)(ml + rows * stride * head_dim);
}

bool shared_prefix_supported(int elem_bytes, int head_dim, int group, int group_size);
hipError_t launch_prefix_partials(const SharedPrefixArgs& a, const CacheGeom& g, hipStream_t stream);
hipError_t launch_decode_own_and_merge(const SharedPrefixArgs& a, const CacheGeom& g,
                                       hipStream_t stream);

// Copies every kv head's K and V of block pairs[2i] to block pairs[2i+1]
// (device int32 pairs).
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                              const CacheGeom& g, hipStream_t stream);

// Rejection sampling of drafted tokens (speculative decoding).
struct SpecVerifyArgs {
  const float* target_probs;   // [num_reqs][k+1][vocab]
  const float* draft_probs;    // [num_reqs][k][vocab] or null
  const int32_t* draft_tokens; // [num_reqs][k]
  const float* uniforms;       // [num_reqs][k+1]
  int32_t* out_tokens;         // [num_reqs][k+1]
  int32_t* num_out;            // [num_reqs]
  void* workspace;             // spec_verify_workspace_bytes(num_reqs, vocab) bytes
  int num_reqs;
  int k;
  int vocab;
};

size_t spec_verify_workspace_bytes(int num_reqs, int vocab);
hipError_t launch_spec_verify(const SpecVerifyArgs& a, hipStream_t stream);

// Streaming-read probe over 4 KiB tiles in the given order.
hipError_t launch_bw_probe(const void* buf, size_t bytes, const int32_t* order, int ntiles,
                           uint32_t* sink, hipStream_t stream);

}  // namespace pa
