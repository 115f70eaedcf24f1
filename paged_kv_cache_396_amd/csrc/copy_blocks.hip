// Block copy for copy-on-write: before a request writes into a partly
// filled block that other requests still hold, it gets a private copy of
// that block (zihan-zhang.net vLLM study, 3.2.2).  Every kv head's K and V
// of block src are copied to block dst, raw bits.
//
// In both pools a block's tiles of all kv heads are one contiguous run of
// Hkv * 16 * D * eb bytes, so a pair is two flat copies.  One workgroup per
// (pair, pool); 16-byte loads and stores.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(char* __restrict__ k_cache,
                                                                   char* __restrict__ v_cache,
                                                                   const int32_t* __restrict__ pairs,
                                                                   int num_blocks, int64_t block_bytes) {
  const int i = blockIdx.x;
  const int src = pairs[2 * i], dst = pairs[2 * i + 1];
  // ids outside the pool are skipped (the host does not see device values)
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  char* pool = blockIdx.y == 0 ? k_cache : v_cache;
  const uint4* s = (const uint4*)(pool + (int64_t)src * block_bytes);
  uint4* d = (uint4*)(pool + (int64_t)dst * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t c = threadIdx.x; c < n; c += kCopyThreads) d[c] = s[c];
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                              const CacheGeom& g, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t block_bytes = (int64_t)g.num_kv_heads * kBlock * g.head_dim * g.elem_bytes;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs, 2), dim3(kCopyThreads), 0,
                     stream, (char*)k_cache, (char*)v_cache, pairs, g.num_blocks, block_bytes);
  return hipGetLastError();
}

}  // namespace pa
