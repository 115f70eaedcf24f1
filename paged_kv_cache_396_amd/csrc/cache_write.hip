// Cache write: scatter each new token's K and V rows into its pool slot.
//
// The pages only name slot_mapping ("vLLM: from PagedAttention to Speculative
// Decoding", 3.3); the reading used here is slot = block * 16 + offset, with a
// negative slot marking a padding token that writes nothing.  The copy moves
// raw bits (no conversion), so the result is bit-exact by construction.
//
// One thread moves one 16-byte chunk of a (token, kv head) row.  K rows land
// as contiguous 16-byte stores; the V tile is dim-major (16 tokens of one dim
// together), so each V element of the row goes out as its own 2- or 4-byte
// store, 16 elements apart.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

template <int EB>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slots,
    int64_t total_chunks, int chunks_per_row, int num_kv_heads, int head_dim, int64_t pool_slots,
    uint4* __restrict__ k_cache, char* __restrict__ v_cache) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_chunks) return;
  const int64_t row = idx / chunks_per_row;  // token * Hkv + g
  const int chunk = (int)(idx - row * chunks_per_row);
  const int64_t tok = row / num_kv_heads;
  const int g = (int)(row - tok * num_kv_heads);
  // the row loads do not depend on the slot: issue all three together
  const uint4 kv = k[idx];
  const uint4 vv = v[idx];
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= pool_slots) return;
  const int64_t b = slot / kBlock;
  const int o = (int)(slot - b * kBlock);
  const int64_t base = tile_base(b, g, num_kv_heads, head_dim);  // elements

  // K: element (b, g, o, x) at base + o * D + x
  const int64_t kdst = (base + (int64_t)o * head_dim) * EB / 16 + chunk;
  k_cache[kdst] = kv;

  // V: element (b, g, o, x) at base + x * 16 + o
  constexpr int E = 16 / EB;  // elements in this chunk
  const int x0 = chunk * E;
  const int64_t vrow = base + (int64_t)x0 * kBlock + o;
  if constexpr (EB == 2) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(v_cache) + vrow;
    const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t word = w[e >> 1];
      dst[e * kBlock] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
    }
  } else {
    uint32_t* dst = reinterpret_cast<uint32_t*>(v_cache) + vrow;
    const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e * kBlock] = w[e];
  }
}

hipError_t launch_cache_write(const void* k, const void* v, const int64_t* slots, int num_tokens,
                              void* k_cache, void* v_cache, const CacheGeom& g, hipStream_t stream) {
  const int row_bytes = g.head_dim * g.elem_bytes;
  const int cpr = row_bytes / 16;
  const int64_t total = (int64_t)num_tokens * g.num_kv_heads * cpr;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  const int64_t pool_slots = (int64_t)g.num_blocks * kBlock;
  if (g.elem_bytes == 2) {
    hipLaunchKernelGGL(cache_write_kernel<2>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint4*)k, (const uint4*)v, slots, total, cpr, g.num_kv_heads,
                       g.head_dim, pool_slots, (uint4*)k_cache, (char*)v_cache);
  } else {
    hipLaunchKernelGGL(cache_write_kernel<4>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint4*)k, (const uint4*)v, slots, total, cpr, g.num_kv_heads,
                       g.head_dim, pool_slots, (uint4*)k_cache, (char*)v_cache);
  }
  return hipGetLastError();
}

}  // namespace pa
