// Streaming-read probe: reads a buffer of 4 KiB tiles once, in a caller-given
// order, the way paged attention reads its K/V tiles (a block table turns
// logical order into scattered physical tiles).  It measures the read
// bandwidth the device sustains for that pattern, the practical ceiling
// beside the published HBM peak (zihan-zhang.net vLLM study, 1.4: decode is
// bound by the bytes it moves).
//
// One 256-thread workgroup reads kTilesPerGroup tiles, each thread one
// 16-byte piece per tile, four tiles in flight, with non-temporal loads.  The
// data is folded into one word that is written only if it equals a value
// the caller never produces, so the loads cannot be removed.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kProbeTilesPerGroup = 16;
constexpr int kProbeTileChunks = 256;  // 16-byte pieces per 4 KiB tile

__global__ __launch_bounds__(kProbeTileChunks) void bw_probe_kernel(const uint4* __restrict__ buf,
                                                                    const int32_t* __restrict__ order,
                                                                    int ntiles, int nbuf_tiles,
                                                                    uint32_t* sink) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  uint32_t acc = 0;
  const int t0 = blockIdx.x * kProbeTilesPerGroup;
#pragma unroll
  for (int t = 0; t < kProbeTilesPerGroup; t += 4) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = min(t0 + t + u, ntiles - 1);
      int tile = order[i];
      tile = tile < 0 ? 0 : (tile >= nbuf_tiles ? nbuf_tiles - 1 : tile);
      v[u] = __builtin_nontemporal_load(
          (const u32x4*)(buf + (int64_t)tile * kProbeTileChunks + threadIdx.x));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t launch_bw_probe(const void* buf, size_t bytes, const int32_t* order, int ntiles,
                           uint32_t* sink, hipStream_t stream) {
  const int nbuf_tiles = (int)(bytes / (kProbeTileChunks * 16));
  const int grid = (ntiles + kProbeTilesPerGroup - 1) / kProbeTilesPerGroup;
  hipLaunchKernelGGL(bw_probe_kernel, dim3(grid), dim3(kProbeTileChunks), 0, stream,
                     (const uint4*)buf, order, ntiles, nbuf_tiles, sink);
  return hipGetLastError();
}

}  // namespace pa
