// Cache write: scatter each new token's K and V rows into its pool slot.
//
// The pages only name slot_mapping ("vLLM: from PagedAttention to Speculative
// Decoding", 3.3); the reading used here is slot = block * 16 + offset, with a
// negative slot marking a padding token that writes nothing.  The copy moves
// raw bits (no conversion), so the result is bit-exact by construction.
//
// One workgroup takes 16 consecutive input tokens of one kv head.
//  * When their slots are consecutive (s0, s0+1, .., s0+15: the tokens of a
//    bulk fill or of a prefill chunk, wherever the run starts in the input
//    and in its block) they fill the tail of block s0 / 16 from offset
//    s0 % 16 and, unless s0 % 16 is 0, the head of the next block.  K rows
//    are written row by row; V, dim-major in the pool, is transposed through
//    LDS and written as 16-byte chunks of dim rows, with the one partial
//    chunk per dim row and block at a run's edge written element by element.
//  * Otherwise (a decode step's scattered tokens, padding, a group holding
//    the end of one run and the start of another) every token is scattered
//    on its own: its K row as 16-byte stores, its V elements one by one, 16
//    elements apart.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kCwThreads = 256;
constexpr int kCwMaxChunks = 2;  // 16 tokens x (D * eb / 16) chunks <= 512 for D <= 128, eb <= 4

template <int EB>
__global__ __launch_bounds__(kCwThreads) void cache_write_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slots,
    int num_tokens, int num_kv_heads, int head_dim, int64_t pool_slots, uint4* __restrict__ k_cache,
    char* __restrict__ v_cache) {
  // row = one token's D values of one kv head; RC 16-byte chunks per row
  __shared__ int64_t sl[kBlock];
  // V rows of the group, token-major, padded by 16 bytes per row
  extern __shared__ __attribute__((aligned(16))) char vstage[];

  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int64_t i0 = (int64_t)blockIdx.x * kBlock;
  const int RB = head_dim * EB;  // bytes of one row
  const int RC = RB / 16;        // 16-byte chunks per row
  const int nch = kBlock * RC;   // chunks of the group
  auto row_of = [&](int64_t tok) { return (tok * num_kv_heads + g) * RC; };  // in 16-byte chunks

  // The rows do not depend on the slots: load them together with the slots,
  // so that the group waits on one memory round trip.
  uint4 kr[kCwMaxChunks], vr[kCwMaxChunks];
#pragma unroll
  for (int u = 0; u < kCwMaxChunks; ++u) {
    const int c = tid + u * kCwThreads;
    const int j = c / RC, x = c - j * RC;
    if (c < nch && i0 + j < num_tokens) {
      kr[u] = k[row_of(i0 + j) + x];
      vr[u] = v[row_of(i0 + j) + x];
    }
  }
  // The group is one run when slot j is s0 + j for all 16 tokens, inside
  // the pool.
  bool in_run = true;
  if (tid < kBlock) {
    const bool real = i0 + tid < num_tokens;
    const int64_t s0 = slots[i0];
    const int64_t mine = real ? slots[i0 + tid] : -1;
    sl[tid] = mine;
    in_run = real && s0 >= 0 && s0 + kBlock <= pool_slots && mine == s0 + tid;
  }
  const bool run = __syncthreads_and(in_run);

  if (run) {
    // token j sits in block b0 at offset o0 + j, or (past the block) in
    // block b0 + 1 at offset o0 + j - 16
    const int64_t b0 = sl[0] / kBlock;
    const int o0 = (int)(sl[0] - b0 * kBlock);
    const int stage_rb = RB + 16;
    auto tile_bytes = [&](int blk) { return tile_base(b0 + blk, g, num_kv_heads, head_dim) * EB; };
#pragma unroll
    for (int u = 0; u < kCwMaxChunks; ++u) {
      const int c = tid + u * kCwThreads;
      if (c < nch) {
        const int j = c / RC, x = c - j * RC;
        const int blk = o0 + j >= kBlock ? 1 : 0;
        const int o = o0 + j - blk * kBlock;
        k_cache[(tile_bytes(blk) + (int64_t)o * RB) / 16 + x] = kr[u];
        *(uint4*)(vstage + j * stage_rb + x * 16) = vr[u];
      }
    }
    __syncthreads();
    // V: chunk c of a tile is dim c / CPD, offsets TPC * (c % CPD) ..; the
    // run covers offsets o0 .. 15 of the first block and 0 .. o0 - 1 of the
    // second
    constexpr int TPC = 16 / EB;       // tokens per 16-byte chunk
    constexpr int CPD = kBlock / TPC;  // chunks per dim row
    const int nblk = o0 > 0 ? 2 : 1;
    for (int c = tid; c < nblk * head_dim * CPD; c += kCwThreads) {
      const int blk = c / (head_dim * CPD);
      const int cc = c - blk * head_dim * CPD;
      const int x = cc / CPD, of = (cc - x * CPD) * TPC;
      const int j0 = of - o0 + blk * kBlock;  // token at offset `of`
      char* dst = v_cache + tile_bytes(blk) + (int64_t)cc * 16;
      auto elem = [&](int j) -> uint32_t {
        if constexpr (EB == 2) return *(const uint16_t*)(vstage + j * stage_rb + x * 2);
        else return *(const uint32_t*)(vstage + j * stage_rb + x * 4);
      };
      if (j0 >= 0 && j0 + TPC <= kBlock) {
        uint32_t w[4];
        if constexpr (EB == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = elem(j0 + 2 * e) | (elem(j0 + 2 * e + 1) << 16);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = elem(j0 + e);
        }
        *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
#pragma unroll
        for (int e = 0; e < TPC; ++e) {
          const int j = j0 + e;
          if (j < 0 || j >= kBlock) continue;  // another run's slot: left alone
          if constexpr (EB == 2)
            *(uint16_t*)(dst + e * 2) = (uint16_t)elem(j);
          else
            *(uint32_t*)(dst + e * 4) = elem(j);
        }
      }
    }
    return;
  }

  // scattered tokens: each token on its own
#pragma unroll
  for (int u = 0; u < kCwMaxChunks; ++u) {
    const int c = tid + u * kCwThreads;
    if (c >= nch) continue;
    const int j = c / RC, chunk = c - j * RC;
    const int64_t slot = sl[j];  // -1 for tokens past the end
    if (slot < 0 || slot >= pool_slots) continue;
    const int64_t b = slot / kBlock;
    const int o = (int)(slot - b * kBlock);
    const int64_t base = tile_base(b, g, num_kv_heads, head_dim);  // elements
    // K: element (b, g, o, x) at base + o * D + x
    k_cache[(base + (int64_t)o * head_dim) * EB / 16 + chunk] = kr[u];
    // V: element (b, g, o, x) at base + x * 16 + o
    constexpr int E = 16 / EB;  // elements in this chunk
    const int64_t vrow = base + (int64_t)(chunk * E) * kBlock + o;
    const uint32_t w[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
    if constexpr (EB == 2) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(v_cache) + vrow;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t word = w[e >> 1];
        dst[e * kBlock] = (uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu));
      }
    } else {
      uint32_t* dst = reinterpret_cast<uint32_t*>(v_cache) + vrow;
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e * kBlock] = w[e];
    }
  }
}

// ---- fp8 (E4M3) pools
//
// An fp8 pool stores one E4M3 code per element (1 sign, 4 exponent bits with
// bias 7, 3 mantissa bits; no infinities, largest magnitude 448) and one fp32
// scale per pool: code c stands for value(c) * scale.  The pages only say
// that an fp8 KV cache doubles capacity and halves attention's bytes
// (zihan-zhang.net vLLM study, 4.2.1); the format, the per-pool scale and
// the rounding below are the readings taken for it.  An incoming bf16 value
// x becomes the E4M3 code nearest to x / scale (one correctly rounded fp32
// division), ties to the even code, magnitudes beyond 448 saturating; a NaN
// becomes 0x7F with x's sign bit (quantize4).

// One workgroup takes 16 consecutive input tokens of one kv head, as the
// bf16/fp32 kernel does, with the same run and scatter paths.  Input chunk c
// (8 bf16 of one token) becomes 8 codes.
__global__ __launch_bounds__(kCwThreads) void cache_write_fp8_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slots,
    int num_tokens, int num_kv_heads, int head_dim, int64_t pool_slots, float k_scale,
    float v_scale, char* __restrict__ k_cache, char* __restrict__ v_cache) {
  __shared__ int64_t sl[kBlock];
  // codes of the V tile, dim-major: byte (x, o) at x * 16 + o
  __shared__ __attribute__((aligned(16))) uint8_t vt[128 * kBlock];

  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int64_t i0 = (int64_t)blockIdx.x * kBlock;
  const int RC = head_dim / 8;   // 16-byte input chunks per row
  const int nch = kBlock * RC;   // <= kCwThreads
  const int j = tid / RC, x = tid - j * RC;
  const bool mine = tid < nch && i0 + j < num_tokens;
  uint2 kq = make_uint2(0, 0), vq = make_uint2(0, 0);
  if (mine) {
    const int64_t row = ((i0 + j) * num_kv_heads + g) * RC + x;
    const uint4 kr = k[row], vr = v[row];
    kq = make_uint2(quantize4(kr.x, kr.y, k_scale), quantize4(kr.z, kr.w, k_scale));
    vq = make_uint2(quantize4(vr.x, vr.y, v_scale), quantize4(vr.z, vr.w, v_scale));
  }
  bool in_run = true;
  if (tid < kBlock) {
    const bool real = i0 + tid < num_tokens;
    const int64_t s0 = slots[i0];
    const int64_t s = real ? slots[i0 + tid] : -1;
    sl[tid] = s;
    in_run = real && s0 >= 0 && s0 + kBlock <= pool_slots && s == s0 + tid;
  }
  const bool run = __syncthreads_and(in_run);
  const uint8_t* vb = (const uint8_t*)&vq;

  if (run) {
    // token j sits in block b0 at offset o0 + j, or in block b0 + 1 at
    // offset o0 + j - 16; vt holds the group's codes by token (x * 16 + j)
    const int64_t b0 = sl[0] / kBlock;
    const int o0 = (int)(sl[0] - b0 * kBlock);
    if (tid < nch) {
      const int blk = o0 + j >= kBlock ? 1 : 0;
      const int64_t base = tile_base(b0 + blk, g, num_kv_heads, head_dim);  // bytes
      *(uint2*)(k_cache + base + (o0 + j - blk * kBlock) * head_dim + x * 8) = kq;
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(x * 8 + e) * kBlock + j] = vb[e];
    }
    __syncthreads();
    if (o0 == 0) {
      const int64_t base = tile_base(b0, g, num_kv_heads, head_dim);
      if (tid < head_dim) *(uint4*)(v_cache + base + tid * kBlock) = *(const uint4*)&vt[tid * kBlock];
      return;
    }
    // dim row x of the first block takes offsets o0 .. 15 (tokens 0 ..),
    // of the second offsets 0 .. o0 - 1 (tokens 16 - o0 ..): byte stores,
    // neighbouring threads on neighbouring bytes
    for (int c = tid; c < 2 * head_dim * kBlock; c += kCwThreads) {
      const int blk = c / (head_dim * kBlock);
      const int cc = c - blk * head_dim * kBlock;
      const int xx = cc / kBlock, o = cc - xx * kBlock;
      const int jj = blk == 0 ? o - o0 : o + kBlock - o0;
      if (jj < 0 || jj >= kBlock) continue;  // another run's slot: left alone
      const int64_t base = tile_base(b0 + blk, g, num_kv_heads, head_dim);
      v_cache[base + xx * kBlock + o] = (char)vt[xx * kBlock + jj];
    }
    return;
  }

  // scattered tokens: each token on its own
  if (!mine) return;
  const int64_t slot = sl[j];
  if (slot < 0 || slot >= pool_slots) return;
  const int64_t b = slot / kBlock;
  const int o = (int)(slot - b * kBlock);
  const int64_t base = tile_base(b, g, num_kv_heads, head_dim);
  *(uint2*)(k_cache + base + o * head_dim + x * 8) = kq;
#pragma unroll
  for (int e = 0; e < 8; ++e) v_cache[base + (x * 8 + e) * kBlock + o] = (char)vb[e];
}

hipError_t launch_cache_write(const void* k, const void* v, const int64_t* slots, int num_tokens,
                              void* k_cache, void* v_cache, const CacheGeom& g, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t groups = ((int64_t)num_tokens + kBlock - 1) / kBlock;
  if (groups >= ((int64_t)1 << 31) || g.num_kv_heads > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)groups, (unsigned)g.num_kv_heads);
  if (g.elem_bytes == 1) {
    // bf16 input rows: 16 tokens x D / 8 chunks, one per thread
    if (g.head_dim % 8 != 0 || g.head_dim > 128) return hipErrorInvalidValue;
    hipLaunchKernelGGL(cache_write_fp8_kernel, grid, dim3(kCwThreads), 0, stream, (const uint4*)k,
                       (const uint4*)v, slots, num_tokens, g.num_kv_heads, g.head_dim,
                       (int64_t)g.num_blocks * kBlock, g.k_scale, g.v_scale, (char*)k_cache,
                       (char*)v_cache);
    return hipGetLastError();
  }
  if ((int64_t)kBlock * g.head_dim * g.elem_bytes / 16 > (int64_t)kCwMaxChunks * kCwThreads)
    return hipErrorInvalidValue;
  const size_t lds = (size_t)kBlock * (g.head_dim * g.elem_bytes + 16);
  const int64_t pool_slots = (int64_t)g.num_blocks * kBlock;
  if (g.elem_bytes == 2) {
    hipLaunchKernelGGL(cache_write_kernel<2>, grid, dim3(kCwThreads), lds, stream,
                       (const uint4*)k, (const uint4*)v, slots, num_tokens, g.num_kv_heads,
                       g.head_dim, pool_slots, (uint4*)k_cache, (char*)v_cache);
  } else {
    hipLaunchKernelGGL(cache_write_kernel<4>, grid, dim3(kCwThreads), lds, stream,
                       (const uint4*)k, (const uint4*)v, slots, num_tokens, g.num_kv_heads,
                       g.head_dim, pool_slots, (uint4*)k_cache, (char*)v_cache);
  }
  return hipGetLastError();
}

}  // namespace pa
