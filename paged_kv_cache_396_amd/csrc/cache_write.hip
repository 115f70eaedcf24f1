// Cache write: scatter each new token's K and V rows into its pool slot.
//
// The pages only name slot_mapping ("vLLM: from PagedAttention to Speculative
// Decoding", 3.3); the reading used here is slot = block * 16 + offset, with a
// negative slot marking a padding token that writes nothing.  The copy moves
// raw bits (no conversion), so the result is bit-exact by construction.
//
// Tokens are written by "segments": a segment is a run of tokens whose
// slots are consecutive inside one block.  It starts at a token whose slot
// opens a block or does not continue the previous token's slot, and takes
// the following tokens while their slots continue it, up to the block's
// end.  One workgroup takes the segments that start among 16 consecutive
// input tokens of one kv head (reading up to 15 tokens of the next 16), so
// the tokens of a bulk fill or of a prefill chunk fill each block from one
// workgroup wherever their run starts, and every V store is a whole 16-byte
// chunk of a dim row except at the two ends of a run.  (With groups cut at
// input boundaries instead, a run starting mid-block split every dim row of
// every block between two workgroups, and those partial-sector writes made
// a 70B-layer history fill 1.8x slower than the same fill starting at block
// boundaries.)  Scattered tokens (a decode step's) are segments of one.
//  * K: each owned token's row goes straight to its slot (16-byte stores).
//  * V: the owned rows are staged in LDS by token and written as chunks of
//    the dim-major tile; a chunk only partly inside the segment is written
//    element by element.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kCwThreads = 256;
constexpr int kCwWin = 2 * kBlock;  // input tokens a workgroup may read

// Slots of input tokens i0 - 1 .. i0 + 31 (-1: none, negative or outside the
// pool) and the segments that start at tokens i0 .. i0 + 15.
struct CwSegments {
  int64_t sw[kCwWin + 1];  // slot of input i0 - 1 + t
  int t0[kBlock];          // first token of segment k (window index: input i0 + t0)
  int n[kBlock];           // its length
  int owner[kCwWin];       // segment of window token t, or -1
  int count;
  int multi;  // some segment is longer than one token (its V goes through LDS)
  int tail;   // some segment reaches into tokens i0 + 16 ..
};

__device__ inline void cw_find_segments(CwSegments& sg, const int64_t* slots, int64_t i0,
                                        int num_tokens, int64_t pool_slots) {
  const int tid = threadIdx.x;
  if (tid <= kCwWin) {
    const int64_t idx = i0 - 1 + tid;
    int64_t sv = idx >= 0 && idx < num_tokens ? slots[idx] : -1;
    sg.sw[tid] = sv >= 0 && sv < pool_slots ? sv : -1;
  }
  if (tid < kCwWin) sg.owner[tid] = -1;
  if (tid == 0) {
    sg.count = 0;
    sg.multi = 0;
    sg.tail = 0;
  }
  __syncthreads();
  if (tid < kBlock) {
    const int64_t sv = sg.sw[tid + 1];
    if (sv >= 0 && (sv % kBlock == 0 || sg.sw[tid] != sv - 1)) {
      const int lim = kBlock - (int)(sv % kBlock);
      int len = 1;
      while (len < lim && tid + len < kCwWin && sg.sw[tid + 1 + len] == sv + len) ++len;
      const int k = atomicAdd(&sg.count, 1);  // segment order does not matter
      sg.t0[k] = tid;
      sg.n[k] = len;
      for (int e = 0; e < len; ++e) sg.owner[tid + e] = k;
      if (len > 1) sg.multi = 1;
      if (tid + len > kBlock) sg.tail = 1;
    }
  }
  __syncthreads();
}

// Rows are read in two passes.  The group's own 16 tokens are read at once,
// together with the slots, so a scattered step's tokens wait on one memory
// round trip; the window's next 16 tokens are read after the segments are
// known, and only when a run continues into them.  A token that is a
// segment of its own (a decode step's) writes its V elements straight from
// registers, one element per dim row; longer segments go through LDS.

// One 16-byte chunk x of token t's K and V rows, t owned: K to its slot, V
// into the stage, or (a one-token segment) V element by element.
template <int EB>
__device__ inline void cw_place(const CwSegments& sg, int t, int x, uint4 kr, uint4 vr, int g,
                                int num_kv_heads, int head_dim, uint4* k_cache, char* v_cache,
                                char* vstage, int stage_rb) {
  const int RB = head_dim * EB;
  const int64_t sv = sg.sw[t + 1];
  const int64_t b = sv / kBlock;
  const int o = (int)(sv - b * kBlock);
  const int64_t base = tile_base(b, g, num_kv_heads, head_dim);  // elements
  k_cache[(base * EB + o * RB) / 16 + x] = kr;
  if (sg.n[sg.owner[t]] > 1) {
    *(uint4*)(vstage + t * stage_rb + x * 16) = vr;
    return;
  }
  // V: element (b, g, o, d) at base + d * 16 + o; this chunk holds dims E x ..
  constexpr int E = 16 / EB;
  const uint32_t w[4] = {vr.x, vr.y, vr.z, vr.w};
  if constexpr (EB == 2) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(v_cache) + base + (int64_t)(x * E) * kBlock + o;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e * kBlock] = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
  } else {
    uint32_t* dst = reinterpret_cast<uint32_t*>(v_cache) + base + (int64_t)(x * E) * kBlock + o;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e * kBlock] = w[e];
  }
}

template <int EB>
__global__ __launch_bounds__(kCwThreads) void cache_write_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slots,
    int num_tokens, int num_kv_heads, int head_dim, int64_t pool_slots, uint4* __restrict__ k_cache,
    char* __restrict__ v_cache) {
  __shared__ CwSegments sg;
  // V rows of the window's tokens, token-major, padded by 16 bytes per row
  extern __shared__ __attribute__((aligned(16))) char vstage[];

  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int64_t i0 = (int64_t)blockIdx.x * kBlock;
  const int RC = head_dim * EB / 16;  // 16-byte chunks per row
  const int stage_rb = head_dim * EB + 16;
  const int own = kBlock * RC;        // chunks of one read pass (16 tokens): <= 2 per thread

  // first read pass: chunks tid and tid + 256 of the group's own rows
  const int c0 = tid, c1 = tid + kCwThreads;
  const int t0r = c0 / RC, t1r = c1 / RC;
  const bool h0 = c0 < own && i0 + t0r < num_tokens;
  const bool h1 = EB == 4 && c1 < own && i0 + t1r < num_tokens;
  uint4 k0 = make_uint4(0, 0, 0, 0), v0 = k0, k1 = k0, v1 = k0;
  if (h0) {
    const int64_t row = ((i0 + t0r) * num_kv_heads + g) * RC + (c0 - t0r * RC);
    k0 = k[row];
    v0 = v[row];
  }
  if (h1) {
    const int64_t row = ((i0 + t1r) * num_kv_heads + g) * RC + (c1 - t1r * RC);
    k1 = k[row];
    v1 = v[row];
  }
  cw_find_segments(sg, slots, i0, num_tokens, pool_slots);
  if (sg.count == 0) return;  // uniform

  if (h0 && sg.owner[t0r] >= 0)
    cw_place<EB>(sg, t0r, c0 - t0r * RC, k0, v0, g, num_kv_heads, head_dim, k_cache, v_cache, vstage, stage_rb);
  if (h1 && sg.owner[t1r] >= 0)
    cw_place<EB>(sg, t1r, c1 - t1r * RC, k1, v1, g, num_kv_heads, head_dim, k_cache, v_cache, vstage, stage_rb);
  if (!sg.multi) return;  // uniform: every segment was one token
  // second read pass: tokens i0 + 16 .. that continue a run
  if (sg.tail) {  // uniform
    for (int c = tid; c < own; c += kCwThreads) {
      const int t = kBlock + c / RC, x = c % RC;
      if (sg.owner[t] < 0) continue;
      const int64_t row = ((i0 + t) * num_kv_heads + g) * RC + x;
      cw_place<EB>(sg, t, x, k[row], v[row], g, num_kv_heads, head_dim, k_cache, v_cache, vstage, stage_rb);
    }
  }
  __syncthreads();

  // V of the longer segments: chunk (x, kc) of a tile holds dim x, offsets
  // TPC * kc .. TPC * kc + TPC - 1; a chunk only partly inside the segment
  // is written element by element
  constexpr int TPC = 16 / EB;       // offsets per 16-byte chunk
  constexpr int CPD = kBlock / TPC;  // chunks per dim row
  for (int sgi = 0; sgi < sg.count; ++sgi) {
    const int t0 = sg.t0[sgi], len = sg.n[sgi];
    if (len == 1) continue;  // uniform: written from registers
    const int64_t sv = sg.sw[t0 + 1];
    const int64_t b = sv / kBlock;
    const int o = (int)(sv - b * kBlock);
    const int kc0 = o / TPC, nk = (o + len - 1) / TPC - kc0 + 1;
    char* tile = v_cache + tile_base(b, g, num_kv_heads, head_dim) * EB;
    for (int it = tid; it < head_dim * nk; it += kCwThreads) {
      const int x = it / nk, kc = kc0 + (it - x * nk);
      const int of = kc * TPC;  // offset of the chunk's first element
      // staged element of offset off (o <= off < o + len): token t0 + off - o
      auto elem = [&](int off) -> uint32_t {
        const char* r = vstage + (t0 + off - o) * stage_rb + x * EB;
        if constexpr (EB == 2) return *(const uint16_t*)r;
        else return *(const uint32_t*)r;
      };
      char* dst = tile + (int64_t)(x * CPD + kc) * 16;
      if (of >= o && of + TPC <= o + len) {
        uint32_t w[4];
        if constexpr (EB == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = elem(of + 2 * e) | (elem(of + 2 * e + 1) << 16);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = elem(of + e);
        }
        *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
#pragma unroll
        for (int e = 0; e < TPC; ++e) {
          const int off = of + e;
          if (off < o || off >= o + len) continue;  // another segment's slot: left alone
          if constexpr (EB == 2)
            *(uint16_t*)(dst + e * 2) = (uint16_t)elem(off);
          else
            *(uint32_t*)(dst + e * 4) = elem(off);
        }
      }
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

// The same segments and read passes as the bf16 / fp32 kernel.  Input chunk
// c (8 bf16 of one token) becomes 8 codes.
__global__ __launch_bounds__(kCwThreads) void cache_write_fp8_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slots,
    int num_tokens, int num_kv_heads, int head_dim, int64_t pool_slots, float k_scale,
    float v_scale, char* __restrict__ k_cache, char* __restrict__ v_cache) {
  __shared__ CwSegments sg;
  // V codes of the window's tokens, token-major: byte (t, x) at t * 128 + x
  __shared__ __attribute__((aligned(16))) uint8_t vt[kCwWin * 128];

  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int64_t i0 = (int64_t)blockIdx.x * kBlock;
  const int RC = head_dim / 8;  // 16-byte input chunks per row
  const int own = kBlock * RC;  // <= 256: one chunk per thread per read pass

  // chunk x of token t's rows, t owned: K codes to the slot; V codes into
  // LDS, or (a one-token segment) byte by byte into its 8 dim rows
  auto place = [&](int t, int x, uint4 kr, uint4 vr) {
    const uint2 kq = make_uint2(quantize4(kr.x, kr.y, k_scale), quantize4(kr.z, kr.w, k_scale));
    const uint2 vq = make_uint2(quantize4(vr.x, vr.y, v_scale), quantize4(vr.z, vr.w, v_scale));
    const int64_t sv = sg.sw[t + 1];
    const int64_t b = sv / kBlock;
    const int o = (int)(sv - b * kBlock);
    const int64_t base = tile_base(b, g, num_kv_heads, head_dim);
    *(uint2*)(k_cache + base + o * head_dim + x * 8) = kq;
    if (sg.n[sg.owner[t]] > 1) {
      *(uint2*)(vt + t * 128 + x * 8) = vq;
      return;
    }
    char* dst = v_cache + base + (int64_t)(x * 8) * kBlock + o;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e * kBlock] = (char)(((e < 4 ? vq.x : vq.y) >> (8 * (e & 3))) & 0xffu);
  };

  const int tr = tid / RC;
  const bool have = tid < own && i0 + tr < num_tokens;
  uint4 kr = make_uint4(0, 0, 0, 0), vr = kr;
  if (have) {
    const int64_t row = ((i0 + tr) * num_kv_heads + g) * RC + (tid - tr * RC);
    kr = k[row];
    vr = v[row];
  }
  cw_find_segments(sg, slots, i0, num_tokens, pool_slots);
  if (sg.count == 0) return;  // uniform

  if (have && sg.owner[tr] >= 0) place(tr, tid - tr * RC, kr, vr);
  if (!sg.multi) return;  // uniform
  if (sg.tail && tid < own) {
    const int t = kBlock + tr, x = tid - tr * RC;
    if (sg.owner[t] >= 0) {
      const int64_t row = ((i0 + t) * num_kv_heads + g) * RC + x;
      place(t, x, k[row], v[row]);
    }
  }
  __syncthreads();

  // V of the longer segments: dim row x of a tile is 16 codes (offsets
  // 0 .. 15), one 16-byte chunk
  for (int sgi = 0; sgi < sg.count; ++sgi) {
    const int t0 = sg.t0[sgi], len = sg.n[sgi];
    if (len == 1) continue;  // uniform: written from registers
    const int64_t sv = sg.sw[t0 + 1];
    const int64_t b = sv / kBlock;
    const int o = (int)(sv - b * kBlock);
    char* tile = v_cache + tile_base(b, g, num_kv_heads, head_dim);
    if (len == kBlock) {  // the whole tile
      for (int x = tid; x < head_dim; x += kCwThreads) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)vt[(t0 + 4 * e) * 128 + x] | ((uint32_t)vt[(t0 + 4 * e + 1) * 128 + x] << 8) |
                 ((uint32_t)vt[(t0 + 4 * e + 2) * 128 + x] << 16) |
                 ((uint32_t)vt[(t0 + 4 * e + 3) * 128 + x] << 24);
        *(uint4*)(tile + x * kBlock) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {  // codes at offsets o .. o + len - 1 of every dim row
      for (int it = tid; it < head_dim * len; it += kCwThreads) {
        const int x = it / len, e = it - x * len;
        tile[x * kBlock + o + e] = (char)vt[(t0 + e) * 128 + x];
      }
    }
  }
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
  if (g.head_dim > 128) return hipErrorInvalidValue;
  const size_t lds = (size_t)kCwWin * (g.head_dim * g.elem_bytes + 16);
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
