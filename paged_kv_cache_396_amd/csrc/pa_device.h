// Device-side helpers shared by the gfx950 paged-attention kernels:
// pool addressing, bf16 handling and wave64 cross-lane exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;       // tokens per KV block
constexpr int kWave = 64;        // CDNA wavefront width
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Pool layout.  One (block, kv head) tile is contiguous:
//   K: [16 tokens][D]          (token-major rows)
//   V: [D][16 tokens]          (dim-major rows)
// Both tiles hold 16 * D elements, so the tile base is the same for K and V.
__host__ __device__ constexpr int64_t tile_elems(int D) { return (int64_t)kBlock * D; }

__device__ inline int64_t tile_base(int64_t block, int kv_head, int num_kv_heads, int D) {
  return (block * num_kv_heads + kv_head) * tile_elems(D);
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is the upper half of an fp32, so widening is a shift.
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even pack of two fp32 values (gfx950 v_cvt_pk_bf16_f32).
__device__ inline uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ inline uint16_t to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Two E4M3 codes (the low or the high 16 bits of w) widened to a bf16 pair;
// exact, since every E4M3 value is a bf16 value (scale 1.0 leaves it as is).
template <bool HI>
__device__ inline uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// E4M3 encoding of bf16 values for fp8 pools (code c stands for value(c) *
// scale): the code nearest to x / scale (one correctly rounded fp32
// division), ties to the even code, magnitudes beyond 448 saturating; a NaN
// becomes 0x7F with x's sign bit.
// Four bf16 values (two words, element order lo, hi, lo, hi) -> one word of
// four codes, element i in byte i.
__device__ inline uint32_t quantize4(uint32_t w0, uint32_t w1, float scale) {
  const float x[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = fminf(fmaxf(x[i] / scale, -448.f), 448.f);
  // the conversion rounds to nearest even; the clamp keeps it in range
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], r, true);
  uint32_t keep = 0xffffffffu, nan = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (x[i] != x[i]) {
      keep &= ~(0xffu << (8 * i));
      nan |= (0x7fu | ((__float_as_uint(x[i]) >> 31) << 7)) << (8 * i);
    }
  }
  return ((uint32_t)r & keep) | nan;
}

// a.lo*b.lo + a.hi*b.hi + c with bf16 inputs and fp32 accumulation.
__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------------------
// Cross-lane exchange: returns the value held by lane (lane ^ MASK).
// Masks inside a 16-lane row map to DPP (no LDS traffic); others use
// ds_swizzle (xor within 32 lanes) or ds_bpermute (xor 32).
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <int MASK>
__device__ inline float xor_lane(float v) {
  static_assert(MASK > 0 && MASK < 64, "lane mask");
  if constexpr (MASK == 1) {
    return dpp_f<0xB1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (MASK == 2) {
    return dpp_f<0x4E>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (MASK == 3) {
    return dpp_f<0x1B>(v);  // quad_perm [3,2,1,0]
  } else if constexpr (MASK == 7) {
    return dpp_f<0x141>(v);  // row_half_mirror
  } else if constexpr (MASK == 15) {
    return dpp_f<0x140>(v);  // row_mirror
  } else if constexpr (MASK == 8) {
    return dpp_f<0x128>(v);  // row_ror:8 == xor 8 inside a 16-lane row
  } else if constexpr (MASK < 32) {
    // ds_swizzle bit-mask mode: and_mask 0x1f, or_mask 0, xor_mask MASK
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (MASK << 10)));
  } else {
    const int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ MASK) << 2, __float_as_int(v)));
  }
}

template <int MASK>
__device__ inline float xor_max(float v) { return fmaxf(v, xor_lane<MASK>(v)); }
template <int MASK>
__device__ inline float xor_add(float v) { return v + xor_lane<MASK>(v); }

// Max / sum over every lane whose id differs from ours only in the bits of BITS.
template <int BITS>
__device__ inline float group_max(float v) {
  if constexpr (BITS & 1) v = xor_max<1>(v);
  if constexpr (BITS & 2) v = xor_max<2>(v);
  if constexpr (BITS & 4) v = xor_max<4>(v);
  if constexpr (BITS & 8) v = xor_max<8>(v);
  if constexpr (BITS & 16) v = xor_max<16>(v);
  if constexpr (BITS & 32) v = xor_max<32>(v);
  return v;
}
template <int BITS>
__device__ inline float group_sum(float v) {
  if constexpr (BITS & 1) v = xor_add<1>(v);
  if constexpr (BITS & 2) v = xor_add<2>(v);
  if constexpr (BITS & 4) v = xor_add<4>(v);
  if constexpr (BITS & 8) v = xor_add<8>(v);
  if constexpr (BITS & 16) v = xor_add<16>(v);
  if constexpr (BITS & 32) v = xor_add<32>(v);
  return v;
}

__host__ __device__ constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }
__host__ __device__ constexpr int cmin(int a, int b) { return a < b ? a : b; }
__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }

}  // namespace pa
