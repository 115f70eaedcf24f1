// Paged decode attention for gfx950 (one query token per sequence).
//
// What is computed: for every sequence s and query head h,
//   out[s,h] = softmax(scale * K_s q_{s,h}) V_s
// over the sequence's ctx_s cached tokens, where K_s/V_s are read block by
// block through the block table (zihan-zhang.net vLLM study, 3.2: per block,
// look up the physical block, score its 16 keys, then weight its 16 values;
// 1.1.1 for the attention formula) and the softmax is evaluated online
// (same page, 4.3.1: keep a running max m and sum l, rescale the running
// output by exp(m_old - m_new) when m grows, divide by l at the end).
//
// Mapping onto CDNA4:
//  * one workgroup (4 waves) per (sequence, kv head, partition); a partition
//    is a run of consecutive 16-token blocks.  The G = Hq/Hkv query heads of
//    the kv head share every K/V byte read (GQA).
//  * wave w takes blocks w, w+4, ... of the partition.  A (block, kv head)
//    tile of K is one contiguous 16*D run; each load instruction reads whole
//    128-byte lines.  The next block's K and V are loaded into registers
//    before the current block is computed.
//  * Q.K: a K row is spread over LPR lanes; every lane forms partial dots for
//    its rows and all G heads (bf16 dot2, fp32 accumulate), then a
//    reduce-scatter over the LPR lanes (DPP mirrors and quad permutes) leaves
//    each lane with complete scores for one head and one or two tokens.
//  * softmax: scores are kept in the log2 domain.  The running max is only
//    raised when some score exceeds it by more than 2^8, which after the first
//    block is rare; the rescale is exact whenever it happens, so the result
//    is the same softmax (the reference max only has to be common to all
//    terms that are summed together).
//  * P.V: V tiles are dim-major, so a lane's 16-byte V chunk holds 8 (bf16)
//    or 4 (fp32) consecutive tokens of one dim.  Probabilities go through LDS
//    as bf16 pairs of consecutive tokens; each lane does bf16 dot2 over token
//    pairs for its dims and all G heads, accumulating fp32, and the lanes
//    that hold the other tokens of the same dims are summed at the end.
//  * the 4 waves merge their (m, l, O) in LDS with the same rescale.  With
//    one partition the workgroup writes the output; otherwise it writes its
//    partial state and decode_reduce merges the partitions (a merge done by
//    the last partition to finish, found with an arrival counter, measured
//    slower: publishing partial states across XCDs takes an agent-scope
//    release, which writes back the whole L2 of the XCD).

#include <float.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif
constexpr int kDecodeWaves = PA_DECODE_WAVES;      // waves per workgroup

constexpr float kRescaleGap = 8.0f;   // log2 units: p may reach 2^8 before a rescale
constexpr float kNegBig = -FLT_MAX;   // "no score yet"; keeps exp2 of differences finite

// Raw buffer descriptor over [ptr, ptr + bytes): loads beyond `bytes` return 0.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const char* ptr, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)ptr, (short)0, bytes, 0x00020000);
}

// 16-byte KV load at byte offset `off`.  KV is streamed once per call, so the
// load is marked non-temporal (cache policy bit nt).
__device__ inline uint4 load16(__amdgpu_buffer_rsrc_t r, int off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, PA_DECODE_NT ? 2 : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int EB, int D, int G>
struct DecodeCfg {
  static constexpr int RB = D * EB;                  // bytes of one K row
  static constexpr int QB = EB == 4 ? 4 : 2;         // bytes of a q / out element (bf16 for fp8 pools)
  static constexpr int QRB = D * QB;                 // bytes of one q row
  static constexpr int LPR = RB >= 256 ? 16 : 8;     // lanes per K row
  static constexpr int U = RB / 16 / LPR;            // 16-byte chunks per lane per row
  static constexpr int NR = LPR / 4;                 // K rows per lane per tile
  static constexpr int EPC = 16 / EB;                // elements per 16-byte chunk
  static constexpr int QCH = EPC * QB / 16;          // 16-byte q chunks per K chunk
  static constexpr int N0 = NR * G;                  // partial dots per lane
  static constexpr int LOGL = ilog2(LPR);
  static constexpr int HALV = cmin(LOGL, ilog2(N0)); // halving steps of the reduce-scatter
  static constexpr int AR = LOGL - HALV;             // trailing all-reduce steps
  static constexpr int NF = N0 >> HALV;              // complete scores per lane
  static constexpr int HEAD_SPAN = NR / NF;          // lanes (after AR) sharing one head
  static constexpr int HEAD_BITS = (HEAD_SPAN - 1) << AR;
  static constexpr int DUP_BITS = (1 << AR) - 1;     // lanes holding identical scores
  static constexpr int ROW_BITS = (kWave - 1) & ~(LPR - 1);
  // V: D dim-rows of 16 tokens per tile; chunk i of lane l is chunk
  // l + 64 i of the tile: dim (l + 64 i) / VCPR, tokens VTPC * (l % VCPR) ..
  static constexpr int VTPC = 16 / EB;               // tokens per V chunk
  static constexpr int VCPR = kBlock / VTPC;         // chunks per dim-row (= EB)
  static constexpr int NV = D * VCPR / kWave;        // V chunks (dims) per lane
  static constexpr int VPART_BITS = VCPR - 1;        // lanes holding other tokens of our dims
  static constexpr int PWORDS = EB == 4 ? 2 : 1;     // 32-bit words per (pair, head) of P
  static_assert(NF <= 2 && NF <= NR, "unsupported GQA group for this head size");
  static_assert(NV >= 1 && D * VCPR % kWave == 0, "V chunk mapping");
  static_assert(U >= 1, "K row shorter than one chunk per lane");
};

struct DecodeParams {
  void* out;
  const void* q;
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int max_blocks_per_seq;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int num_blocks;
  int num_partitions;
  int partition_blocks;
  float scale_log2;
  float v_scale;  // fp8 pools: applied with the final normalisation
  // shared-prefix decode only: the partial states of (seq, q head) row r sit
  // in slots r * ws_stride + (0 .. npre-1) (the prefix partitions, written by
  // the prefix kernel) and npre + part (the sequence's own blocks)
  const int32_t* prefix_lens;  // shared tokens of each group (multiple of 16)
  int group_size;              // sequences per group
  int prefix_partition;        // tokens per prefix partition
  int max_prefix;              // prefix tokens the prefix kernel covers at most
  int ws_stride;               // partial slots per row
  // balanced schedule only
  int num_ranges;              // ranges per kv head the grid offers
  int max_ctx;                 // host bound on every context length
  // fused append (pa_decode_append) only: row s of new_k / new_v (q dtype,
  // [num_seqs][num_kv_heads][D]) is sequence s's newest token, written to
  // pool slot new_slots[s]; null when the call appends nothing
  const char* new_k;
  const char* new_v;
  const int64_t* new_slots;
  float k_quant_scale;         // fp8 pools: the pools' scales for encoding
  float v_quant_scale;
};

// Shared tokens of sequence s's group, clamped to its context and rounded
// down to whole blocks.
__device__ inline int prefix_of(const DecodeParams& p, int s, int ctx) {
  const int cap = ctx < p.max_prefix ? ctx : p.max_prefix;
  const int pl = p.prefix_lens[s / p.group_size];
  return (pl < 0 ? 0 : (pl > cap ? cap : pl)) & ~(kBlock - 1);
}
__device__ inline int prefix_parts(const DecodeParams& p, int pl) {
  return (pl + p.prefix_partition - 1) / p.prefix_partition;
}

// Context length actually processed: bounded by the table row and the grid.
__device__ inline int clamp_ctx(int ctx, const DecodeParams& p) {
  long cap = (long)p.max_blocks_per_seq * kBlock;
  const long grid_cap = (long)p.num_partitions * p.partition_blocks * kBlock;
  if (grid_cap < cap) cap = grid_cap;
  if (ctx < 0) ctx = 0;
  return ctx > cap ? (int)cap : ctx;
}

// Reduce-scatter of L partial dots over the LPR lanes of a K row.  Step k
// pairs lanes through a mask whose highest set bit is (LPR >> (k+1)); the
// lane with that bit set keeps the upper half of the values.  After log2 L
// halvings (capped at log2 LPR) the lane with row index c holds the complete
// sums for values c*NF .. c*NF+NF-1; any remaining steps sum over the low
// lane bits (those lanes then hold identical values).
template <int LPR, int L>
__device__ inline void reduce_scatter_lpr(float (&v)[L], int c) {
  constexpr int LOGL = ilog2(LPR);
  constexpr int HALV = cmin(LOGL, ilog2(L));
  // masks per step for a 16-lane row: 15 (row_mirror), 7 (half mirror), 2, 1;
  // for an 8-lane row: 7, 2, 1.
  auto step = [&](auto kconst) {
    constexpr int k = decltype(kconst)::value;
    constexpr int bit = LPR >> (k + 1);
    constexpr int mask = (LPR == 16) ? (k == 0 ? 15 : k == 1 ? 7 : k == 2 ? 2 : 1)
                                     : (k == 0 ? 7 : k == 1 ? 2 : 1);
    if constexpr (k < HALV) {
      constexpr int n = L >> k;
      const bool upper = (c & bit) != 0;
#pragma unroll
      for (int i = 0; i < n / 2; ++i) {
        const float a = v[i];
        const float b = v[i + n / 2];
        const float keep = upper ? b : a;
        const float send = upper ? a : b;
        v[i] = keep + xor_lane<mask>(send);
      }
    } else {
      v[0] = v[0] + xor_lane<mask>(v[0]);
    }
  };
  step(std::integral_constant<int, 0>{});
  step(std::integral_constant<int, 1>{});
  step(std::integral_constant<int, 2>{});
  if constexpr (LOGL == 4) step(std::integral_constant<int, 3>{});
}


// Per-wave decode state and the arithmetic of one (block, kv head) tile,
// shared by both decode kernels.  Lane geometry: a K row is spread over LPR
// lanes (c = lane within the row, r = row group); V chunk i of the lane is
// chunk lane + 64 i of the tile.
template <int EB, int D, int G>
struct WaveDecoder {
  using C = DecodeCfg<EB, D, G>;
  int lane, c, r, vpart, vdim0;
  int hh, tk0;  // this lane's scores: head hh, tokens tk0 (+1 if NF == 2)
  float scale_log2;
  uint32_t* pb;  // this wave's probability exchange buffer in LDS
  uint4 qv[G][C::U * C::QCH];
  float o[G][C::NV];
  float m_mine;  // reference max (log2 units) of this lane's head
  float l_mine;  // sum of this lane's probabilities

  __device__ void init(uint32_t* pbuf_wave, float sl2) {
    lane = threadIdx.x & (kWave - 1);
    c = lane & (C::LPR - 1);
    r = lane / C::LPR;
    vpart = lane & C::VPART_BITS;
    vdim0 = lane / C::VCPR;
    const int j0 = (c >> C::AR) * C::NF;
    hh = j0 / C::NR;
    tk0 = r * C::NR + (j0 % C::NR);
    scale_log2 = sl2;
    pb = pbuf_wave;
  }

  __device__ void reset() {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int x = 0; x < C::NV; ++x) o[h][x] = 0.f;
    m_mine = kNegBig;
    l_mine = 0.f;
  }

  // q chunks of the G heads of one kv head; qbase points at its first head's
  // row.  K chunk u of the lane holds elements (u * LPR + c) * EPC + 0..EPC-1;
  // the matching q elements are QCH 16-byte chunks.
  __device__ void load_q(const char* qbase, uint4 (&dst)[G][C::U * C::QCH]) const {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int u = 0; u < C::U; ++u)
#pragma unroll
        for (int j = 0; j < C::QCH; ++j)
          dst[h][u * C::QCH + j] = *(const uint4*)(qbase + (int64_t)h * C::QRB +
                                                   ((u * C::LPR + c) * C::QCH + j) * 16);
  }

  // One (block, kv head) tile through buffer descriptors of nrec bytes: a
  // tile that must not be read gets nrec = 0, its loads return zeros without
  // touching memory but still retire in order (static wait counts).
  __device__ void load_tile(const char* kp, const char* vp, int nrec, uint4 (&kk)[C::NR][C::U],
                            uint4 (&vv)[C::NV]) const {
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kp, nrec);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vp, nrec);
#pragma unroll
    for (int i = 0; i < C::NR; ++i)
#pragma unroll
      for (int u = 0; u < C::U; ++u)
        kk[i][u] = load16(kr, (r * C::NR + i) * C::RB + (u * C::LPR + c) * 16);
#pragma unroll
    for (int i = 0; i < C::NV; ++i) vv[i] = load16(vr, (lane + kWave * i) * 16);
  }

  // Scores, online-softmax update and P.V for one tile whose first `nvalid`
  // tokens belong to the context (0 for a tile that must be skipped).
  __device__ void process(uint4 (&kc)[C::NR][C::U], uint4 (&vc)[C::NV], int nvalid) {
    // ---- partial dots
    float acc[C::N0];
    if constexpr (EB == 1) {
      // every code widens exactly to bf16: word w of a chunk gives the bf16
      // pairs of elements 4w, 4w+1 and 4w+2, 4w+3
      uint32_t kw[C::NR][C::U][8];
#pragma unroll
      for (int i = 0; i < C::NR; ++i)
#pragma unroll
        for (int u = 0; u < C::U; ++u) {
          const uint32_t w4[4] = {kc[i][u].x, kc[i][u].y, kc[i][u].z, kc[i][u].w};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            kw[i][u][2 * w] = fp8x2_to_bf16x2<false>(w4[w]);
            kw[i][u][2 * w + 1] = fp8x2_to_bf16x2<true>(w4[w]);
          }
        }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < C::NR; ++i) {
          float a = 0.f;
#pragma unroll
          for (int u = 0; u < C::U; ++u)
#pragma unroll
            for (int pr = 0; pr < 8; ++pr)
              a = dot2_bf16(((const uint32_t*)&qv[h][u * 2 + (pr >> 2)])[pr & 3], kw[i][u][pr], a);
          acc[h * C::NR + i] = a;
        }
    } else
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < C::NR; ++i) {
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < C::U; ++u) {
          const uint4 kk = kc[i][u];
          const uint4 qq = qv[h][u];
          if constexpr (EB == 2) {
            a = dot2_bf16(qq.x, kk.x, a);
            a = dot2_bf16(qq.y, kk.y, a);
            a = dot2_bf16(qq.z, kk.z, a);
            a = dot2_bf16(qq.w, kk.w, a);
          } else {
            a = fmaf(__uint_as_float(qq.x), __uint_as_float(kk.x), a);
            a = fmaf(__uint_as_float(qq.y), __uint_as_float(kk.y), a);
            a = fmaf(__uint_as_float(qq.z), __uint_as_float(kk.z), a);
            a = fmaf(__uint_as_float(qq.w), __uint_as_float(kk.w), a);
          }
        }
        acc[h * C::NR + i] = a;
      }
    reduce_scatter_lpr<C::LPR, C::N0>(acc, c);

    // ---- scores (log2 units), masking tokens past the context
    float z[C::NF];
#pragma unroll
    for (int k = 0; k < C::NF; ++k) {
      z[k] = acc[k] * scale_log2;
      if (nvalid < kBlock) z[k] = (tk0 + k < nvalid) ? z[k] : -INFINITY;
    }
    if (nvalid < kBlock) {
      // zero V of hidden tokens: a zero probability must not meet a NaN
      uint32_t keep[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (EB == 1) {
          uint32_t m = 0;  // bytes 0..3 hold tokens 4e..4e+3
#pragma unroll
          for (int b = 0; b < 4; ++b) m |= (4 * e + b < nvalid ? 0xffu : 0u) << (8 * b);
          keep[e] = m;
        } else if constexpr (EB == 2) {
          const int t0 = vpart * C::VTPC + 2 * e;
          keep[e] = t0 >= nvalid ? 0u : (t0 + 1 >= nvalid ? 0x0000ffffu : 0xffffffffu);
        } else {
          keep[e] = vpart * C::VTPC + e >= nvalid ? 0u : 0xffffffffu;
        }
      }
#pragma unroll
      for (int i = 0; i < C::NV; ++i) {
        uint32_t* wv = (uint32_t*)&vc[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[e] &= keep[e];
      }
    }

    // ---- online softmax: raise the reference max only when needed
    bool over = false;
#pragma unroll
    for (int k = 0; k < C::NF; ++k) over |= z[k] > m_mine + kRescaleGap;
    if (__builtin_amdgcn_ballot_w64(over)) {
      float bm = z[0];
#pragma unroll
      for (int k = 1; k < C::NF; ++k) bm = fmaxf(bm, z[k]);
      bm = group_max<C::HEAD_BITS | C::ROW_BITS>(bm);
      const float m_new = fmaxf(m_mine, bm);
      const float alpha = exp2f(m_mine - m_new);
      l_mine *= alpha;
      m_mine = m_new;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ah = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), head_lane(h)));
#pragma unroll
        for (int x = 0; x < C::NV; ++x) o[h][x] *= ah;
      }
    }
    float pr[C::NF];
#pragma unroll
    for (int k = 0; k < C::NF; ++k) pr[k] = exp2f(z[k] - m_mine);

    // ---- probabilities -> LDS as [pair][head] (bf16 pairs or fp32 pairs).
    // With bf16 P the running sum adds the rounded weights, the same ones
    // P.V applies, so the output is a convex combination of V rows.
    if constexpr (EB <= 2) {
      if constexpr (C::NF == 2) {
        const uint32_t pw = pack_bf16(pr[0], pr[1]);
        l_mine += bf16_lo(pw) + bf16_hi(pw);
        pb[(tk0 >> 1) * G + hh] = pw;
      } else {
        const uint16_t pw = to_bf16(pr[0]);
        l_mine += bf16_lo(pw);
        if ((c & C::DUP_BITS) == 0)
          ((uint16_t*)pb)[((tk0 >> 1) * G + hh) * 2 + (tk0 & 1)] = pw;
      }
    } else {
#pragma unroll
      for (int k = 0; k < C::NF; ++k) l_mine += pr[k];
      if ((c & C::DUP_BITS) == 0) {
#pragma unroll
        for (int k = 0; k < C::NF; ++k) {
          const int t = tk0 + k;
          ((float*)pb)[((t >> 1) * G + hh) * 2 + (t & 1)] = pr[k];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- P.V: word e of a V chunk holds tokens 2e, 2e+1 of the chunk (bf16)
    // or token e (fp32)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (EB == 1) {
        // word e of a V chunk holds the codes of tokens 4e..4e+3 (one dim)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int tp = 2 * e + half;  // token pair within the block
          uint32_t pw[G];
          if constexpr (G % 4 == 0) {
#pragma unroll
            for (int h4 = 0; h4 < G / 4; ++h4) {
              const uint4 t4 = *(const uint4*)&pb[tp * G + h4 * 4];
              pw[h4 * 4 + 0] = t4.x; pw[h4 * 4 + 1] = t4.y;
              pw[h4 * 4 + 2] = t4.z; pw[h4 * 4 + 3] = t4.w;
            }
          } else {
#pragma unroll
            for (int h = 0; h < G; ++h) pw[h] = pb[tp * G + h];
          }
#pragma unroll
          for (int i = 0; i < C::NV; ++i) {
            const uint32_t raw = ((const uint32_t*)&vc[i])[e];
            const uint32_t wv = half ? fp8x2_to_bf16x2<true>(raw) : fp8x2_to_bf16x2<false>(raw);
#pragma unroll
            for (int h = 0; h < G; ++h) o[h][i] = dot2_bf16(pw[h], wv, o[h][i]);
          }
        }
      } else if constexpr (EB == 2) {
        const int tp = vpart * (C::VTPC / 2) + e;  // token pair within the block
        uint32_t pw[G];
        if constexpr (G % 4 == 0) {
#pragma unroll
          for (int h4 = 0; h4 < G / 4; ++h4) {
            const uint4 t4 = *(const uint4*)&pb[tp * G + h4 * 4];
            pw[h4 * 4 + 0] = t4.x; pw[h4 * 4 + 1] = t4.y;
            pw[h4 * 4 + 2] = t4.z; pw[h4 * 4 + 3] = t4.w;
          }
        } else {
#pragma unroll
          for (int h = 0; h < G; ++h) pw[h] = pb[tp * G + h];
        }
#pragma unroll
        for (int i = 0; i < C::NV; ++i) {
          const uint32_t wv = ((const uint32_t*)&vc[i])[e];
#pragma unroll
          for (int h = 0; h < G; ++h) o[h][i] = dot2_bf16(pw[h], wv, o[h][i]);
        }
      } else {
        const int t = vpart * C::VTPC + e;  // token within the block
        float pp[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pp[h] = ((const float*)pb)[((t >> 1) * G + h) * 2 + (t & 1)];
#pragma unroll
        for (int i = 0; i < C::NV; ++i) {
          const float vf = __uint_as_float(((const uint32_t*)&vc[i])[e]);
#pragma unroll
          for (int h = 0; h < G; ++h) o[h][i] = fmaf(pp[h], vf, o[h][i]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // Wave totals: afterwards lanes with vpart == 0 hold the complete o[h][x]
  // for dims vdim0 + (64 / VCPR) x, and lane head_lane(h) holds head h's
  // reference max (m_mine) and returned sum.
  __device__ float totals() {
    float l_head = (c & C::DUP_BITS) == 0 ? l_mine : 0.f;
    l_head = group_sum<C::HEAD_BITS | C::DUP_BITS | C::ROW_BITS>(l_head);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int x = 0; x < C::NV; ++x) o[h][x] = group_sum<C::VPART_BITS>(o[h][x]);
    return l_head;
  }

  static __device__ constexpr int head_lane(int h) { return (h * C::HEAD_SPAN) << C::AR; }
  __device__ int dim_of(int x) const { return vdim0 + (kWave / C::VCPR) * x; }

  // ---- fused append: one new token's K and V rows in the register layout
  // of a tile (knew[u]: K chunk u of the lane; vnew[i]: the element of the
  // dim of V chunk i), encoded as the pool stores them.
  __device__ void load_new_row(const char* krow, const char* vrow, float ksc, float vsc,
                               uint4 (&knew)[C::U], uint32_t (&vnew)[C::NV]) const {
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      const int ch = u * C::LPR + c;  // 16-byte chunk of the pool row
      if constexpr (EB == 1) {
        // 16 codes from 16 bf16 inputs
        const uint4 a = *(const uint4*)(krow + ch * 32);
        const uint4 b = *(const uint4*)(krow + ch * 32 + 16);
        knew[u] = make_uint4(quantize4(a.x, a.y, ksc), quantize4(a.z, a.w, ksc),
                             quantize4(b.x, b.y, ksc), quantize4(b.z, b.w, ksc));
      } else {
        knew[u] = *(const uint4*)(krow + ch * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < C::NV; ++i) {
      const int dim = (lane + kWave * i) / C::VCPR;
      if constexpr (EB == 1)
        vnew[i] = quantize4(*(const uint16_t*)(vrow + dim * 2), 0u, vsc) & 0xffu;
      else if constexpr (EB == 2)
        vnew[i] = *(const uint16_t*)(vrow + dim * 2);
      else
        vnew[i] = *(const uint32_t*)(vrow + dim * 4);
    }
  }

  // Keeps the new row in this wave's LDS stash: K chunks in pool order, one
  // V element (low bits of a word) per dim.
  __device__ void stash_new_row(uint4* sk, uint32_t* sv, const uint4 (&knew)[C::U],
                                const uint32_t (&vnew)[C::NV]) const {
    if (r == 0) {
#pragma unroll
      for (int u = 0; u < C::U; ++u) sk[u * C::LPR + c] = knew[u];
    }
    if (vpart == 0) {
#pragma unroll
      for (int i = 0; i < C::NV; ++i) sv[(lane + kWave * i) / C::VCPR] = vnew[i];
    }
  }

  // A tile whose token 0 is the stashed row (the other tokens are zeros and
  // are masked by the caller's nvalid = 1).
  __device__ void stashed_tile(const uint4* sk, const uint32_t* sv, uint4 (&kt)[C::NR][C::U],
                               uint4 (&vt)[C::NV]) const {
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < C::NR; ++i)
#pragma unroll
      for (int u = 0; u < C::U; ++u) kt[i][u] = (r == 0 && i == 0) ? sk[u * C::LPR + c] : z;
#pragma unroll
    for (int i = 0; i < C::NV; ++i)
      vt[i] = vpart == 0 ? make_uint4(sv[(lane + kWave * i) / C::VCPR], 0, 0, 0) : z;
  }
};

// Occupancy target (waves per SIMD) the register allocator must meet.
#ifndef PA_DECODE_OCC_BF16_G4
#define PA_DECODE_OCC_BF16_G4 3
#endif
#ifndef PA_DECODE_OCC_FP8_G4
#define PA_DECODE_OCC_FP8_G4 3
#endif
template <int EB, int D, int G>
constexpr int decode_waves_per_eu() {
  return (EB == 1) ? (G <= 4 ? PA_DECODE_OCC_FP8_G4 : 2)
         : (EB == 2 && G <= 4) ? PA_DECODE_OCC_BF16_G4
         : (EB == 4 && D == 64 && G <= 2) ? 3 : (EB == 4 && D == 128 && G >= 4) ? 1 : 2;
}

// Register tile slots per wave (one computed, the others in flight).  A
// third slot for the half-size fp8 tiles measured the same as two.
#ifndef PA_DECODE_SLOTS_FP8
#define PA_DECODE_SLOTS_FP8 2
#endif
#ifndef PA_DECODE_SLOTS_BF16
#define PA_DECODE_SLOTS_BF16 2
#endif
template <int EB>
constexpr int decode_slots() {
  return EB == 1 ? PA_DECODE_SLOTS_FP8 : EB == 2 ? PA_DECODE_SLOTS_BF16 : 2;
}

// LDS of one decode workgroup: the waves' probability exchange buffers and
// their (m, l, O) for the final merge.
template <int EB, int D, int G>
struct DecodeLds {
  using C = DecodeCfg<EB, D, G>;
  __attribute__((aligned(16))) uint32_t pbuf[kDecodeWaves][8 * G * C::PWORDS];
  float sm[kDecodeWaves][G];
  float sl[kDecodeWaves][G];
  __attribute__((aligned(16))) float so[kDecodeWaves][G][D];
  // fused append: each wave's copy of the newest token's K row (pool
  // encoding) and V elements
  uint4 newk[kDecodeWaves][C::RB / 16];
  uint32_t newv[kDecodeWaves][D];
};

// Streams blocks [b0, b1) of one sequence (ctx tokens, block table row bt)
// for kv head g through wave w's register tile ring: the wave takes blocks
// b0 + w, b0 + w + NW, ...  On entry my_ids holds, one per lane, the ids of
// blocks b0 + w + NW * lane (or anything for blocks at or past b1), fetched
// by the caller so that the fetch overlaps its other loads.
// Fused append: when `s` is not negative, b1 is the sequence's last block
// and row s of the new rows is its newest token, at position ctx - 1.  The
// wave that takes that block loads the token's rows with its first block
// ids and keeps a copy in LDS (a later kernel of the call writes them to
// the pool: a store here would hold up this wave's later tile waits until
// it is acknowledged, behind the whole read stream).  If the slot
// is row tn = (ctx - 1) % 16 of that block (the case the contract asks
// for), the block is scored without its pool row tn, and after the last
// block the token is scored from the LDS copy as a one-token tile: the same
// set of tokens as a decode over the written pool, with no read of the
// written row in this launch.
template <int EB, int D, int G>
__device__ inline void stream_blocks(WaveDecoder<EB, D, G>& wd, DecodeLds<EB, D, G>& lds,
                                     const DecodeParams& p, const int32_t* bt, int g, int w,
                                     int b0, int b1, int ctx, int my_ids, int s = -1) {
  using C = DecodeCfg<EB, D, G>;
  constexpr int NW = kDecodeWaves;
  const int lane = wd.lane;
  const int64_t tile_bytes = (int64_t)kBlock * C::RB;

  const bool app = s >= 0 && w == (b1 - 1 - b0) % NW;  // uniform
  const int tn = (ctx - 1) & (kBlock - 1);
  int64_t slot = -1, slot_in = -1;
  bool hit = false;  // the last block was scored without its row tn
  uint4 knew[C::U];
  uint32_t vnew[C::NV];
  if (app) {
    const int64_t row = ((int64_t)s * p.num_kv_heads + g) * C::QRB;
    slot_in = p.new_slots[s];
    wd.load_new_row(p.new_k + row, p.new_v + row, p.k_quant_scale, p.v_quant_scale, knew, vnew);
  }
  // block ids of this wave's blocks, one per lane, refreshed every 64 blocks
  auto fetch_ids = [&](int n0) {
    const int jb = b0 + w + NW * (n0 + lane);
    my_ids = jb < b1 ? bt[jb] : 0;
  };

  constexpr int NS = decode_slots<EB>();
  uint4 kb[NS][C::NR][C::U], vb[NS][C::NV];  // tile slots: NS - 1 tiles in flight
  auto load_tile = [&](int id, bool real, uint4 (&kk)[C::NR][C::U], uint4 (&vv)[C::NV]) {
    const int64_t base = ((int64_t)id * p.num_kv_heads + g) * tile_bytes;
    wd.load_tile(p.k_cache + base, p.v_cache + base, real ? (int)tile_bytes : 0, kk, vv);
  };
  auto id_ok = [&](int id) { return id >= 0 && id < p.num_blocks; };
  const int nmine = b1 > b0 + w ? (b1 - b0 - w + NW - 1) / NW : 0;

  auto process = [&](uint4 (&kc)[C::NR][C::U], uint4 (&vc)[C::NV], int id_cur, int n) {
    const int jblk = b0 + w + NW * n;
    int nvalid = id_ok(id_cur) ? min(kBlock, ctx - jblk * kBlock) : 0;
    if (app && jblk == b1 - 1 && nvalid == tn + 1 && (int64_t)id_cur * kBlock + tn == slot) {
      nvalid = tn;  // the token itself comes from the LDS copy
      hit = true;
    }
    wd.process(kc, vc, nvalid);
  };

  // Blocks are taken in chunks of 64 (one block id per lane).  NS register
  // slots rotate: while one tile is computed the next NS - 1 are in flight.
  // The loads are unconditional (a tile past the chunk's end is an empty
  // descriptor), so the wait before each tile is a static count.  The first
  // chunk's first loads are issued before the loop, and the appended row's
  // registers die before it.
  int cnt = min(64, nmine);
  auto id_at = [&](int i) { return __builtin_amdgcn_readlane(my_ids, min(i, cnt - 1)); };
  auto prologue = [&]() {
#pragma unroll
    for (int t = 0; t < NS - 1; ++t) load_tile(id_at(t), t < cnt && id_ok(id_at(t)), kb[t], vb[t]);
  };
  if (app) {
    // the new row was loaded right after the block ids, which the first
    // tile loads wait for anyway: keep its copy before them (after them,
    // the wait for the row would also cover the first tile)
    slot = ((int64_t)__builtin_amdgcn_readfirstlane((int)(slot_in >> 32)) << 32) |
           (uint32_t)__builtin_amdgcn_readfirstlane((int)slot_in);
    wd.stash_new_row(lds.newk[w], lds.newv[w], knew, vnew);
  }
  if (nmine > 0) prologue();
  for (int c0 = 0; c0 < nmine;) {
    for (int n = 0; n < cnt; n += NS) {
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        const int t = n + sl + NS - 1;  // tile whose load goes out now
        load_tile(id_at(t), t < cnt && id_ok(id_at(t)), kb[(sl + NS - 1) % NS], vb[(sl + NS - 1) % NS]);
        if (n + sl < cnt) process(kb[sl], vb[sl], id_at(n + sl), c0 + n + sl);
      }
    }
    c0 += 64;
    if (c0 >= nmine) break;
    cnt = min(64, nmine - c0);
    fetch_ids(c0);
    prologue();
  }
  if (hit) {
    wd.stashed_tile(lds.newk[w], lds.newv[w], kb[0], vb[0]);
    wd.process(kb[0], vb[0], 1);
  }
}

// Wave totals, then the merge of the NW waves' (m, l, O) in LDS with the
// online-softmax rescale.  With `single` the workgroup writes the normalised
// output rows of (sequence s, kv head g); otherwise query head h of the group
// leaves its partial state in workspace slot base + h * stride.  Ends with the
// LDS still in use: the caller syncs before the next tile of work.
template <int EB, int D, int G>
__device__ inline void finish_waves(WaveDecoder<EB, D, G>& wd, DecodeLds<EB, D, G>& lds,
                                    const DecodeParams& p, int w, int s, int g, bool single,
                                    int64_t base, int64_t stride) {
  using C = DecodeCfg<EB, D, G>;
  constexpr int NW = kDecodeWaves;
  const int lane = wd.lane;
  const float l_head = wd.totals();
  if ((lane & (C::ROW_BITS | C::HEAD_BITS | C::DUP_BITS)) == 0) {
    lds.sm[w][wd.hh] = wd.m_mine;
    lds.sl[w][wd.hh] = l_head;
  }
  if (wd.vpart == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int x = 0; x < C::NV; ++x) lds.so[w][h][wd.dim_of(x)] = wd.o[h][x];
  }
  __syncthreads();

  for (int e = threadIdx.x; e < G * D; e += NW * kWave) {
    const int h = e / D;
    const int x = e - h * D;
    float M = lds.sm[0][h];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, lds.sm[ww][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = exp2f(lds.sm[ww][h] - M);
      L = fmaf(lds.sl[ww][h], f, L);
      O = fmaf(lds.so[ww][h][x], f, O);
    }
    if (single) {
      const int64_t row = (int64_t)s * p.num_q_heads + g * G + h;
      float val = L > 0.f ? O / L : 0.f;
      if constexpr (EB == 1) val *= p.v_scale;
      if constexpr (EB <= 2)
        ((uint16_t*)p.out)[row * D + x] = to_bf16(val);
      else
        ((float*)p.out)[row * D + x] = val;
    } else {
      const int64_t slot = base + h * stride;
      p.ws_o[slot * D + x] = O;
      if (x == 0) {
        p.ws_m[slot] = M;
        p.ws_l[slot] = L;
      }
    }
  }
}

// CASC: shared-prefix decode.  The workgroup covers a partition of the
// sequence's own blocks only (those after its group's shared prefix) and
// always leaves a partial state for the merge.
template <int EB, int D, int G, bool CASC = false>
__global__ __launch_bounds__(kDecodeWaves * kWave)
__attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<EB, D, G>())))
void decode_partition_kernel(DecodeParams p) {
  constexpr int NW = kDecodeWaves;
  __shared__ DecodeLds<EB, D, G> lds;

  const int bid = blockIdx.x;
  const int g = bid % p.num_kv_heads;
  const int s = (bid / p.num_kv_heads) % p.num_seqs;
  // partitions past the first exist only for the longer sequences: they are
  // dispatched first, so the last workgroups to start are first partitions,
  // which every (sequence, kv head) has and which even out the tail
  const int part = p.num_partitions - 1 - bid / (p.num_kv_heads * p.num_seqs);

  // wave index, provably uniform so that loop control stays scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  WaveDecoder<EB, D, G> wd;
  wd.init(lds.pbuf[w], p.scale_log2);
  const int lane = wd.lane;
  const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks_per_seq;

  int b0, ctx, nblk, nparts, pre = 0;
  int my_ids;  // id of block b0 + w + NW * lane
  if constexpr (!CASC) {
    b0 = part * p.partition_blocks;
    // The first block ids of this wave and q do not depend on the context
    // length: issue them together with its load, so the first KV tile waits
    // on one memory round trip instead of two.
    {
      const int jb = b0 + w + NW * lane;
      my_ids = jb < min(p.max_blocks_per_seq, b0 + p.partition_blocks) ? bt[jb] : 0;
    }
    wd.load_q((const char*)p.q + ((int64_t)s * p.num_q_heads + (int64_t)g * G) * DecodeCfg<EB, D, G>::QRB, wd.qv);
    ctx = clamp_ctx(p.context_lens[s], p);
    nblk = (ctx + kBlock - 1) / kBlock;
    nparts = nblk == 0 ? 1 : (nblk + p.partition_blocks - 1) / p.partition_blocks;
  } else {
    wd.load_q((const char*)p.q + ((int64_t)s * p.num_q_heads + (int64_t)g * G) * DecodeCfg<EB, D, G>::QRB, wd.qv);
    ctx = max(0, min(p.context_lens[s], p.max_blocks_per_seq * kBlock));
    const int pl = prefix_of(p, s, ctx);
    pre = prefix_parts(p, pl);
    // own blocks [pl / 16, nblk), cut into at most num_partitions partitions
    nblk = min((ctx + kBlock - 1) / kBlock, pl / kBlock + p.num_partitions * p.partition_blocks);
    ctx = min(ctx, nblk * kBlock);
    const int own = nblk - pl / kBlock;
    nparts = own == 0 ? 1 : (own + p.partition_blocks - 1) / p.partition_blocks;
    b0 = pl / kBlock + part * p.partition_blocks;
    const int jb = b0 + w + NW * lane;
    my_ids = jb < min(nblk, b0 + p.partition_blocks) ? bt[jb] : 0;
  }
  if (part >= nparts) return;  // uniform over the workgroup
  const int b1 = min(nblk, b0 + p.partition_blocks);
  wd.reset();
  const bool append = !CASC && p.new_k != nullptr && b1 == nblk && ctx > 0;
  stream_blocks(wd, lds, p, bt, g, w, b0, b1, ctx, my_ids, append ? s : -1);

  const int64_t row0 = (int64_t)s * p.num_q_heads + g * G;
  const int64_t stride = CASC ? p.ws_stride : p.num_partitions;
  finish_waves(wd, lds, p, w, s, g, !CASC && nparts == 1, row0 * stride + pre + part, stride);
}

// ---------------------------------------------------------------------------
// Work-balanced schedule.  For one kv head, the blocks of all sequences in
// sequence order form one list of T = sum_s ceil(ctx_s / 16) entries.  The
// list is cut into R ranges of equal length (entry j belongs to range
// floor(j R / T)) and workgroup (range, kv head) reads exactly its range, so
// every workgroup streams the same number of tiles whatever the mix of
// context lengths and no long sequence leaves a tail of late workgroups.
// A range holds pieces ("segments") of one or more sequences.  A sequence
// that lies wholly inside a range is finished there; otherwise the range's
// first segment (slot 0) or last segment (slot 1) leaves a partial state and
// the merge kernel combines the pieces of the sequence, range by range.
constexpr int kBalancedMinBlocks = 8;   // blocks a range holds at least

// Ranges actually used for a list of T blocks when the grid offers R.
__device__ inline int balanced_ranges(int R, int T) {
  return max(1, min(R, (T + kBalancedMinBlocks - 1) / kBalancedMinBlocks));
}
__device__ inline int range_of(int j, int T, int R) { return (int)((int64_t)j * R / T); }
__device__ inline int range_start(int w, int T, int R) {
  return (int)(((int64_t)w * T + R - 1) / R);
}
// Tokens of a context that the balanced schedule reads: bounded by the table
// row and by the host's bound on every context length.
__device__ inline int balanced_ctx(int ctx, const DecodeParams& p) {
  const int cap = min(p.max_blocks_per_seq * kBlock, p.max_ctx);
  return max(0, min(ctx, cap));
}

template <int EB, int D, int G>
__global__ __launch_bounds__(kDecodeWaves * kWave)
__attribute__((amdgpu_waves_per_eu(decode_waves_per_eu<EB, D, G>())))
void decode_balanced_kernel(DecodeParams p) {
  using C = DecodeCfg<EB, D, G>;
  constexpr int NW = kDecodeWaves;
  constexpr int PER_THREAD = kBalancedMaxSeqs / (NW * kWave);
  static_assert(PER_THREAD * NW * kWave == kBalancedMaxSeqs, "scan layout");
  __shared__ DecodeLds<EB, D, G> lds;
  __shared__ int cum[kBalancedMaxSeqs + 1];  // blocks before sequence s
  __shared__ int sctx[kBalancedMaxSeqs];     // context of sequence s
  __shared__ int wtot[NW];

  const int g = blockIdx.x % p.num_kv_heads;
  const int range = blockIdx.x / p.num_kv_heads;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int S = p.num_seqs;

  // ---- block counts of every sequence and their exclusive prefix sums
  const int sfirst = threadIdx.x * PER_THREAD;
  int cl[PER_THREAD];
  int run = 0;
#pragma unroll
  for (int i = 0; i < PER_THREAD; ++i) {
    cl[i] = sfirst + i < S ? balanced_ctx(p.context_lens[sfirst + i], p) : 0;
    run += (cl[i] + kBlock - 1) / kBlock;
  }
  int inc = run;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == kWave - 1) wtot[w] = inc;
  __syncthreads();
  int excl = inc - run, T = 0;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    excl += ww < w ? wtot[ww] : 0;
    T += wtot[ww];
  }
#pragma unroll
  for (int i = 0; i < PER_THREAD; ++i) {
    if (sfirst + i < S) {
      cum[sfirst + i] = excl;
      sctx[sfirst + i] = cl[i];
    }
    excl += (cl[i] + kBlock - 1) / kBlock;
  }
  if (threadIdx.x == 0) cum[S] = T;
  __syncthreads();

  T = __builtin_amdgcn_readfirstlane(T);
  if (T == 0) return;
  const int R = balanced_ranges(p.num_ranges, T);
  if (range >= R) return;
  const int B0 = range_start(range, T, R);
  const int B1 = range_start(range + 1, T, R);
  if (B0 >= B1) return;
  // first sequence of the range: the last s with cum[s] <= B0
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(cum[mid]) <= B0)
      lo = mid;
    else
      hi = mid - 1;
  }

  WaveDecoder<EB, D, G> wd;
  wd.init(lds.pbuf[w], p.scale_log2);
  // The segments of the range, in sequence order.  A segment's block ids
  // and q are requested before the previous segment's wave merge, so their
  // memory round trip overlaps it.
  auto next_segment = [&](int s) {  // first sequence >= s with blocks in the range, or S
    for (; s < S; ++s) {
      const int cs = __builtin_amdgcn_readfirstlane(cum[s]);
      if (cs >= B1) return S;
      const int ce = __builtin_amdgcn_readfirstlane(cum[s + 1]);
      if (max(B0, cs) < min(B1, ce)) return s;  // else a sequence with no blocks
    }
    return S;
  };
  auto fetch = [&](int s) {  // ids of this wave's blocks of segment s; its q into wd.qv
    const int cs = __builtin_amdgcn_readfirstlane(cum[s]);
    const int ce = __builtin_amdgcn_readfirstlane(cum[s + 1]);
    const int jb = max(B0, cs) - cs + w + NW * lane;
    const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    const int ids = jb < min(B1, ce) - cs ? bt[jb] : 0;
    wd.load_q((const char*)p.q + ((int64_t)s * p.num_q_heads + (int64_t)g * G) * C::QRB, wd.qv);
    return ids;
  };
  int s = next_segment(lo);
  int my_ids = s < S ? fetch(s) : 0;
  while (s < S) {
    const int cs = __builtin_amdgcn_readfirstlane(cum[s]);
    const int ce = __builtin_amdgcn_readfirstlane(cum[s + 1]);
    const int sb = max(B0, cs), se = min(B1, ce);
    const int ctx = __builtin_amdgcn_readfirstlane(sctx[s]);
    const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks_per_seq;
    wd.reset();
    const bool append = p.new_k != nullptr && se == ce && ctx > 0;
    stream_blocks(wd, lds, p, bt, g, w, sb - cs, se - cs, ctx, my_ids, append ? s : -1);
    const int s_next = next_segment(s + 1);
    const int ids_next = s_next < S ? fetch(s_next) : 0;
    const bool whole = cs >= B0 && ce <= B1;
    const int slot = sb == B0 ? 0 : 1;
    finish_waves(wd, lds, p, w, s, g, whole,
                 ((int64_t)(g * p.num_ranges + range) * 2 + slot) * G, 1);
    __syncthreads();
    s = s_next;
    my_ids = ids_next;
  }
}

// Fused append: one wave writes sequence s's newest token for kv head g to
// its slot, encoded as the cache write encodes it (a bit copy; E4M3 codes
// for fp8 pools).  Rows whose context length is not positive, or whose slot
// is negative or outside the pool, are not written.
template <int EB, int D>
__device__ inline void write_new_row(const DecodeParams& p, int s, int g) {
  constexpr int RB = D * EB;                   // pool bytes of one row
  constexpr int QB = EB == 4 ? 4 : 2;          // bytes of an input element
  const int lane = threadIdx.x;
  const int64_t slot = p.new_slots[s];
  const int ctx = p.context_lens[s];
  const char* krow = p.new_k + ((int64_t)s * p.num_kv_heads + g) * D * QB;
  const char* vrow = p.new_v + ((int64_t)s * p.num_kv_heads + g) * D * QB;
  uint4 kc = make_uint4(0, 0, 0, 0);
  if (lane < RB / 16) {
    if constexpr (EB == 1) {
      const uint4 a = *(const uint4*)(krow + lane * 32);
      const uint4 b = *(const uint4*)(krow + lane * 32 + 16);
      kc = make_uint4(quantize4(a.x, a.y, p.k_quant_scale), quantize4(a.z, a.w, p.k_quant_scale),
                      quantize4(b.x, b.y, p.k_quant_scale), quantize4(b.z, b.w, p.k_quant_scale));
    } else {
      kc = *(const uint4*)(krow + lane * 16);
    }
  }
  constexpr int XL = D / kWave;
  uint32_t ve[XL];
#pragma unroll
  for (int e = 0; e < XL; ++e) {
    const int dim = lane + e * kWave;
    if constexpr (EB == 1)
      ve[e] = quantize4(*(const uint16_t*)(vrow + dim * 2), 0u, p.v_quant_scale) & 0xffu;
    else if constexpr (EB == 2)
      ve[e] = *(const uint16_t*)(vrow + dim * 2);
    else
      ve[e] = *(const uint32_t*)(vrow + dim * 4);
  }
  if (ctx <= 0 || slot < 0 || slot >= (int64_t)p.num_blocks * kBlock) return;
  const int64_t base = (slot / kBlock * p.num_kv_heads + g) * (int64_t)kBlock * RB;
  const int o = (int)(slot % kBlock);
  if (lane < RB / 16) *(uint4*)(p.k_cache + base + o * RB + lane * 16) = kc;
#pragma unroll
  for (int e = 0; e < XL; ++e) {
    char* dst = (char*)p.v_cache + base + ((int64_t)(lane + e * kWave) * kBlock + o) * EB;
    if constexpr (EB == 1)
      *(uint8_t*)dst = (uint8_t)ve[e];
    else if constexpr (EB == 2)
      *(uint16_t*)dst = (uint16_t)ve[e];
    else
      *(uint32_t*)dst = ve[e];
  }
}

// Merge of the balanced schedule: one wave per (sequence, query head).  The
// wave recomputes the list position of the sequence's blocks, finds the
// ranges that hold them and merges their partial states in range order with
// the online-softmax rescale.  Sequences finished inside one range are left
// alone; sequences without blocks get a zero row.
// Workgroups past num_seqs * num_q_heads (launched for a fused append) each
// write one (sequence, kv head)'s new row; the merge waves do not wait on
// those stores.
template <int EB, int D>
__global__ __launch_bounds__(kWave) void decode_balanced_reduce_kernel(DecodeParams p) {
  if (blockIdx.x >= p.num_seqs * p.num_q_heads) {
    const int r = blockIdx.x - p.num_seqs * p.num_q_heads;
    write_new_row<EB, D>(p, r / p.num_kv_heads, r % p.num_kv_heads);
    return;
  }
  const int s = blockIdx.x / p.num_q_heads;
  const int hq = blockIdx.x - s * p.num_q_heads;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int g = hq / G;
  const int h = hq - g * G;
  const int lane = threadIdx.x;
  const int64_t row = (int64_t)s * p.num_q_heads + hq;
  constexpr int XL = D / kWave;  // dims per lane

  int tot = 0, before = 0;
  for (int i = lane; i < p.num_seqs; i += kWave) {
    const int n = (balanced_ctx(p.context_lens[i], p) + kBlock - 1) / kBlock;
    tot += n;
    before += i < s ? n : 0;
  }
#pragma unroll
  for (int m = kWave / 2; m > 0; m >>= 1) {
    tot += __shfl_xor(tot, m);
    before += __shfl_xor(before, m);
  }
  const int nb = (balanced_ctx(p.context_lens[s], p) + kBlock - 1) / kBlock;
  if (nb == 0) {
#pragma unroll
    for (int e = 0; e < XL; ++e) {
      const int x = lane + e * kWave;
      if constexpr (EB <= 2)
        ((uint16_t*)p.out)[row * D + x] = 0;
      else
        ((float*)p.out)[row * D + x] = 0.f;
    }
    return;
  }
  const int R = balanced_ranges(p.num_ranges, tot);
  const int wf = range_of(before, tot, R);
  const int wl = range_of(before + nb - 1, tot, R);
  if (wf == wl) return;  // finished by the decode kernel
  const int first_slot = before > range_start(wf, tot, R) ? 1 : 0;
  const int nparts = wl - wf + 1;
  auto slot_of = [&](int q) {
    return ((int64_t)(g * p.num_ranges + wf + q) * 2 + (q == 0 ? first_slot : 0)) * G + h;
  };

  float acc[XL];
#pragma unroll
  for (int e = 0; e < XL; ++e) acc[e] = 0.f;
  float L = 0.f, M = kNegBig;
  constexpr int PG = 8;  // partial states loaded together
  for (int q0 = 0; q0 < nparts; q0 += PG) {
    float mq[PG], lq[PG], oq[PG][XL];
#pragma unroll
    for (int j = 0; j < PG; ++j) {
      const int64_t sl = slot_of(min(q0 + j, nparts - 1));
      mq[j] = p.ws_m[sl];
      lq[j] = p.ws_l[sl];
#pragma unroll
      for (int e = 0; e < XL; ++e) oq[j][e] = p.ws_o[sl * D + lane + e * kWave];
    }
    float Mg = M;
#pragma unroll
    for (int j = 0; j < PG; ++j)
      if (q0 + j < nparts) Mg = fmaxf(Mg, mq[j]);
    const float r = exp2f(M - Mg);  // rescale of what was merged so far
    L *= r;
#pragma unroll
    for (int e = 0; e < XL; ++e) acc[e] *= r;
#pragma unroll
    for (int j = 0; j < PG; ++j) {
      const float f = q0 + j < nparts ? exp2f(mq[j] - Mg) : 0.f;
      L = fmaf(lq[j], f, L);
#pragma unroll
      for (int e = 0; e < XL; ++e) acc[e] = fmaf(oq[j][e], f, acc[e]);
    }
    M = Mg;
  }
  float inv = L > 0.f ? 1.f / L : 0.f;
  if constexpr (EB == 1) inv *= p.v_scale;
#pragma unroll
  for (int e = 0; e < XL; ++e) {
    const float val = acc[e] * inv;
    const int x = lane + e * kWave;
    if constexpr (EB <= 2)
      ((uint16_t*)p.out)[row * D + x] = to_bf16(val);
    else
      ((float*)p.out)[row * D + x] = val;
  }
}


// Split-K merge: every partition p of a sequence left (m_p, l_p, O_p) with
// m in log2 units and O unnormalised.  The partitions are merged with the
// same rescale the online softmax uses within one:
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  out = sum_p O_p 2^(m_p - M) / L.
// One wave per (sequence, query head); sequences with a single partition were
// finished by the partition kernel.
// CASC: shared-prefix decode; a row's slots are its group's prefix
// partitions followed by its own partitions, and every row is merged here.
template <int EB, int D, bool CASC = false>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(DecodeParams p) {
  const int s = blockIdx.x / p.num_q_heads;
  const int hq = blockIdx.x - s * p.num_q_heads;
  const int64_t row = (int64_t)s * p.num_q_heads + hq;
  const int stride = CASC ? p.ws_stride : p.num_partitions;  // slots per row
  const float* wm = p.ws_m + row * stride;
  const float* wl = p.ws_l + row * stride;
  const float* wo = p.ws_o + row * stride * D;
  const int lane = threadIdx.x;

  constexpr int XL = D / kWave;  // dims per lane
  float acc[XL];
#pragma unroll
  for (int e = 0; e < XL; ++e) acc[e] = 0.f;
  float L = 0.f;
  // Up to 8 partitions at a time: their m, l and O are loaded together and
  // merged after one memory round trip (the running maximum is carried from
  // group to group with the same rescale).  The first group's loads are
  // issued before the context length is known (slots below num_partitions
  // always exist), so a short merge costs a single round trip.
  constexpr int PG = 8;
  float M = kNegBig;
  int nparts = PG;  // refined below once the context length has arrived
  for (int q0 = 0; q0 < nparts; q0 += PG) {
    float mq[PG], lq[PG], oq[PG][XL];
#pragma unroll
    for (int j = 0; j < PG; ++j) {
      const int q = min(q0 + j, (q0 == 0 ? stride : nparts) - 1);
      mq[j] = wm[q];
      lq[j] = wl[q];
#pragma unroll
      for (int e = 0; e < XL; ++e) oq[j][e] = wo[(int64_t)q * D + lane + e * kWave];
    }
    if (q0 == 0) {
      if constexpr (!CASC) {
        const int ctx = clamp_ctx(p.context_lens[s], p);
        const int nblk = (ctx + kBlock - 1) / kBlock;
        nparts = (nblk + p.partition_blocks - 1) / p.partition_blocks;
        if (nparts <= 1) return;  // finished by the partition kernel
      } else {
        const int ctx = max(0, min(p.context_lens[s], p.max_blocks_per_seq * kBlock));
        const int pl = prefix_of(p, s, ctx);
        const int nblk = min((ctx + kBlock - 1) / kBlock,
                             pl / kBlock + p.num_partitions * p.partition_blocks);
        const int own = nblk - pl / kBlock;
        nparts = prefix_parts(p, pl) + (own == 0 ? 1 : (own + p.partition_blocks - 1) / p.partition_blocks);
      }
    }
    float Mg = M;
#pragma unroll
    for (int j = 0; j < PG; ++j)
      if (q0 + j < nparts) Mg = fmaxf(Mg, mq[j]);
    const float r = exp2f(M - Mg);  // rescale of what was merged so far
    L *= r;
#pragma unroll
    for (int e = 0; e < XL; ++e) acc[e] *= r;
#pragma unroll
    for (int j = 0; j < PG; ++j) {
      const float f = q0 + j < nparts ? exp2f(mq[j] - Mg) : 0.f;
      L = fmaf(lq[j], f, L);
#pragma unroll
      for (int e = 0; e < XL; ++e) acc[e] = fmaf(oq[j][e], f, acc[e]);
    }
    M = Mg;
  }
  float inv = L > 0.f ? 1.f / L : 0.f;
  if constexpr (EB == 1) inv *= p.v_scale;
#pragma unroll
  for (int e = 0; e < XL; ++e) {
    const float val = acc[e] * inv;
    const int x = lane + e * kWave;
    if constexpr (EB <= 2)
      ((uint16_t*)p.out)[row * D + x] = to_bf16(val);
    else
      ((float*)p.out)[row * D + x] = val;
  }
}

// Fused append with per-partition workgroups: the new rows of every
// (sequence, kv head), one wave each, after the decode of the call.
template <int EB, int D>
__global__ __launch_bounds__(kWave) void append_rows_kernel(DecodeParams p) {
  write_new_row<EB, D>(p, blockIdx.x / p.num_kv_heads, blockIdx.x % p.num_kv_heads);
}

template <int EB, int D, int G>
static hipError_t launch_decode_t(const DecodeParams& prm, hipStream_t stream) {
  if (prm.num_ranges > 0) {
    // one range per resident workgroup slot of this variant
    static_assert(decode_waves_per_eu<EB, D, G>() <= kBalancedMaxWgPerCu, "workspace bound");
    DecodeParams bp = prm;
    bp.num_ranges = max(1, prm.num_ranges * decode_waves_per_eu<EB, D, G>() / kBalancedMaxWgPerCu);
    const int64_t rows = (int64_t)bp.num_ranges * 2 * bp.num_q_heads;
    bp.ws_l = bp.ws_m + rows;
    bp.ws_o = bp.ws_m + 2 * rows;
    hipLaunchKernelGGL((decode_balanced_kernel<EB, D, G>),
                       dim3((unsigned)(bp.num_ranges * bp.num_kv_heads)),
                       dim3(kDecodeWaves * kWave), 0, stream, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t writers = bp.new_k ? (int64_t)bp.num_seqs * bp.num_kv_heads : 0;
    hipLaunchKernelGGL((decode_balanced_reduce_kernel<EB, D>),
                       dim3((unsigned)(bp.num_seqs * bp.num_q_heads + writers)), dim3(kWave), 0,
                       stream, bp);
    return hipGetLastError();
  }
  const int64_t grid = (int64_t)prm.num_partitions * prm.num_seqs * prm.num_kv_heads;
  hipLaunchKernelGGL((decode_partition_kernel<EB, D, G>), dim3((unsigned)grid),
                     dim3(kDecodeWaves * kWave), 0, stream, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (prm.num_partitions > 1) {
    hipLaunchKernelGGL((decode_reduce_kernel<EB, D>),
                       dim3((unsigned)(prm.num_seqs * prm.num_q_heads)), dim3(kWave), 0, stream, prm);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (prm.new_k) {
    hipLaunchKernelGGL((append_rows_kernel<EB, D>),
                       dim3((unsigned)(prm.num_seqs * prm.num_kv_heads)), dim3(kWave), 0, stream, prm);
    e = hipGetLastError();
  }
  return e;
}

bool decode_supported(int elem_bytes, int head_dim, int group) {
  const bool shape = elem_bytes == 1 ? head_dim == 128
                                     : (elem_bytes == 2 || elem_bytes == 4) && (head_dim == 64 || head_dim == 128);
  return shape && (group == 1 || group == 2 || group == 4 || group == 8);
}

template <int EB, int D, int G>
static hipError_t launch_own_and_merge_t(const DecodeParams& prm, hipStream_t stream) {
  const int64_t grid = (int64_t)prm.num_partitions * prm.num_seqs * prm.num_kv_heads;
  hipLaunchKernelGGL((decode_partition_kernel<EB, D, G, true>), dim3((unsigned)grid),
                     dim3(kDecodeWaves * kWave), 0, stream, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_reduce_kernel<EB, D, true>),
                     dim3((unsigned)(prm.num_seqs * prm.num_q_heads)), dim3(kWave), 0, stream, prm);
  return hipGetLastError();
}

hipError_t launch_decode_own_and_merge(const SharedPrefixArgs& a, const CacheGeom& g,
                                       hipStream_t stream) {
  DecodeParams p = {};
  p.out = a.d.out;
  p.q = a.d.q;
  p.k_cache = (const char*)a.d.k_cache;
  p.v_cache = (const char*)a.d.v_cache;
  p.block_tables = a.d.block_tables;
  p.context_lens = a.d.context_lens;
  const int64_t rows = (int64_t)a.d.num_seqs * a.d.num_q_heads;
  p.ws_m = a.d.ws;
  p.ws_l = a.d.ws + rows * a.ws_stride;
  p.ws_o = a.d.ws + (2 * rows * a.ws_stride + 3) / 4 * 4;
  p.max_blocks_per_seq = a.d.max_blocks_per_seq;
  p.num_seqs = a.d.num_seqs;
  p.num_q_heads = a.d.num_q_heads;
  p.num_kv_heads = g.num_kv_heads;
  p.num_blocks = g.num_blocks;
  p.num_partitions = a.d.num_partitions;
  p.partition_blocks = a.d.partition_blocks;
  p.scale_log2 = a.d.scale * g.k_scale * kLog2e;
  p.v_scale = g.v_scale;
  p.prefix_lens = a.prefix_lens;
  p.group_size = a.group_size;
  p.prefix_partition = a.prefix_partition;
  p.max_prefix = a.prefix_parts * a.prefix_partition;
  p.ws_stride = a.ws_stride;
  const int G = a.d.num_q_heads / g.num_kv_heads;
#define PA_OWN_CASE(EB_, D_, G_) \
  if (g.elem_bytes == EB_ && g.head_dim == D_ && G == G_) return launch_own_and_merge_t<EB_, D_, G_>(p, stream);
  PA_OWN_CASE(2, 128, 1) PA_OWN_CASE(2, 128, 2) PA_OWN_CASE(2, 128, 4) PA_OWN_CASE(2, 128, 8)
  PA_OWN_CASE(2, 64, 1) PA_OWN_CASE(2, 64, 2) PA_OWN_CASE(2, 64, 4) PA_OWN_CASE(2, 64, 8)
  PA_OWN_CASE(1, 128, 1) PA_OWN_CASE(1, 128, 2) PA_OWN_CASE(1, 128, 4) PA_OWN_CASE(1, 128, 8)
#undef PA_OWN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, const CacheGeom& g, hipStream_t stream) {
  DecodeParams p = {};
  p.out = a.out;
  p.q = a.q;
  p.k_cache = (const char*)a.k_cache;
  p.v_cache = (const char*)a.v_cache;
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  // partial slots (seq, q head, partition): m, l, then o (the balanced
  // schedule lays out its own (kv head, range, 2, group head) slots)
  const int64_t rows = (int64_t)a.num_seqs * a.num_q_heads * a.num_partitions;
  p.ws_m = a.ws;
  p.ws_l = a.ws ? a.ws + rows : nullptr;
  p.ws_o = a.ws ? a.ws + 2 * rows : nullptr;
  p.num_ranges = a.num_ranges;
  p.max_ctx = a.max_ctx;
  p.new_k = (const char*)a.new_k;
  p.new_v = (const char*)a.new_v;
  p.new_slots = a.new_slots;
  p.k_quant_scale = g.k_scale;
  p.v_quant_scale = g.v_scale;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.num_seqs = a.num_seqs;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = g.num_kv_heads;
  p.num_blocks = g.num_blocks;
  p.num_partitions = a.num_partitions;
  p.partition_blocks = a.partition_blocks;
  // fp8 pools: the K scale multiplies every score, the V scale the output
  p.scale_log2 = a.scale * g.k_scale * kLog2e;
  p.v_scale = g.v_scale;
  const int G = a.num_q_heads / g.num_kv_heads;

#define PA_DECODE_CASE(EB_, D_, G_) \
  if (g.elem_bytes == EB_ && g.head_dim == D_ && G == G_) return launch_decode_t<EB_, D_, G_>(p, stream);
#define PA_DECODE_GROUPS(EB_, D_) \
  PA_DECODE_CASE(EB_, D_, 1) PA_DECODE_CASE(EB_, D_, 2) PA_DECODE_CASE(EB_, D_, 4) PA_DECODE_CASE(EB_, D_, 8)
  PA_DECODE_GROUPS(2, 128)
  PA_DECODE_GROUPS(2, 64)
  PA_DECODE_GROUPS(4, 128)
  PA_DECODE_GROUPS(4, 64)
  PA_DECODE_GROUPS(1, 128)
#undef PA_DECODE_GROUPS
#undef PA_DECODE_CASE
  return hipErrorInvalidValue;
}

}  // namespace pa
