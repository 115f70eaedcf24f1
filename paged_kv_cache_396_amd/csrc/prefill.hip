// Chunked-prefill attention over paged KV for gfx950 (bf16 matrix cores).
//
// What is computed: a long prompt is processed one chunk at a time, and the
// tokens of one step from several requests are flattened into one batch
// (zihan-zhang.net vLLM study, 3.5 and 5.6).  For
// request r with chunk rows query_start_loc[r] .. query_start_loc[r+1]-1
// (n_r of them) and context ctx_r (prior tokens plus the chunk, all already in
// the pools), query i sits at position pos = ctx_r - n_r + i and attends
// causally (same page, 1.1.1) to keys 0 .. pos:
//   out[i, h] = softmax(scale * K[0..pos, h/G] q[i, h]) V[0..pos, h/G]
// with K and V read block by block through the request's block table
// (same page, 3.2) and the softmax evaluated online (same page, 4.3.1).
//
// Mapping onto CDNA4:
//  * one workgroup of 4 waves per (request, kv head, tile of query rows).
//    A "column" is one (query, q head) pair; the G q heads of the kv head and
//    QT consecutive queries give 128 * NCB columns, 32 * NCB per wave.
//    Workgroup ids are mapped so that all tiles of one (request, kv head)
//    run on the same XCD and share its L2 copy of the K/V tiles.
//  * the workgroup walks the keys 64 at a time (four 16-token blocks).  The
//    K and V tiles of the four blocks are copied from the pools into LDS
//    (double buffered, the next tile's global loads in flight while the
//    current one is computed).  Blocks past the context are never read.
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 (32 keys x 32 columns per instruction), so
//    each lane holds one column's scores for 16 keys and the row max of the
//    softmax needs a single exchange between the two lane halves.  The MFMA
//    row -> key assignment is permuted so that the 8 fp32 scores a lane holds
//    for one 16-key step are 8 consecutive keys: after conversion to bf16
//    they are directly the B operand of the P V product.
//  * O^T = V^T P accumulates in fp32 (32 dims x 32 columns per instruction);
//    the V tile in LDS is dim-major, so each A fragment is one 16-byte read.
//  * softmax state (running max in log2 units, running sum) is per lane;
//    the max is raised only when a score exceeds it by more than 2^8 (the
//    rescale is exact when it happens; any common reference max gives the
//    same softmax).  P is rounded to bf16 for the matrix product.
#include <float.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

#ifndef PA_PF_NCB
#define PA_PF_NCB 1
#endif
#ifndef PA_PF_WAVES_PER_EU
#define PA_PF_WAVES_PER_EU 2
#endif

#ifndef PA_PF_WAVES
#define PA_PF_WAVES 4
#endif
#ifndef PA_PF_SCHED
#define PA_PF_SCHED 0
#endif

constexpr int kPfWaves = PA_PF_WAVES;  // waves per workgroup
constexpr int kPfKT = 64;          // keys per iteration (four 16-token blocks)
constexpr int kPfBlocks = kPfKT / kBlock;
constexpr float kPfGap = 8.0f;     // log2 units a score may exceed the reference max
constexpr float kPfNegBig = -FLT_MAX;

template <int D>
struct PrefillCfg {
  static constexpr int RB = D * 2;             // bytes of one K row (bf16)
  static constexpr int KCH = RB / 16;          // 16-byte chunks per K row
  static constexpr int DS = D / 16;            // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;            // 32-dim blocks of O^T
  static constexpr int VRB = kPfKT * 2;        // bytes of one V row (one dim) of a tile
  // LDS rows are padded by 16 bytes: the 32 rows one MFMA fragment reads at
  // a fixed 16-byte chunk then fall on distinct banks (row strides of 17 or
  // 9 chunks are odd), whether the bank array is 128 or 256 bytes wide, and
  // every fragment address is a per-lane base plus an immediate offset.
  static constexpr int KRS = RB + 16;          // LDS stride of one K row
  static constexpr int VRS = VRB + 16;         // LDS stride of one V row
  static constexpr int K_LDS = kPfKT * KRS;    // one K stage
  static constexpr int V_LDS = D * VRS;        // one V stage
  static constexpr int STAGE = K_LDS + V_LDS;
  static constexpr int NKL = kPfKT * KCH / (kPfWaves * kWave);  // K chunks per thread
  static constexpr int NVL = 2 * D * kPfBlocks / (kPfWaves * kWave);  // V chunks per thread
  static_assert(NKL >= 1 && NVL >= 1, "tile too small for the workgroup");
};

struct PrefillParams {
  void* out;
  const char* q;
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_tables;
  const int32_t* query_start_loc;
  const int32_t* context_lens;
  int max_blocks_per_seq;
  int num_reqs;
  int total_q_tokens;
  int num_q_heads;
  int num_kv_heads;
  int num_blocks;
  int num_qtiles;
  float scale_log2;
};

// Key (within a 32-key block) that MFMA row m of S^T stands for.  Rows are
// permuted inside each group of 16 (quads 1 and 2 swapped) so that the
// accumulator registers 8t..8t+7 of lane l hold keys 16t + 8(l/32) + 0..7.
// The permutation is its own inverse; the K tile is stored in LDS in this
// row order, so fragment lane m simply reads LDS row m.
__device__ inline int pf_row_key(int m) {
  const int quad = (m >> 2) & 3;
  const int sq = quad == 1 ? 2 : quad == 2 ? 1 : quad;
  return (m & 16) + sq * 4 + (m & 3);
}

template <int D, int G, int NCB>
__global__ __launch_bounds__(kPfWaves * kWave)
__attribute__((amdgpu_waves_per_eu(PA_PF_WAVES_PER_EU))) void prefill_chunk_kernel(PrefillParams p) {
  using C = PrefillCfg<D>;
  constexpr int COLS = kPfWaves * 32 * NCB;  // columns per workgroup
  constexpr int QT = COLS / G;               // queries per workgroup
  static_assert(COLS % G == 0, "group must divide the column tile");

  __shared__ __attribute__((aligned(16))) char lds[2][C::STAGE];

  // ---- which (request, kv head, query tile): tiles of one (request, kv
  // head) are consecutive in the "logical" order, and logical runs are
  // assigned to one XCD (workgroups go round-robin over the 8 XCDs)
  const int N = p.num_qtiles * p.num_reqs * p.num_kv_heads;
  const int L = blockIdx.x;
  const int xcd = L & 7, slot = L >> 3;
  const int per = N >> 3, rem = N & 7;
  const int logical = xcd * per + min(xcd, rem) + slot;
  const int tile = logical % p.num_qtiles;
  const int pair = logical / p.num_qtiles;
  const int g = pair % p.num_kv_heads;
  const int r = pair / p.num_kv_heads;

  int qs = p.query_start_loc[r];
  int qe = p.query_start_loc[r + 1];
  qs = max(0, min(qs, p.total_q_tokens));
  qe = max(qs, min(qe, p.total_q_tokens));
  const int n_r = qe - qs;
  const int q0 = tile * QT;
  if (q0 >= n_r) return;  // uniform
  const int ctx_cap = p.max_blocks_per_seq * kBlock;
  const int ctx = max(0, min(p.context_lens[r], ctx_cap));
  const int prior = ctx - n_r;  // < 0 only for out-of-contract input
  const int q_end = min(n_r, q0 + QT);
  const int nk = max(0, min(ctx, prior + q_end));  // keys this workgroup needs
  const int iters = (nk + kPfKT - 1) / kPfKT;
  const int nblk = (ctx + kBlock - 1) / kBlock;

  const int tid = threadIdx.x;
  __builtin_assume(tid < kPfWaves * kWave);
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int half = lane >> 5;
  const int cw = lane & 31;
  const int32_t* bt = p.block_tables + (int64_t)r * p.max_blocks_per_seq;

  // Scores are scaled by |scale|; a negative scale is applied by flipping the
  // sign of q, which is exact in bf16.
  const float sl = fabsf(p.scale_log2);
  const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;

  // ---- this lane's columns and their query positions
  int pos[NCB];
  uint4 qf[NCB][C::DS];
  int wave_max_pos = -1, wave_min_pos = 0x7fffffff;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int c = 32 * (w * NCB + cb) + cw;
    const int qi = q0 + c / G;
    const int hh = c % G;
    const bool valid = qi < n_r;
    pos[cb] = valid ? prior + qi : -1;
    const char* qrow = p.q + ((int64_t)(qs + (valid ? qi : 0)) * p.num_q_heads + g * G + hh) * C::RB;
#pragma unroll
    for (int s = 0; s < C::DS; ++s)
    {
      uint4 v = valid ? *(const uint4*)(qrow + (2 * s + half) * 16) : make_uint4(0, 0, 0, 0);
      v.x ^= qsign; v.y ^= qsign; v.z ^= qsign; v.w ^= qsign;
      qf[cb][s] = v;
    }
    // first and last query of this column block (columns are query-major)
    const int qa = q0 + (32 * (w * NCB + cb)) / G;
    const int qb = min(n_r - 1, q0 + (32 * (w * NCB + cb) + 31) / G);
    if (qa < n_r) {
      wave_max_pos = max(wave_max_pos, prior + qb);
      wave_min_pos = min(wave_min_pos, prior + qa);
    }
  }
  if (q0 + (32 * (w * NCB + NCB - 1) + 31) / G >= n_r) wave_min_pos = -1;  // has padding columns

  f32x16_t acco[NCB][C::DB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acco[cb][db][i] = 0.f;
  float m_run[NCB], l_run[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    m_run[cb] = kPfNegBig;
    l_run[cb] = 0.f;
  }

  // ---- global -> register -> LDS staging of one 64-key tile
  // Each (block, kv head) tile is one contiguous run of 16 * RB bytes for K
  // and for V, i.e. TPB 16-byte chunks (256 for D = 128).  Thread t loads
  // chunk t % TPB of block NBP * u + t / TPB for u = 0 .. NKL-1, so every
  // load instruction reads consecutive 16-byte pieces of one tile, and the
  // block a wave loads is known per wave (t / TPB is uniform in a wave).
  constexpr int TPB = kBlock * C::RB / 16;           // chunks per tile
  constexpr int NBP = kPfWaves * kWave / TPB;        // blocks per load pass
  static_assert(TPB % kWave == 0 && C::NKL * NBP == kPfBlocks && C::NVL == C::NKL, "staging map");
  const int jt = tid % TPB;                          // chunk within the tile
  const int bsub = NBP > 1 ? (w * kWave) / TPB : 0;  // uniform: which block of the pass
  uint4 kreg[C::NKL], vreg[C::NVL];
  // Byte offsets of the next tile's four (block, kv head) tiles in the pools
  // (uniform).  A block past the context or an id outside the pool is read
  // from block 0 instead (always in bounds) and flagged in `bad`; its K and
  // V are replaced by zeros before they reach LDS, i.e. it is an empty block.
  //
  // The ids of a tile are loaded one iteration before they are needed, by
  // one vector load (lane l reads block 4 it + l % 4); they are turned into
  // scalar offsets just before the tile's loads are issued, when the load
  // that fetched them has long completed, so no wait on the memory counter
  // ever covers tile loads still in flight.
  constexpr int64_t tile_bytes = (int64_t)kBlock * C::RB;
  const char* kbase0 = p.k_cache + (int64_t)g * tile_bytes;
  const char* vbase0 = p.v_cache + (int64_t)g * tile_bytes;
  const int64_t bstride = (int64_t)p.num_kv_heads * tile_bytes;  // bytes per block
  const unsigned jt16 = (unsigned)jt * 16u;
  int idv = -1;  // lane l: raw id of block 4 * (tile) + l % 4 of the tile being fetched
  auto issue_ids = [&](int it) {
    const int jb = it * kPfBlocks + (lane & (kPfBlocks - 1));
    idv = jb < nblk ? bt[jb] : -1;
  };
  int64_t off0 = 0, off1 = 0, off2 = 0, off3 = 0;
  int bad_inflight = 0;
  static_assert(kPfBlocks == 4, "four block ids per tile");
  auto resolve_ids = [&]() {
    int bad = 0;
    auto one = [&](int b) -> int64_t {
      const int id = __builtin_amdgcn_readlane(idv, b);
      const bool ok = id >= 0 && id < p.num_blocks;
      bad |= ok ? 0 : 1 << b;
      return (int64_t)(ok ? id : 0) * bstride;
    };
    off0 = one(0);
    off1 = one(1);
    off2 = one(2);
    off3 = one(3);
    bad_inflight = bad;
  };
  auto off_of = [&](int b) { return b == 0 ? off0 : b == 1 ? off1 : b == 2 ? off2 : off3; };
  auto global_load = [&]() {
#pragma unroll
    for (int u = 0; u < C::NKL; ++u) {
      const int64_t o = off_of(NBP * u + bsub);
      kreg[u] = *(const uint4*)(kbase0 + o + jt16);
      vreg[u] = *(const uint4*)(vbase0 + o + jt16);
    }
  };
  // LDS destinations of this thread's chunks (block b adds a constant):
  // K chunk jt of block b is key 16 b + jt / KCH, stored in row
  // 16 b + pf_row_key(jt / KCH); V chunk jt is dim jt / 2, keys 8 (jt % 2)..
  const int kst = pf_row_key(jt / C::KCH) * C::KRS + (jt % C::KCH) * 16;
  const int vst = C::K_LDS + (jt >> 1) * C::VRS + (jt & 1) * 16;
  auto lds_store = [&](int it, char* st) {
    // keys past the context hold whatever the pool has (possibly NaN): a
    // zero probability must meet a finite value, so clear them here
    const bool tail = it * kPfKT + kPfKT > ctx;  // uniform
#pragma unroll
    for (int u = 0; u < C::NKL; ++u) {
      const int b = NBP * u + bsub;
      if (bad_inflight & (1 << b)) {  // uniform, rare
        kreg[u] = make_uint4(0, 0, 0, 0);
        vreg[u] = make_uint4(0, 0, 0, 0);
      }
      *(uint4*)(st + kst + b * kBlock * C::KRS) = kreg[u];
      uint4 v = vreg[u];
      if (tail) {
        const int key0 = it * kPfKT + b * kBlock + (jt & 1) * 8;
        uint32_t* wv = (uint32_t*)&v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = key0 + 2 * e;
          wv[e] &= t >= ctx ? 0u : (t + 1 >= ctx ? 0x0000ffffu : 0xffffffffu);
        }
      }
      *(uint4*)(st + vst + b * 32) = v;
    }
  };

  if (iters > 0) {
    issue_ids(0);
    resolve_ids();
    if (iters > 1) issue_ids(1);
    global_load();
    lds_store(0, lds[0]);
  }

  // fragment read bases: K row cw (key pf_row_key(cw)) dims 8 half ..;
  // V row (dim) cw keys 8 half ..
  const int kfr = cw * C::KRS + half * 16;
  const int vfr = C::K_LDS + cw * C::VRS + half * 16;

  // One 64-key tile: S^T = K Q^T, online softmax, O^T += V^T P.  MASK
  // selects the variant for tiles that reach past some column's position
  // (the causal diagonal, the context end or padding columns).
  auto tile_step = [&](const char* st, int k0, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    // The two key blocks' accumulator chains alternate, and the K fragments
    // of step s+1 are read while the products of step s run.
    f32x16_t sacc[NCB][2];
    uint4 ka[2][2];
    auto kfrag = [&](int s, int kb) { return *(const uint4*)(st + kfr + kb * 32 * C::KRS + s * 32); };
    ka[0][0] = kfrag(0, 0);
    ka[0][1] = kfrag(0, 1);
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      if (s + 1 < C::DS) {
        ka[(s + 1) & 1][0] = kfrag(s + 1, 0);
        ka[(s + 1) & 1][1] = kfrag(s + 1, 1);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const f32x16_t zero = {};
          sacc[cb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, ka[s & 1][kb]), __builtin_bit_cast(bf16x8_t, qf[cb][s]),
              s == 0 ? zero : sacc[cb][kb], 0, 0, 0);
        }
    }

    // register i of key block kb is key k0 + 32 kb + 16 (i / 8) + 8 half + i % 8.
    // The max is taken on raw scores (the scale is >= 0 here); scale and max
    // are then applied in one fma per score.  In masked tiles a hidden key's
    // probability is selected to zero, which also discards any NaN from a
    // poisoned slot past the context.
    bf16x8_t pf[NCB][2][2];
    float nm[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      auto visible = [&](int kb, int i) {
        return k0 + 32 * kb + 16 * (i >> 3) + 8 * half + (i & 7) <= pos[cb];
      };
      float mraw = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = sacc[cb][kb][i];
          mraw = fmaxf(mraw, (MASK && !visible(kb, i)) ? -INFINITY : v);
        }
      mraw = fmaxf(mraw, xor_lane<32>(mraw));
      const float mx = mraw == -INFINITY ? -INFINITY : mraw * sl;
      if (__builtin_amdgcn_ballot_w64(mx > m_run[cb] + kPfGap)) {
        const float m_new = fmaxf(m_run[cb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[cb] - m_new);
        m_run[cb] = m_new;
        l_run[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acco[cb][db][i] *= alpha;
      }
      nm[cb] = -m_run[cb];
    }

    // probabilities of key block kb -> bf16 B operands; then O^T += V^T P for
    // that block.  Block 0's products are issued before block 1's
    // exponentials so that the matrix cores and the VALU overlap.
    auto probs = [&](int kb) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        float lsum = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          uint32_t wds[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i0 = 8 * t + 2 * e;
            float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[cb][kb][i0], sl, nm[cb]));
            float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[cb][kb][i0 + 1], sl, nm[cb]));
            if (MASK) {
              const int lim = pos[cb] - (k0 + 32 * kb + 16 * t + 8 * half);
              p0 = 2 * e <= lim ? p0 : 0.f;
              p1 = 2 * e + 1 <= lim ? p1 : 0.f;
            }
            wds[e] = pack_bf16(p0, p1);
            // the sum runs over the bf16 weights the P V product applies
            lsum = dot2_bf16(wds[e], 0x3f803f80u, lsum);
          }
          pf[cb][kb][t] = __builtin_bit_cast(bf16x8_t, make_uint4(wds[0], wds[1], wds[2], wds[3]));
        }
        l_run[cb] += lsum;
      }
    };
    // the DB output chains alternate; V fragments are read one step ahead
    auto vfrag = [&](int kb, int t, int db) {
      return *(const uint4*)(st + vfr + 32 * db * C::VRS + (4 * kb + 2 * t) * 16);
    };
    auto pv = [&](int kb) {
      uint4 va[2][C::DB];
#pragma unroll
      for (int db = 0; db < C::DB; ++db) va[0][db] = vfrag(kb, 0, db);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (t == 0) {
#pragma unroll
          for (int db = 0; db < C::DB; ++db) va[1][db] = vfrag(kb, 1, db);
        }
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            acco[cb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, va[t][db]), pf[cb][kb][t], acco[cb][db], 0, 0, 0);
      }
    };
    probs(0);
    pv(0);
    probs(1);
    pv(1);
#if PA_PF_SCHED == 1
    // exponentials of block 1 between the products of block 0
#pragma unroll
    for (int i = 0; i < 2 * C::DB * NCB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
    }
#endif
  };

  // One pipelined iteration: wait for tile it in LDS, start the global
  // loads of tile it+1, compute tile it, then park tile it+1 in the other
  // LDS buffer.  Every wave of the workgroup runs every iteration.
  auto iteration = [&](int it, auto mask_c) {
    __syncthreads();
    if (it + 1 < iters) {
      resolve_ids();                      // tile it+1 (ids loaded last iteration)
      if (it + 2 < iters) issue_ids(it + 2);
      global_load();
    }
    const int k0 = it * kPfKT;
    if (k0 <= wave_max_pos)  // uniform: some column of this wave sees a key here
      tile_step(lds[it & 1], k0, mask_c);
    if (it + 1 < iters) lds_store(it + 1, lds[(it + 1) & 1]);
  };
  // Tiles that end before the workgroup's first query position need no
  // mask for any column; the rest (the causal diagonal, the context end and
  // padding columns) take the masked variant.  Two plain loops keep the
  // accumulators in fixed registers across iterations.
  const int wg_min_pos = prior + q0;
  const int n_plain = wg_min_pos >= 0 ? min(iters, (wg_min_pos + 1) / kPfKT) : 0;
  for (int it = 0; it < n_plain; ++it) iteration(it, std::false_type{});
  for (int it = n_plain; it < iters; ++it) iteration(it, std::true_type{});

  // ---- normalise and store: register i of dim block db is dim
  // 32 db + 8 (i / 4) + 4 half + i % 4 of this lane's column
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const float lt = l_run[cb] + xor_lane<32>(l_run[cb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int c = 32 * (w * NCB + cb) + cw;
    const int qi = q0 + c / G;
    if (qi >= n_r) continue;
    char* orow = (char*)p.out + ((int64_t)(qs + qi) * p.num_q_heads + g * G + c % G) * C::RB;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x16_t& a = acco[cb][db];
        uint2 v;
        v.x = pack_bf16(a[4 * i4 + 0] * inv, a[4 * i4 + 1] * inv);
        v.y = pack_bf16(a[4 * i4 + 2] * inv, a[4 * i4 + 3] * inv);
        *(uint2*)(orow + (32 * db + 8 * i4 + 4 * half) * 2) = v;
      }
  }
}

template <int D, int G>
static hipError_t launch_prefill_t(const PrefillParams& prm, hipStream_t stream) {
  constexpr int NCB = PA_PF_NCB;
  const int64_t grid = (int64_t)prm.num_qtiles * prm.num_reqs * prm.num_kv_heads;
  hipLaunchKernelGGL((prefill_chunk_kernel<D, G, NCB>), dim3((unsigned)grid),
                     dim3(kPfWaves * kWave), 0, stream, prm);
  return hipGetLastError();
}

int prefill_queries_per_tile(int group) { return kPfWaves * 32 * PA_PF_NCB / group; }

bool prefill_supported(int elem_bytes, int head_dim, int group) {
  return elem_bytes == 2 && (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_prefill(const PrefillArgs& a, const CacheGeom& g, hipStream_t stream) {
  PrefillParams p;
  p.out = a.out;
  p.q = (const char*)a.q;
  p.k_cache = (const char*)a.k_cache;
  p.v_cache = (const char*)a.v_cache;
  p.block_tables = a.block_tables;
  p.query_start_loc = a.query_start_loc;
  p.context_lens = a.context_lens;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.num_reqs = a.num_reqs;
  p.total_q_tokens = a.total_q_tokens;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = g.num_kv_heads;
  p.num_blocks = g.num_blocks;
  p.scale_log2 = a.scale * kLog2e;
  const int G = a.num_q_heads / g.num_kv_heads;
  const int qt = prefill_queries_per_tile(G);
  p.num_qtiles = (a.max_q_len + qt - 1) / qt;

#define PA_PREFILL_CASE(D_, G_) \
  if (g.head_dim == D_ && G == G_) return launch_prefill_t<D_, G_>(p, stream);
  PA_PREFILL_CASE(128, 1) PA_PREFILL_CASE(128, 2) PA_PREFILL_CASE(128, 4) PA_PREFILL_CASE(128, 8)
  PA_PREFILL_CASE(64, 1) PA_PREFILL_CASE(64, 2) PA_PREFILL_CASE(64, 4) PA_PREFILL_CASE(64, 8)
#undef PA_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace pa
