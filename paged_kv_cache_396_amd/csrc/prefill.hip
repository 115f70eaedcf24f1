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
//  * one workgroup of 8 waves (two per SIMD) per (request, kv head, tile of
//    query rows).  A "column" is one (query, q head) pair; the G q heads of
//    the kv head and QT consecutive queries give 256 columns, 32 per wave.
//    Workgroup ids are mapped so that all tiles of one (request, kv head)
//    run on the same XCD and share its L2 copy of the K/V tiles.
//  * the workgroup walks the keys 64 at a time (four 16-token blocks).  The
//    pool tiles are copied straight into LDS by buffer loads that write LDS
//    (no registers, no LDS store instructions), into a ring of four stages,
//    so the loads of a tile are issued three iterations before it is used.
//    Each wave copies one block of every tile; a block past the context or
//    with an id outside the pool is an empty buffer range.  V values of keys
//    past the context are cleared in registers in the tile that holds the
//    context end.
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16 (32 keys x 32 columns per instruction), so
//    each lane holds one column's scores for 16 keys and the row max of the
//    softmax needs a single exchange between the two lane halves.  The MFMA
//    row -> key assignment is permuted so that the 8 fp32 scores a lane holds
//    for one 16-key step are 8 consecutive keys: after conversion to bf16
//    they are directly the B operand of the P V product.
//  * each 64-key tile is taken as two 32-key blocks, each a full online
//    softmax step, so that one block's vector work can overlap the other
//    block's matrix products.  When a request's rows fill at most half of a
//    narrow workgroup's columns (speculative verification), two waves share
//    each column block and take one 32-key block each; their states are
//    merged with the online-softmax rescale at the end.
//  * O^T = V^T P accumulates in fp32 (32 dims x 32 columns per instruction);
//    the V tiles are dim-major in the pool and in LDS, so each A fragment is
//    one 16-byte read.
//  * LDS rows are unpadded; 16-byte chunks are XOR-swizzled within a row so
//    that the 16 rows one fragment read touches fall on distinct banks.
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
#define PA_PF_WAVES 8
#endif
#ifndef PA_PF_STAGES
#define PA_PF_STAGES 4
#endif

constexpr int kPfWaves = PA_PF_WAVES;    // waves per workgroup
constexpr int kPfStages = PA_PF_STAGES;  // LDS ring depth (tiles)
constexpr int kPfKT = 64;                // keys per iteration (four 16-token blocks)
constexpr int kPfBlocks = kPfKT / kBlock;
constexpr float kPfGap = 8.0f;           // log2 units a score may exceed the reference max
constexpr float kPfNegBig = -FLT_MAX;
constexpr int kPfDma = 1024;             // bytes one LDS-writing load instruction moves
// Narrow shape for chunks of a few query rows (speculative verification,
// shared-prefix groups): with 4 waves and 2 stages a workgroup needs half
// the LDS, so two share a compute unit and twice as many waves compute.
// With at most 64 columns it runs paired (two waves per column block).
constexpr int kPfNarrowWaves = 4;
constexpr int kPfNarrowStages = 2;

// KB: bytes of a pool element, 2 (bf16) or 1 (fp8 E4M3 codes, widened to
// bf16 in registers after the LDS read).
template <int D, int W = kPfWaves, int KB = 2>
struct PrefillCfg {
  static constexpr int QRB = D * 2;            // bytes of one q / out row (bf16)
  static constexpr int RB = D * KB;            // bytes of one K row in the pool
  static constexpr int KCH = RB / 16;          // 16-byte chunks per K row
  static constexpr int DS = D / 16;            // k-steps of S^T = K Q^T (16 dims each)
  static constexpr int DB = D / 32;            // 32-dim blocks of O^T
  static constexpr int BLK = kBlock * RB;      // one pool tile (block, kv head) of K or V
  static constexpr int TILE = kPfBlocks * BLK;  // K or V of one 64-key tile in LDS
  static constexpr int DPB = BLK / kPfDma;     // load instructions per pool tile
  static constexpr int WPB = W / kPfBlocks;    // waves sharing one block
  static constexpr int QPW = DPB / WPB;        // K (and V) instructions per wave per tile
  static constexpr int RPI = kPfDma / RB;      // K rows one instruction fills
  static_assert(W % kPfBlocks == 0, "whole waves per block");
  static_assert(QPW >= 1 && QPW * WPB == DPB, "load split");
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
  float v_scale;  // fp8 pools: applied with the final normalisation
  // shared-prefix mode only: group p's sequences p * group_size .. are the
  // queries; the workgroup covers prefix partition j (prefix_partition keys)
  // and leaves its partial state in slot row * ws_stride + j
  const int32_t* prefix_lens;
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int group_size;
  int prefix_partition;
  int prefix_parts;  // grid extent (partitions of the longest prefix)
  int ws_stride;
  // split chunk mode (max_parts > 1): workgroup (tile, request, kv head,
  // part) covers keys [part * part_keys, +part_keys) of its tile's need;
  // tiles needing more than one part leave partial states in slot
  // row * ws_stride + part (ws_stride = max_parts) for prefill_merge_kernel
  int part_keys;
  int max_parts;
  int qt;  // queries per tile of the launched variant
};

// Keys a query tile of request r needs (the chunk's rows up to q_end see
// keys 0 .. prior + q_end - 1), clamped to the context and, when split, to
// the grid's parts.
__device__ inline int pf_tile_keys(int ctx, int prior, int q_end) {
  return max(0, min(ctx, prior + q_end));
}

// Row order of a 16-key block in LDS: row m holds key pf_key16(m), i.e. the
// rows of quads 1 and 2 are swapped.  With this order the accumulator
// registers 8t..8t+7 of lane l of S^T = K Q^T hold keys 16t + 8(l/32) + 0..7.
// The permutation is its own inverse.
__device__ inline int pf_key16(int m) {
  const int quad = (m >> 2) & 3;
  const int sq = quad == 1 ? 2 : quad == 2 ? 1 : quad;
  return (m & ~12) | (sq << 2);
}

// Chunk swizzle of K row m in LDS: chunk c sits at slot c ^ pf_ksw(m).  The
// 16 rows a fragment read touches at one chunk then cover all 16 bank
// groups of 16 bytes (rows of 256 bytes: slot = c ^ m; rows of 128 bytes:
// two rows per 256 bytes, slot = c ^ (m / 2)).
template <int RB>
__device__ inline int pf_ksw(int m) {
  return RB == 256 ? (m & 15) : ((m >> 1) & 7);
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (export and LDS counters left alone).
__host__ __device__ constexpr int pf_vmcnt(int n) {
  return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
}

typedef int pf_rsrc __attribute__((ext_vector_type(4)));

__device__ inline unsigned pf_lds_addr(const char* p) {
  return __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p);
}

// One 1 KiB piece from a buffer range into LDS: lane l's 16 bytes at byte
// offset voff of the range land at LDS address lds + 16 l (zeros when voff
// is past the range).  Written as assembly so that the compiler, which
// cannot see the copy, adds no waits of its own: the consumer waits on the
// vector-memory counter and a barrier before reading the stage.  M0 carries
// the LDS address and is not used by the compiler between these
// statements (nothing in this kernel needs it).
__device__ inline void pf_copy_to_lds(const pf_rsrc& rs, unsigned lds, int voff) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  __asm__ volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :
                   : "s"(lds), "v"(voff), "s"(rs)
                   : "memory", "m0");
#pragma clang diagnostic pop
}

// PFX: shared-prefix mode.  The queries are the newest tokens of the
// group_size sequences of one group (all G heads of one kv head), every
// query sees every key of the partition (they all sit past the prefix), and
// the result is a partial state (running max in log2 units, sum, unscaled
// output) for the decode merge instead of a normalised row.
template <int D, int G, int NCB, bool PFX = false, int W = kPfWaves, int S = kPfStages, int KB = 2,
          bool KS = false>
__global__ __launch_bounds__(W * kWave)
__attribute__((amdgpu_waves_per_eu(PA_PF_WAVES_PER_EU))) void prefill_chunk_kernel(PrefillParams p) {
  using C = PrefillCfg<D, W, KB>;
  // CVT (fp8 pools, wide shape): each tile is widened to bf16 once, by all
  // waves together, into an LDS buffer laid out as a bf16 tile; the
  // fragment reads then follow the bf16 path.  CR and KBR describe what the
  // fragment reads see.
  constexpr bool CVT = KB == 1 && W == 8 && !KS;
  constexpr int KBR = CVT ? 2 : KB;
  using CR = PrefillCfg<D, W, KBR>;
  // KS (paired waves): waves 2 i and 2 i + 1 share column block i and take
  // the first and the second 32-key block of every tile, each with its own
  // online-softmax state; the two states are merged at the end.
  constexpr int CW = KS ? W / 2 : W;  // waves with distinct columns
  constexpr int COLS = CW * 32 * NCB;  // columns per workgroup
  constexpr int QT = COLS / G;        // queries per workgroup
  static_assert(S == 2 || S == 4, "stage count: even, and a power of two");
  static_assert(COLS % G == 0, "group must divide the column tile");

  // The ring: each stage holds the K tile, then the V tile.  A stage is
  // named by a compile-time index (inside the unrolled rounds) or by the
  // tile number (the single iterations around them: one body for all
  // stages, so the compiler keeps one register assignment for O instead of
  // one per stage joined by copies of the whole accumulator).
  __shared__ __attribute__((aligned(1024))) char ring[S][2 * C::TILE];
  auto stage = [&](auto J) -> char* {
    if constexpr (std::is_same_v<decltype(J), int>) return ring[J & (S - 1)];
    else return ring[decltype(J)::value % S];
  };
  auto kstage = [&](auto J) -> char* { return stage(J); };
  auto vstage = [&](auto J) -> char* { return stage(J) + C::TILE; };
  // widened tiles (CVT): tile t in buffer t % 2, K then V
  __shared__ __attribute__((aligned(1024))) char cvb[CVT ? 2 : 1][CVT ? 2 * CR::TILE : 16];
  auto rkstage = [&](auto J, int t) -> const char* {
    if constexpr (CVT) return cvb[t & 1];
    else return kstage(J);
  };
  auto rvstage = [&](auto J, int t) -> const char* {
    if constexpr (CVT) return cvb[t & 1] + CR::TILE;
    else return vstage(J);
  };

  // ---- which queries and which keys.  Chunk mode: (request, kv head, query
  // tile); tiles of one (request, kv head) are consecutive in the "logical"
  // order, and logical runs are assigned to one XCD (workgroups go
  // round-robin over the 8 XCDs).  Shared-prefix mode: (group, kv head,
  // prefix partition).
  const int L = blockIdx.x;
  int g, r, qs, n_r, q0, ctx, kbeg, nk, part = 0, prior;
  bool partial = PFX;  // leaves a partial state instead of a normalised row
  if constexpr (!PFX) {
    const int N = p.num_qtiles * p.num_reqs * p.num_kv_heads * p.max_parts;
    const int xcd = L & 7, slot = L >> 3;
    const int per = N >> 3, rem = N & 7;
    const int logical = xcd * per + min(xcd, rem) + slot;
    const int tile = logical % p.num_qtiles;
    const int rest = logical / p.num_qtiles;
    part = rest % p.max_parts;
    const int pair = rest / p.max_parts;
    g = pair % p.num_kv_heads;
    r = pair / p.num_kv_heads;
    qs = p.query_start_loc[r];
    int qe = p.query_start_loc[r + 1];
    qs = max(0, min(qs, p.total_q_tokens));
    qe = max(qs, min(qe, p.total_q_tokens));
    n_r = qe - qs;
    q0 = tile * QT;
    if (q0 >= n_r) return;  // uniform
    const int ctx_cap = min(p.max_blocks_per_seq * kBlock, p.max_parts * p.part_keys);
    ctx = max(0, min(p.context_lens[r], ctx_cap));
    prior = ctx - n_r;  // < 0 only for out-of-contract input
    const int q_end = min(n_r, q0 + QT);
    nk = pf_tile_keys(ctx, prior, q_end);  // keys this tile needs
    kbeg = part * p.part_keys;
    if (p.max_parts > 1) {
      if (kbeg >= nk && part > 0) return;  // uniform
      partial = nk > p.part_keys;          // the tile needs more than one part
      nk = min(nk, kbeg + p.part_keys);
    }
  } else {
    part = L % p.prefix_parts;
    const int pair = L / p.prefix_parts;
    g = pair % p.num_kv_heads;
    const int grp = pair / p.num_kv_heads;
    r = grp * p.group_size;  // its first sequence holds the shared block table
    qs = r;
    n_r = p.group_size;
    q0 = 0;
    const int cap = min(p.max_blocks_per_seq * kBlock, p.prefix_parts * p.prefix_partition);
    const int pl = max(0, min(p.prefix_lens[grp], cap)) & ~(kBlock - 1);
    kbeg = part * p.prefix_partition;
    if (kbeg >= pl) return;  // uniform
    ctx = min(pl, kbeg + p.prefix_partition);  // keys past ctx belong elsewhere
    nk = ctx;
    prior = ctx - 1;  // every query sees every key of the partition
  }
  const int iters = (nk - kbeg + kPfKT - 1) / kPfKT;
  const int nblk = (ctx + kBlock - 1) / kBlock;

  const int tid = threadIdx.x;
  __builtin_assume(tid < W * kWave);
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wc = KS ? w >> 1 : w;  // column block of this wave
  const int kbw = KS ? w & 1 : 0;  // its key block (paired waves)
  const int half = lane >> 5;
  const int cw = lane & 31;
  // block ids are read through the scalar cache (uniform addresses)
  const __attribute__((address_space(4))) int32_t* bt =
      (const __attribute__((address_space(4))) int32_t*)(p.block_tables + (int64_t)r * p.max_blocks_per_seq);

  // Scores are scaled by |scale|; a negative scale is applied by flipping the
  // sign of q, which is exact in bf16.
  // A zero scale becomes the smallest normal one: every scaled score and
  // max then rounds away in the exponent and the softmax stays uniform,
  // and -inf times the scale stays -inf, so the max needs no guard.
  const float sl = fmaxf(fabsf(p.scale_log2), FLT_MIN);
  const uint32_t qsign = p.scale_log2 < 0.f ? 0x80008000u : 0u;

  // ---- this lane's columns and their query positions
  int pos[NCB];
  uint4 qf[NCB][C::DS];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int c = 32 * (wc * NCB + cb) + cw;
    const int qi = q0 + c / G;
    const int hh = c % G;
    const bool valid = qi < n_r;
    pos[cb] = valid ? (PFX ? prior : prior + qi) : -1;
    const char* qrow = p.q + ((int64_t)(qs + (valid ? qi : 0)) * p.num_q_heads + g * G + hh) * C::QRB;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      // k-step s, lane half h: dims 16 s + 8 h .. (bf16 pools); with fp8
      // pools the dims follow the 16-code chunks a lane reads, 32 (s / 2) +
      // 16 h + 8 (s % 2) .. (the same order on both sides of the product)
      const int qoff = KBR == 2 ? (2 * s + half) * 16 : 64 * (s >> 1) + 32 * half + 16 * (s & 1);
      uint4 v = valid ? *(const uint4*)(qrow + qoff) : make_uint4(0, 0, 0, 0);
      v.x ^= qsign; v.y ^= qsign; v.z ^= qsign; v.w ^= qsign;
      qf[cb][s] = v;
    }
  }

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

  // ---- pool -> LDS copies.  Wave w copies block w / WPB of every tile: the
  // QPW 1 KiB pieces isub .. isub+QPW-1 of its K tile and of its V tile.
  // Each lane's source offset inside the pool tile is fixed; the LDS side of
  // a piece is 64 consecutive 16-byte slots (lane order).
  //  * K piece i fills rows RPI i .. of the block (LDS row m holds key
  //    pf_key16(m)); slot j of row m receives chunk j ^ pf_ksw(m).
  //  * V piece i fills slots 64 i .. of the dim-major block (32 bytes per
  //    dim); slot j of dim x receives chunk j ^ ((x / 8) % 2).  fp8 pools:
  //    16 bytes per dim, copied in order.
  const int bsub = w / C::WPB;
  const int isub = (w % C::WPB) * C::QPW;
  int kvo[C::QPW], vvo[C::QPW];
#pragma unroll
  for (int u = 0; u < C::QPW; ++u) {
    const int i = isub + u;
    const int m = C::RPI * i + lane / C::KCH;
    const int kc = (lane % C::KCH) ^ pf_ksw<C::RB>(m);
    kvo[u] = pf_key16(m) * C::RB + kc * 16;
    const int sp = 64 * i + lane;
    if constexpr (KB == 2) {
      const int x = sp >> 1;
      const int vc = (sp & 1) ^ ((x >> 3) & 1);
      vvo[u] = x * 32 + vc * 16;
    } else {
      vvo[u] = sp * 16;
    }
  }
  const int64_t bstride = (int64_t)p.num_kv_heads * C::BLK;  // bytes per pool block
  // id of this wave's block of tile n; -1 past the keys this workgroup needs
  auto block_id = [&](int n) __attribute__((always_inline)) {
    const int jb = kbeg / kBlock + n * kPfBlocks + bsub;
    return n < iters && jb < nblk ? bt[jb] : -1;
  };
  // Buffer ranges of this wave's pool tiles of tile n.  An empty range (a
  // block past the context, or an id outside the pool) reads as zeros; K
  // rows past the context read as zeros too.
  auto range = [&](const char* pool, int id, int bytes) __attribute__((always_inline)) {
    const bool ok = id >= 0 && id < p.num_blocks;
    const uint64_t base = (uint64_t)(pool + (ok ? (int64_t)id * bstride : 0) + (int64_t)g * C::BLK);
    pf_rsrc rs;
    rs.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    rs.y = __builtin_amdgcn_readfirstlane((int)((base >> 32) & 0xffffu));  // stride 0
    rs.z = __builtin_amdgcn_readfirstlane(ok ? bytes : 0);
    rs.w = 0x00020000;
    return rs;
  };
  // LDS offset of piece u inside a K or V tile
  auto piece_off = [&](int u) { return bsub * C::BLK + (isub + u) * kPfDma; };
  auto copy_k = [&](char* stage, int id, int n) __attribute__((always_inline)) {
    const int rows = min(kBlock, ctx - (kbeg / kBlock + n * kPfBlocks + bsub) * kBlock);
    const pf_rsrc rk = range(p.k_cache, id, rows * C::RB);
#pragma unroll
    for (int u = 0; u < C::QPW; ++u) pf_copy_to_lds(rk, pf_lds_addr(stage + piece_off(u)), kvo[u]);
  };
  auto copy_v = [&](char* stage, int id) __attribute__((always_inline)) {
    const pf_rsrc rv = range(p.v_cache, id, C::BLK);
#pragma unroll
    for (int u = 0; u < C::QPW; ++u) pf_copy_to_lds(rv, pf_lds_addr(stage + piece_off(u)), vvo[u]);
  };
  constexpr int kLoadsPerBatch = 2 * C::QPW;  // vector-memory instructions per batch
  // wait until this wave has at most n batches in flight, then meet the
  // workgroup: every wave's copies of the older batches are then in LDS
  auto stage_barrier = [&](auto n_c) __attribute__((always_inline)) {
    constexpr int n = decltype(n_c)::value;
    __asm__ volatile("" ::: "memory");
    if constexpr (CVT)
      __builtin_amdgcn_s_waitcnt(pf_vmcnt(n * kLoadsPerBatch) & ~(15 << 8));  // and LDS writes done
    else
      __builtin_amdgcn_s_waitcnt(pf_vmcnt(n * kLoadsPerBatch));
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  };

  // fragment read bases.  K: MFMA row cw of key block kb is row cw % 16 of
  // LDS block 2 kb + cw / 16; its chunk 2 s + half sits at slot
  // (2 s + half) ^ sw, so the address of step s is kfb ^ (32 s).  V: dim
  // 32 db + cw of 16-key step st, keys 8 half ..
  const int ksw = pf_ksw<CR::RB>(cw & 15);
  const int kfb = (cw >> 4) * CR::BLK + (cw & 15) * CR::RB + 16 * (half ^ (ksw & 1)) + 32 * (ksw >> 1);
  // the K fragment address of every k-step, kept in registers for the
  // whole loop (an XOR cannot go into the read's offset field)
  int kfs[C::DS];
#pragma unroll
  for (int st = 0; st < C::DS; ++st) {
    kfs[st] = kfb ^ (st * 32);
    __asm__ volatile("" : "+v"(kfs[st]));
  }
  // fp8 V: dim 32 db + cw, keys 8 half .. of a block are 8 bytes at
  // (32 db + cw) * 16 + 8 half
  const int vfb = KBR == 2 ? cw * 32 + 16 * (half ^ ((cw >> 3) & 1)) : cw * 16 + 8 * half;

  // The tile is processed as two 32-key blocks, each a full online-softmax
  // step, so that the vector work of one block overlaps the matrix products
  // of the other: the scores of block 1 run while block 0's exponentials are
  // evaluated, and block 0's P V products run while block 1's are.

  // S^T = K Q^T for key block kb (a chain of DS products); each K fragment
  // is read three products ahead of its use.
#ifndef PA_PF_AHEAD
#define PA_PF_AHEAD 3
#endif
  constexpr int kPfAhead = PA_PF_AHEAD;
  auto scores = [&](const char* st, int kb, f32x16_t (&sacc)[NCB]) __attribute__((always_inline)) {
    auto kfrag = [&](int s) { return *(const uint4*)(st + kb * 2 * CR::BLK + kfs[s]); };
    if constexpr (KBR == 1) {
      // one 16-code chunk per lane feeds two k-steps once widened to bf16
      constexpr int NP = C::DS / 2;
      uint4 ka[2];
      ka[0] = kfrag(0);
#pragma unroll
      for (int sp = 0; sp < NP; ++sp) {
        if (sp + 1 < NP) ka[(sp + 1) & 1] = kfrag(sp + 1);
        const uint4 raw = ka[sp & 1];
        const uint4 w0 = make_uint4(fp8x2_to_bf16x2<false>(raw.x), fp8x2_to_bf16x2<true>(raw.x),
                                    fp8x2_to_bf16x2<false>(raw.y), fp8x2_to_bf16x2<true>(raw.y));
        const uint4 w1 = make_uint4(fp8x2_to_bf16x2<false>(raw.z), fp8x2_to_bf16x2<true>(raw.z),
                                    fp8x2_to_bf16x2<false>(raw.w), fp8x2_to_bf16x2<true>(raw.w));
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const f32x16_t zero = {};
          sacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, w0), __builtin_bit_cast(bf16x8_t, qf[cb][2 * sp]),
              sp == 0 ? zero : sacc[cb], 0, 0, 0);
          sacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, w1), __builtin_bit_cast(bf16x8_t, qf[cb][2 * sp + 1]),
              sacc[cb], 0, 0, 0);
        }
      }
      return;
    }
    uint4 ka[kPfAhead + 1];
#pragma unroll
    for (int s = 0; s < kPfAhead; ++s) ka[s] = kfrag(s);
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      if (s + kPfAhead < C::DS) ka[(s + kPfAhead) % (kPfAhead + 1)] = kfrag(s + kPfAhead);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const f32x16_t zero = {};
        sacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, ka[s % (kPfAhead + 1)]), __builtin_bit_cast(bf16x8_t, qf[cb][s]),
            s == 0 ? zero : sacc[cb], 0, 0, 0);
      }
    }
  };

  // One online-softmax step over key block kb (keys k0 + 32 kb ..).
  // Register i is key k0 + 32 kb + 16 (i / 8) + 8 half + i % 8.  The
  // reference max m_run is raised only when a score exceeds it by more than
  // kPfGap; the factor alpha that brings earlier sums to the new max is
  // returned (exactly 1 when the max stays), and l_run is updated here, O
  // by rescale() before this block's P V products.  The max is taken on raw
  // scores (the scale is >= 0 here); scale and max are then applied in one
  // fma per score.  In masked tiles a hidden key's probability is selected
  // to zero, which also discards any NaN from a poisoned slot past the
  // context.
  bf16x8_t pf[NCB][2][2];
  auto softmax = [&](const f32x16_t (&sacc)[NCB], int k0, int kb, auto mask_c, float (&alpha)[NCB],
                     bool (&raised)[NCB])
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      auto visible = [&](int i) { return k0 + 32 * kb + 16 * (i >> 3) + 8 * half + (i & 7) <= pos[cb]; };
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = (MASK && !visible(i)) ? -INFINITY : sacc[cb][i];
      // max as a tree (short dependency chain).  The NaN-propagating
      // maximum needs no quieting of its inputs (three-input v_maximum3);
      // no NaN reaches it that would not reach the row anyway.
      auto mx3 = [](float a, float b, float c) {
        return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
      };
      float t5[6];
#pragma unroll
      for (int i = 0; i < 5; ++i) t5[i] = mx3(v[3 * i], v[3 * i + 1], v[3 * i + 2]);
      t5[5] = v[15];
      float mraw = __builtin_elementwise_maximum(mx3(t5[0], t5[1], t5[2]), mx3(t5[3], t5[4], t5[5]));
      // the two lane halves hold the two 8-key halves of every 16 keys
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mraw), __float_as_uint(mraw),
                                                        false, false);
      mraw = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const float mx = mraw * sl;
      const bool up = mx > m_run[cb] + kPfGap;
      raised[cb] = up;
      const float m_new = up ? mx : m_run[cb];
      alpha[cb] = up ? __builtin_amdgcn_exp2f(m_run[cb] - m_new) : 1.f;
      m_run[cb] = m_new;
      const float nm = -m_new;
      // two sum chains; the first starts from the earlier sum brought to
      // the new max
      float lsum0 = l_run[cb] * alpha[cb], lsum1 = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint32_t wds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i0 = 8 * t + 2 * e;
          float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[cb][i0], sl, nm));
          float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[cb][i0 + 1], sl, nm));
          if (MASK) {
            const int lim = pos[cb] - (k0 + 32 * kb + 16 * t + 8 * half);
            p0 = 2 * e <= lim ? p0 : 0.f;
            p1 = 2 * e + 1 <= lim ? p1 : 0.f;
          }
          wds[e] = pack_bf16(p0, p1);
          // the sum runs over the bf16 weights the P V product applies
          if (e & 1)
            lsum1 = dot2_bf16(wds[e], 0x3f803f80u, lsum1);
          else
            lsum0 = dot2_bf16(wds[e], 0x3f803f80u, lsum0);
        }
        pf[cb][kb][t] = __builtin_bit_cast(bf16x8_t, make_uint4(wds[0], wds[1], wds[2], wds[3]));
      }
      l_run[cb] = lsum0 + lsum1;
    }
  };
  // O *= alpha before a block's P V products (rare: only when the max rose)
  auto rescale = [&](const float (&alpha)[NCB], const bool (&raised)[NCB]) __attribute__((always_inline)) {
    bool any = false;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) any = any || raised[cb];
    if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acco[cb][db][i] *= alpha[cb];
    }
  };
  // O^T += V^T P for key block kb: the DB output chains alternate; each V
  // fragment is read three products ahead of its use.  In the tile holding the
  // context end the V values of keys past it (whatever the pool holds there,
  // possibly NaN) are cleared in the fragment: a zero probability must meet
  // a finite value.
  auto pv = [&](const char* st, int vf, int k0, int kb, auto mask_c) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr int NJ = 2 * C::DB;  // product j: 16-key step 2 kb + j / DB, dim block j % DB
    auto vfrag = [&](int j) {
      const int step = 2 * kb + j / C::DB, db = j % C::DB;
      if constexpr (KBR == 2) return *(const uint4*)(st + step * CR::BLK + db * 32 * 32 + vf);
      const uint2 raw = *(const uint2*)(st + step * CR::BLK + db * 32 * 16 + vf);
      return make_uint4(fp8x2_to_bf16x2<false>(raw.x), fp8x2_to_bf16x2<true>(raw.x),
                        fp8x2_to_bf16x2<false>(raw.y), fp8x2_to_bf16x2<true>(raw.y));
    };
    const bool tail = MASK && k0 + kPfKT > ctx;  // uniform
    uint4 va[kPfAhead + 1];
#pragma unroll
    for (int j = 0; j < kPfAhead; ++j) va[j] = vfrag(j);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j + kPfAhead < NJ) va[(j + kPfAhead) % (kPfAhead + 1)] = vfrag(j + kPfAhead);
      const int t = j / C::DB, db = j % C::DB, step = 2 * kb + t;
      uint4 f = va[j % (kPfAhead + 1)];
      if constexpr (MASK) {
        if (tail) {
          const int lim = ctx - (k0 + 16 * step + 8 * half);  // keys e < lim are real
          auto keep = [&](int e) { return lim > e + 1 ? 0xffffffffu : (lim > e ? 0x0000ffffu : 0u); };
          f.x &= keep(0);
          f.y &= keep(2);
          f.z &= keep(4);
          f.w &= keep(6);
        }
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acco[cb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, f), pf[cb][kb][t], acco[cb][db], 0, 0, 0);
    }
  };

  // CVT: widen the codes of the fp8 tile in stage st8 into the bf16 buffer
  // dst.  Lane (w, l) takes K chunk 64 w + l (16 codes of one key row) and
  // V row 64 w + l (16 keys of one dim), and writes them where the bf16
  // tile's copies would have put them (same row order and swizzles).
  auto convert = [&](const char* st8, char* dst) __attribute__((always_inline)) {
    static_assert(!CVT || (D == 128 && W * kWave == 512), "one K chunk and one V row per lane");
    const int id = w * kWave + lane;
    const int b = id >> 7;  // block of the tile
    {
      const int m = (id >> 3) & 15, c = id & 7;  // K row, 16-code chunk
      const uint4 raw = *(const uint4*)(st8 + b * C::BLK + m * C::RB + 16 * (c ^ pf_ksw<C::RB>(m)));
      const uint4 w0 = make_uint4(fp8x2_to_bf16x2<false>(raw.x), fp8x2_to_bf16x2<true>(raw.x),
                                  fp8x2_to_bf16x2<false>(raw.y), fp8x2_to_bf16x2<true>(raw.y));
      const uint4 w1 = make_uint4(fp8x2_to_bf16x2<false>(raw.z), fp8x2_to_bf16x2<true>(raw.z),
                                  fp8x2_to_bf16x2<false>(raw.w), fp8x2_to_bf16x2<true>(raw.w));
      const int sw = pf_ksw<CR::RB>(m);
      char* row = dst + b * CR::BLK + m * CR::RB;
      *(uint4*)(row + 16 * ((2 * c) ^ sw)) = w0;
      *(uint4*)(row + 16 * ((2 * c + 1) ^ sw)) = w1;
    }
    {
      const int x = id & 127;  // dim
      const uint4 raw = *(const uint4*)(st8 + C::TILE + b * C::BLK + x * 16);
      const uint4 w0 = make_uint4(fp8x2_to_bf16x2<false>(raw.x), fp8x2_to_bf16x2<true>(raw.x),
                                  fp8x2_to_bf16x2<false>(raw.y), fp8x2_to_bf16x2<true>(raw.y));
      const uint4 w1 = make_uint4(fp8x2_to_bf16x2<false>(raw.z), fp8x2_to_bf16x2<true>(raw.z),
                                  fp8x2_to_bf16x2<false>(raw.w), fp8x2_to_bf16x2<true>(raw.w));
      const int xs = (x >> 3) & 1;
      char* row = dst + CR::TILE + b * CR::BLK + x * 32;
      *(uint4*)(row + 16 * xs) = w0;
      *(uint4*)(row + 16 * (1 ^ xs)) = w1;
    }
  };

  // ---- the ring.  Batch n is K and V of tile n, copied into stage n % S.
  // It is issued at iteration n - S + 1, after the barrier that ends every
  // read of that stage (tile n - S, read at iteration n - S).
  f32x16_t s0[NCB], s1[NCB];  // scores of the two key blocks
  // its first column is a real query (uniform: kept in a scalar register)
  const bool wave_active = __builtin_amdgcn_readfirstlane(q0 + 32 * wc * NCB / G < n_r ? 1 : 0) != 0;
  int id_next = -1;  // id of this wave's block of the next tile to copy
  auto copy_tile = [&](auto J, int n) __attribute__((always_inline)) {
    copy_k(kstage(J), id_next, n);
    copy_v(vstage(J), id_next);
    id_next = block_id(n + 1);
  };
  if (iters > 0) {
    id_next = block_id(0);
    // batches 0 .. S-2
    copy_tile(std::integral_constant<int, 0>{}, 0);
    if constexpr (S > 2) {
      copy_tile(std::integral_constant<int, 1>{}, 1);
      copy_tile(std::integral_constant<int, 2>{}, 2);
    }
    if constexpr (CVT) {
      // tile 0 widened before the loop; the loop widens tile t + 1 at t
      __builtin_amdgcn_s_waitcnt(pf_vmcnt((S - 2) * kLoadsPerBatch));
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      convert(kstage(std::integral_constant<int, 0>{}), cvb[0]);
    }
  }

  // One iteration: wait for tile t in LDS, then S^T = K Q^T, online
  // softmax, O^T += V^T P on tile t, with the copies of tile t+S-1 issued
  // after the first key block's P V products.  (Issued right after the
  // barrier, the copies of all eight waves reach the compute unit's load
  // unit at once and each wave stalls on them; in the middle of the
  // iteration the waves issue them at different times: 1.5% faster.)
  // Every wave runs every iteration.
  auto iteration = [&](auto J, int t, auto mask_c, auto last_c) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last_c)::value;
    const auto JN = [&] {
      if constexpr (std::is_same_v<decltype(J), int>) return J + S - 1;
      else return std::integral_constant<int, decltype(J)::value + S - 1>{};
    }();
    // batch t has landed (CVT: batch t + 1, and the widening of tile t)
    stage_barrier(std::integral_constant<int, CVT ? S - 3 : S - 2>{});
    if constexpr (CVT && !LAST) {
      const auto J1 = [&] {
        if constexpr (std::is_same_v<decltype(J), int>) return J + 1;
        else return std::integral_constant<int, decltype(J)::value + 1>{};
      }();
      convert(kstage(J1), cvb[(t + 1) & 1]);
    }
    // a fresh copy of the V fragment base each iteration: the compiler would
    // otherwise keep every stage's derived addresses live across the loop
    int vf = vfb;
    __asm__ volatile("" : "+v"(vf));
    const int k0 = kbeg + t * kPfKT;
    if constexpr (KS) {
      // paired waves: the copies first (two stages leave one iteration for
      // them to land), then this wave's key block of the tile
      if constexpr (!LAST) copy_tile(JN, t + S - 1);
      if (wave_active) {
        auto block = [&](auto KBc) __attribute__((always_inline)) {
          constexpr int kb = decltype(KBc)::value;
          float a[NCB];
          bool up[NCB];
          scores(kstage(J), kb, s0);
          softmax(s0, k0, kb, mask_c, a, up);
          rescale(a, up);
          pv(vstage(J), vf, k0, kb, mask_c);
        };
        if (kbw)
          block(std::integral_constant<int, 1>{});
        else
          block(std::integral_constant<int, 0>{});
      }
    } else if (wave_active) {  // uniform: a wave with no real column only copies
      float a0[NCB], a1[NCB];
      bool u0[NCB], u1[NCB];
      scores(rkstage(J, t), 0, s0);
      scores(rkstage(J, t), 1, s1);
      softmax(s0, k0, 0, mask_c, a0, u0);
      rescale(a0, u0);
      pv(rvstage(J, t), vf, k0, 0, mask_c);
      if constexpr (!LAST) copy_tile(JN, t + S - 1);
      softmax(s1, k0, 1, mask_c, a1, u1);
      rescale(a1, u1);
      pv(rvstage(J, t), vf, k0, 1, mask_c);
    } else if constexpr (!LAST) {
      copy_tile(JN, t + S - 1);
    }
  };
  auto single = [&](int t, auto mask_c, auto last_c) __attribute__((always_inline)) {
    iteration(t, t, mask_c, last_c);
  };
  // Tiles that end before the workgroup's first query position need no
  // mask for any column; the rest (the causal diagonal, the context end and
  // padding columns) take the masked variant.  The last tile issues no copy.
  const int wg_min_pos = PFX ? prior : prior + q0;
  const int n_plain = wg_min_pos >= kbeg ? min(iters, (wg_min_pos + 1 - kbeg) / kPfKT) : 0;
  // Tiles [from, to): single iterations up to the first tile of stage 0,
  // then whole rounds of S tiles with the stage of every read and copy a
  // constant (one register assignment for the body), then the rest.
  auto run = [&](int from, int to, auto mask_c) __attribute__((always_inline)) {
    using F = std::false_type;
    int t = from;
    while (t < to && (t & (S - 1)) != 0) single(t++, mask_c, F{});
    for (; t + S <= to; t += S) {
      iteration(std::integral_constant<int, 0>{}, t, mask_c, F{});
      iteration(std::integral_constant<int, 1>{}, t + 1, mask_c, F{});
      if constexpr (S > 2) {
        iteration(std::integral_constant<int, 2>{}, t + 2, mask_c, F{});
        iteration(std::integral_constant<int, 3>{}, t + 3, mask_c, F{});
      }
    }
    while (t < to) single(t++, mask_c, F{});
  };
  if (iters > 0) {
    const int split = min(n_plain, iters - 1);
    run(0, split, std::false_type{});
    run(split, iters - 1, std::true_type{});
    if (n_plain >= iters)
      single(iters - 1, std::false_type{}, std::true_type{});
    else
      single(iters - 1, std::true_type{}, std::true_type{});
  }
  // copies of tiles past the end may still be in flight: let them land
  // before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(pf_vmcnt(0));

  if constexpr (KS) {
    // Merge of paired waves through LDS (the ring is free once every wave
    // has left the loop and every copy has landed): the second wave of a
    // pair leaves m, l and O; the first rescales both to the larger max,
    //   m = max(m0, m1),  l = l0 2^(m0 - m) + l1 2^(m1 - m),  O likewise,
    // and goes on as if it had seen every key.
    static_assert(sizeof(ring) >= (size_t)CW * NCB * C::DB * 16 * kWave * 4, "merge area");
    __shared__ float xml[CW][NCB][2][kWave];
    float* xo = (float*)&ring[0][0] + (int64_t)wc * NCB * C::DB * 16 * kWave;
    __syncthreads();
    if (wave_active && kbw == 1) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        xml[wc][cb][0][lane] = m_run[cb];
        xml[wc][cb][1][lane] = l_run[cb];
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) xo[((cb * C::DB + db) * 16 + i) * kWave + lane] = acco[cb][db][i];
      }
    }
    __syncthreads();
    if (kbw == 1) return;  // uniform
    if (wave_active) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const float m1 = xml[wc][cb][0][lane];
        const float mx = fmaxf(m_run[cb], m1);
        const float f0 = __builtin_amdgcn_exp2f(m_run[cb] - mx);
        const float f1 = __builtin_amdgcn_exp2f(m1 - mx);
        m_run[cb] = mx;
        l_run[cb] = l_run[cb] * f0 + xml[wc][cb][1][lane] * f1;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            acco[cb][db][i] = acco[cb][db][i] * f0 + xo[((cb * C::DB + db) * 16 + i) * kWave + lane] * f1;
      }
    }
  }

  // ---- normalise and store (or, in shared-prefix mode, leave the partial
  // state): register i of dim block db is dim 32 db + 8 (i / 4) + 4 half +
  // i % 4 of this lane's column
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const float lt = l_run[cb] + xor_lane<32>(l_run[cb]);
    const int c = 32 * (wc * NCB + cb) + cw;
    const int qi = q0 + c / G;
    if (qi >= n_r) continue;
    if (partial) {  // uniform
      const int64_t slot = ((int64_t)(qs + qi) * p.num_q_heads + g * G + c % G) * p.ws_stride + part;
      if (half == 0) {
        p.ws_m[slot] = m_run[cb];
        p.ws_l[slot] = lt;
      }
      float* orow = p.ws_o + slot * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x16_t& a = acco[cb][db];
          *(float4*)(orow + 32 * db + 8 * i4 + 4 * half) =
              make_float4(a[4 * i4 + 0], a[4 * i4 + 1], a[4 * i4 + 2], a[4 * i4 + 3]);
        }
      continue;
    }
    float inv = lt > 0.f ? 1.f / lt : 0.f;
    if constexpr (KB == 1) inv *= p.v_scale;
    char* orow = (char*)p.out + ((int64_t)(qs + qi) * p.num_q_heads + g * G + c % G) * C::QRB;
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

// Merge of a split chunk: one wave per (request, query row, q head).  The
// row's query tile needed nk keys, cut into ceil(nk / part_keys) parts whose
// partial states (running max in log2 units, sum, unnormalised output) are
// combined with the online-softmax rescale:
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  out = sum_p O_p 2^(m_p - M) / L.
// Rows whose tile needed one part were written by the chunk kernel.
template <int D, int KB>
__global__ __launch_bounds__(kWave) void prefill_merge_kernel(PrefillParams p, int max_q_len) {
  const int h = blockIdx.x % p.num_q_heads;
  const int ri = blockIdx.x / p.num_q_heads;
  const int i = ri % max_q_len;
  const int r = ri / max_q_len;
  const int lane = threadIdx.x;
  constexpr int XL = D / kWave;  // dims per lane
  int qs = p.query_start_loc[r];
  int qe = p.query_start_loc[r + 1];
  const int ctx_raw = p.context_lens[r];
  qs = max(0, min(qs, p.total_q_tokens));
  qe = max(qs, min(qe, p.total_q_tokens));
  const int n_r = qe - qs;
  if (i >= n_r) return;
  const int ctx_cap = min(p.max_blocks_per_seq * kBlock, p.max_parts * p.part_keys);
  const int ctx = max(0, min(ctx_raw, ctx_cap));
  const int prior = ctx - n_r;
  const int q_end = min(n_r, (i / p.qt + 1) * p.qt);
  const int nk = pf_tile_keys(ctx, prior, q_end);
  if (nk <= p.part_keys) return;  // written by the chunk kernel
  const int nparts = (nk + p.part_keys - 1) / p.part_keys;
  const int64_t row = (int64_t)(qs + i) * p.num_q_heads + h;
  const float* wm = p.ws_m + row * p.ws_stride;
  const float* wl = p.ws_l + row * p.ws_stride;
  const float* wo = p.ws_o + row * p.ws_stride * D;
  float acc[XL];
#pragma unroll
  for (int e = 0; e < XL; ++e) acc[e] = 0.f;
  float L = 0.f, M = kPfNegBig;
  constexpr int PG = 8;  // partial states loaded together
  for (int q0 = 0; q0 < nparts; q0 += PG) {
    float mq[PG], lq[PG], oq[PG][XL];
#pragma unroll
    for (int j = 0; j < PG; ++j) {
      const int q = min(q0 + j, nparts - 1);
      mq[j] = wm[q];
      lq[j] = wl[q];
#pragma unroll
      for (int e = 0; e < XL; ++e) oq[j][e] = wo[(int64_t)q * D + lane + e * kWave];
    }
    float Mg = M;
#pragma unroll
    for (int j = 0; j < PG; ++j)
      if (q0 + j < nparts) Mg = fmaxf(Mg, mq[j]);
    const float rs = exp2f(M - Mg);  // rescale of what was merged so far
    L *= rs;
#pragma unroll
    for (int e = 0; e < XL; ++e) acc[e] *= rs;
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
  if constexpr (KB == 1) inv *= p.v_scale;
  uint16_t* orow = (uint16_t*)p.out + row * D;
#pragma unroll
  for (int e = 0; e < XL; ++e) orow[lane + e * kWave] = to_bf16(acc[e] * inv);
}

// Query rows one workgroup of W waves covers for GQA group size G.
constexpr int pf_queries(int W, int G) { return W * 32 * PA_PF_NCB / G; }

// The narrow shape when every request's rows (or a group's sequences) fit
// one narrow workgroup: its other waves would have no column to compute.
inline bool pf_narrow(int rows, int G) { return rows <= pf_queries(kPfNarrowWaves, G); }
// Paired waves when the rows fit half of it: two waves per column block,
// each taking one 32-key half of every tile.
inline bool pf_paired(int rows, int G) { return rows <= pf_queries(kPfNarrowWaves / 2, G); }

template <int D, int G, int KB>
static hipError_t launch_prefill_t(PrefillParams prm, int max_q_len, hipStream_t stream) {
  constexpr int NCB = PA_PF_NCB;
  const bool narrow = pf_narrow(max_q_len, G);
  const bool paired = pf_paired(max_q_len, G);
  prm.qt = paired ? pf_queries(kPfNarrowWaves / 2, G)
                  : narrow ? pf_queries(kPfNarrowWaves, G) : pf_queries(kPfWaves, G);
  prm.num_qtiles = (max_q_len + prm.qt - 1) / prm.qt;
  const int64_t grid = (int64_t)prm.num_qtiles * prm.num_reqs * prm.num_kv_heads * prm.max_parts;
  if (paired) {
    hipLaunchKernelGGL((prefill_chunk_kernel<D, G, NCB, false, kPfNarrowWaves, kPfNarrowStages, KB, true>),
                       dim3((unsigned)grid), dim3(kPfNarrowWaves * kWave), 0, stream, prm);
  } else if (narrow) {
    hipLaunchKernelGGL((prefill_chunk_kernel<D, G, NCB, false, kPfNarrowWaves, kPfNarrowStages, KB>),
                       dim3((unsigned)grid), dim3(kPfNarrowWaves * kWave), 0, stream, prm);
  } else {
    hipLaunchKernelGGL((prefill_chunk_kernel<D, G, NCB, false, kPfWaves, kPfStages, KB>),
                       dim3((unsigned)grid), dim3(kPfWaves * kWave), 0, stream, prm);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || prm.max_parts <= 1) return e;
  hipLaunchKernelGGL((prefill_merge_kernel<D, KB>),
                     dim3((unsigned)((int64_t)prm.num_reqs * max_q_len * prm.num_q_heads)),
                     dim3(kWave), 0, stream, prm, max_q_len);
  return hipGetLastError();
}

template <int D, int G, int KB>
static hipError_t launch_prefix_t(const PrefillParams& prm, int num_groups, hipStream_t stream) {
  constexpr int NCB = PA_PF_NCB;
  const int64_t grid = (int64_t)prm.prefix_parts * num_groups * prm.num_kv_heads;
  if (pf_paired(prm.group_size, G)) {
    hipLaunchKernelGGL((prefill_chunk_kernel<D, G, NCB, true, kPfNarrowWaves, kPfNarrowStages, KB, true>),
                       dim3((unsigned)grid), dim3(kPfNarrowWaves * kWave), 0, stream, prm);
  } else if (pf_narrow(prm.group_size, G)) {
    hipLaunchKernelGGL((prefill_chunk_kernel<D, G, NCB, true, kPfNarrowWaves, kPfNarrowStages, KB>),
                       dim3((unsigned)grid), dim3(kPfNarrowWaves * kWave), 0, stream, prm);
  } else {
    hipLaunchKernelGGL((prefill_chunk_kernel<D, G, NCB, true, kPfWaves, kPfStages, KB>),
                       dim3((unsigned)grid), dim3(kPfWaves * kWave), 0, stream, prm);
  }
  return hipGetLastError();
}

int prefill_queries_per_tile(int group) { return pf_queries(kPfWaves, group); }

bool prefill_narrow(int max_q_len, int group) { return pf_narrow(max_q_len, group); }

int prefill_tile_queries(int max_q_len, int group) {
  return pf_paired(max_q_len, group)   ? pf_queries(kPfNarrowWaves / 2, group)
         : pf_narrow(max_q_len, group) ? pf_queries(kPfNarrowWaves, group)
                                       : pf_queries(kPfWaves, group);
}


hipError_t launch_prefix_partials(const SharedPrefixArgs& a, const CacheGeom& g, hipStream_t stream) {
  if (a.prefix_parts == 0) return hipSuccess;
  PrefillParams p = {};
  p.q = (const char*)a.d.q;
  p.k_cache = (const char*)a.d.k_cache;
  p.v_cache = (const char*)a.d.v_cache;
  p.block_tables = a.d.block_tables;
  p.context_lens = a.d.context_lens;
  p.max_blocks_per_seq = a.d.max_blocks_per_seq;
  p.num_q_heads = a.d.num_q_heads;
  p.num_kv_heads = g.num_kv_heads;
  p.num_blocks = g.num_blocks;
  // fp8 pools: the K scale multiplies every score; partial outputs stay in
  // code units and the merge applies the V scale
  p.scale_log2 = a.d.scale * g.k_scale * kLog2e;
  p.prefix_lens = a.prefix_lens;
  p.group_size = a.group_size;
  p.prefix_partition = a.prefix_partition;
  p.prefix_parts = a.prefix_parts;
  p.ws_stride = a.ws_stride;
  const int64_t rows = (int64_t)a.d.num_seqs * a.d.num_q_heads;
  p.ws_m = a.d.ws;
  p.ws_l = a.d.ws + rows * a.ws_stride;
  p.ws_o = a.d.ws + (2 * rows * a.ws_stride + 3) / 4 * 4;
  const int G = a.d.num_q_heads / g.num_kv_heads;
  const int groups = a.d.num_seqs / a.group_size;
#define PA_PREFIX_CASE(KB_, D_, G_)                           \
  if (g.elem_bytes == KB_ && g.head_dim == D_ && G == G_) \
    return launch_prefix_t<D_, G_, KB_>(p, groups, stream);
  PA_PREFIX_CASE(2, 128, 1) PA_PREFIX_CASE(2, 128, 2) PA_PREFIX_CASE(2, 128, 4) PA_PREFIX_CASE(2, 128, 8)
  PA_PREFIX_CASE(2, 64, 1) PA_PREFIX_CASE(2, 64, 2) PA_PREFIX_CASE(2, 64, 4) PA_PREFIX_CASE(2, 64, 8)
  PA_PREFIX_CASE(1, 128, 1) PA_PREFIX_CASE(1, 128, 2) PA_PREFIX_CASE(1, 128, 4) PA_PREFIX_CASE(1, 128, 8)
#undef PA_PREFIX_CASE
  return hipErrorInvalidValue;
}

bool prefill_supported(int elem_bytes, int head_dim, int group) {
  const bool shape = elem_bytes == 2 ? (head_dim == 64 || head_dim == 128)
                                     : elem_bytes == 1 && head_dim == 128;
  return shape && (group == 1 || group == 2 || group == 4 || group == 8);
}

bool shared_prefix_supported(int elem_bytes, int head_dim, int group, int group_size) {
  return prefill_supported(elem_bytes, head_dim, group) && group_size >= 1 &&
         group_size <= prefill_queries_per_tile(group);
}

hipError_t launch_prefill(const PrefillArgs& a, const CacheGeom& g, hipStream_t stream) {
  PrefillParams p = {};
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
  // fp8 pools: the K scale multiplies every score, the V scale the output
  p.scale_log2 = a.scale * g.k_scale * kLog2e;
  p.v_scale = g.v_scale;
  // split: parts of part_keys keys, partial states in the workspace
  // [rows][max_parts] m, then l, then o (from a 16-byte boundary)
  p.max_parts = a.max_parts > 1 ? a.max_parts : 1;
  p.part_keys = a.max_parts > 1 ? a.part_keys : (1 << 30);
  if (p.max_parts > 1) {
    const int64_t slots = (int64_t)a.total_q_tokens * a.num_q_heads * p.max_parts;
    p.ws_stride = p.max_parts;
    p.ws_m = a.ws;
    p.ws_l = a.ws + slots;
    p.ws_o = a.ws + (2 * slots + 3) / 4 * 4;
  }
  const int G = a.num_q_heads / g.num_kv_heads;

#define PA_PREFILL_CASE(KB_, D_, G_)                  \
  if (g.elem_bytes == KB_ && g.head_dim == D_ && G == G_) \
    return launch_prefill_t<D_, G_, KB_>(p, a.max_q_len, stream);
  PA_PREFILL_CASE(2, 128, 1) PA_PREFILL_CASE(2, 128, 2) PA_PREFILL_CASE(2, 128, 4) PA_PREFILL_CASE(2, 128, 8)
  PA_PREFILL_CASE(2, 64, 1) PA_PREFILL_CASE(2, 64, 2) PA_PREFILL_CASE(2, 64, 4) PA_PREFILL_CASE(2, 64, 8)
  PA_PREFILL_CASE(1, 128, 1) PA_PREFILL_CASE(1, 128, 2) PA_PREFILL_CASE(1, 128, 4) PA_PREFILL_CASE(1, 128, 8)
#undef PA_PREFILL_CASE
  return hipErrorInvalidValue;
}

}  // namespace pa
