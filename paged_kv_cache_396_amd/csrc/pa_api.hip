// C ABI of libpa.so: argument validation, variant dispatch, split-K sizing.
// The semantics of every entry point are documented in include/pa.h.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <mutex>
#include <string>

#include "block_pool.h"
#include "pa_launch.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return PA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes_of(int32_t dtype) {
  if (dtype == PA_F32) return 4;
  if (dtype == PA_BF16) return 2;
  if (dtype == PA_FP8_E4M3) return 1;
  return 0;
}

// Validates a cache descriptor; fills geometry on success.
int check_desc(const pa_cache_desc* d, pa::CacheGeom* g) {
  if (!d) return fail(PA_ERR_NULL, "cache descriptor is NULL");
  const int eb = elem_bytes_of(d->dtype);
  if (!eb) return fail(PA_ERR_DTYPE, "unknown dtype %d", (int)d->dtype);
  if (d->block_size != PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d (only %d is built)", (int)d->block_size,
                PA_BLOCK_SIZE);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d (64 or 128 are built)", (int)d->head_dim);
  if (d->num_blocks < 1 || d->num_kv_heads < 1)
    return fail(PA_ERR_SHAPE, "num_blocks %d / num_kv_heads %d must be >= 1", (int)d->num_blocks,
                (int)d->num_kv_heads);
  // slots are int64 on the wire but kernels index tokens with 32-bit block
  // offsets times 16; keep num_blocks * 16 below 2^31
  if ((int64_t)d->num_blocks * PA_BLOCK_SIZE >= (int64_t)1 << 31)
    return fail(PA_ERR_OVERFLOW, "num_blocks %d * 16 slots exceeds 2^31", (int)d->num_blocks);
  if (eb == 1 && !(std::isfinite(d->k_scale) && d->k_scale > 0.f && std::isfinite(d->v_scale) &&
                   d->v_scale > 0.f))
    return fail(PA_ERR_SHAPE, "fp8 pools need finite positive k_scale / v_scale (%g, %g)",
                (double)d->k_scale, (double)d->v_scale);
  if (g) {
    g->num_blocks = d->num_blocks;
    g->num_kv_heads = d->num_kv_heads;
    g->head_dim = d->head_dim;
    g->elem_bytes = eb;
    g->k_scale = eb == 1 ? d->k_scale : 1.f;
    g->v_scale = eb == 1 ? d->v_scale : 1.f;
  }
  return PA_OK;
}

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

int32_t round_up16(int64_t x) { return (int32_t)((x + 15) / 16 * 16); }

// Resolves the partition size (tokens) for a decode call.
int32_t resolve_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx, int32_t req) {
  const int32_t whole = max_ctx < 16 ? 16 : round_up16(max_ctx);
  if (req < 0) return whole;
  if (req > 0) return req;
  // automatic: every workgroup pays a fixed start-up cost (dependent memory
  // round trips that take microseconds once the memory system is loaded),
  // every extra partition adds merge traffic, and workgroups of one sequence
  // that run together share its blocks through the caches (shared prefixes).
  // With at least 4 (sequence, kv head) units per compute unit there is no
  // split.  Otherwise split towards 8 workgroups per compute unit (shorter
  // pieces even out sequences of unequal length), but never below 512
  // tokens or 1/16 of the longest context per partition.
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  const int64_t cus = device_cu_count();
  if (units >= 4 * cus) return whole;
  const int64_t target = 8 * cus;
  int64_t splits = target / (units > 0 ? units : 1);
  int32_t part = round_up16((max_ctx + splits - 1) / splits);
  const int32_t floor_part = max_ctx / 16 > 512 ? round_up16(max_ctx / 16) : 512;
  if (part < floor_part) part = floor_part;
  return part >= whole ? whole : part;
}

// Upper bound on the ranges per kv head of the balanced schedule (it sizes
// the workspace), or 0 for per-partition workgroups.  The balanced schedule
// serves automatic calls that the rule above would split (few (sequence, kv
// head) units for the chip): it gives every workgroup the same number of
// blocks however unequal the contexts.  The launch takes one range per
// resident workgroup slot of the kernel variant (at most
// kBalancedMaxWgPerCu per compute unit) times kBalancedRounds.
int32_t balanced_ranges(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx, int32_t req) {
  if (req != 0 || num_seqs < 1 || num_seqs > pa::kBalancedMaxSeqs || num_kv_heads < 1 ||
      pa::kBalancedRounds < 1)
    return 0;
  const int32_t whole = max_ctx < 16 ? 16 : round_up16(max_ctx);
  if (resolve_partition(num_seqs, num_kv_heads, max_ctx, 0) >= whole) return 0;
  // block-list positions are int32 on the device
  if ((int64_t)num_seqs * (((int64_t)max_ctx + 15) / 16) >= ((int64_t)1 << 31)) return 0;
  const int64_t r =
      (int64_t)device_cu_count() * pa::kBalancedMaxWgPerCu * pa::kBalancedRounds / num_kv_heads;
  return (int32_t)(r < 1 ? 1 : r);
}

// Workspace bytes of a decode call: partial states of (kv head, range, 2,
// group head) for the balanced schedule, of (seq, q head, partition)
// otherwise; 0 when nothing is split.
size_t decode_ws_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t max_ctx, int32_t req) {
  const int32_t ranges = balanced_ranges(num_seqs, num_kv_heads, max_ctx, req);
  if (ranges > 0) return (size_t)ranges * 2 * num_q_heads * (head_dim + 2) * sizeof(float);
  const int32_t part = resolve_partition(num_seqs, num_kv_heads, max_ctx, req);
  const int64_t nparts = ((int64_t)max_ctx + part - 1) / part;
  if (nparts <= 1) return 0;
  return (size_t)num_seqs * num_q_heads * nparts * (head_dim + 2) * sizeof(float);
}

}  // namespace

PA_API int pa_abi_version(void) { return PA_ABI_VERSION; }

PA_API size_t pa_cache_bytes(const pa_cache_desc* desc) {
  pa::CacheGeom g;
  if (check_desc(desc, &g) != PA_OK) return 0;
  return (size_t)g.num_blocks * g.num_kv_heads * PA_BLOCK_SIZE * g.head_dim * g.elem_bytes;
}

PA_API int pa_reshape_and_cache(const void* k, const void* v, const int64_t* slot_mapping,
                                int32_t num_tokens, void* k_cache, void* v_cache,
                                const pa_cache_desc* desc, void* stream) {
  pa::CacheGeom g;
  int st = check_desc(desc, &g);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens %d < 0", (int)num_tokens);
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !k_cache || !v_cache)
    return fail(PA_ERR_NULL, "k, v, slot_mapping, k_cache and v_cache must be non-NULL");
  if ((int64_t)num_tokens * g.num_kv_heads * g.head_dim * 4 / 16 >= ((int64_t)1 << 40))
    return fail(PA_ERR_OVERFLOW, "too many tokens for one call");
  hipError_t e = pa::launch_cache_write(k, v, slot_mapping, num_tokens, k_cache, v_cache, g,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cache write launch");
  return ok();
}

PA_API int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                        int32_t max_context_len, int32_t partition_size_request) {
  if (num_seqs < 0 || num_kv_heads < 1 || max_context_len < 0)
    return fail(PA_ERR_SHAPE, "num_seqs %d, num_kv_heads %d, max_context_len %d", (int)num_seqs,
                (int)num_kv_heads, (int)max_context_len);
  if (partition_size_request > 0 && partition_size_request % PA_BLOCK_SIZE != 0)
    return fail(PA_ERR_SHAPE, "partition_size %d is not a multiple of 16",
                (int)partition_size_request);
  if (balanced_ranges(num_seqs, num_kv_heads, max_context_len, partition_size_request) > 0)
    return 0;
  return resolve_partition(num_seqs, num_kv_heads, max_context_len, partition_size_request);
}

PA_API size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_context_len,
                                        int32_t partition_size_request) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0)
    return 0;
  if (partition_size_request > 0 && partition_size_request % PA_BLOCK_SIZE != 0) return 0;
  return decode_ws_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                         partition_size_request);
}

namespace {

// pa_decode, and pa_decode_append when new_k is not null.
int decode_call(void* out, const void* q, const void* new_k, const void* new_v,
                const int64_t* new_slots, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                int32_t num_q_heads, float scale, int32_t partition_size, void* workspace,
                size_t workspace_bytes, const pa_cache_desc* desc, void* stream) {
  pa::CacheGeom g;
  int st = check_desc(desc, &g);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 1 || num_q_heads < 1)
    return fail(PA_ERR_SHAPE, "num_seqs %d, max_context_len %d, max_blocks_per_seq %d, num_q_heads %d",
                (int)num_seqs, (int)max_context_len, (int)max_blocks_per_seq, (int)num_q_heads);
  if (num_q_heads % g.num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                (int)num_q_heads, g.num_kv_heads);
  const int group = num_q_heads / g.num_kv_heads;
  if (!pa::decode_supported(g.elem_bytes, g.head_dim, group))
    return fail(PA_ERR_UNSUPPORTED, "decode variant dtype=%d head_dim=%d group=%d is not built",
                (int)desc->dtype, g.head_dim, group);
  if (partition_size > 0 && partition_size % PA_BLOCK_SIZE != 0)
    return fail(PA_ERR_SHAPE, "partition_size %d is not a multiple of 16", (int)partition_size);
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_NULL, "out, q, k_cache, v_cache, block_tables and context_lens must be non-NULL");
  if (new_k && (!new_v || !new_slots))
    return fail(PA_ERR_NULL, "k, v and slot_mapping must be non-NULL");
  const int32_t part = resolve_partition(num_seqs, g.num_kv_heads, max_context_len, partition_size);
  int64_t nparts = ((int64_t)max_context_len + part - 1) / part;
  if (nparts < 1) nparts = 1;
  if (nparts * num_seqs * g.num_kv_heads >= ((int64_t)1 << 31) ||
      (int64_t)num_seqs * num_q_heads >= ((int64_t)1 << 31))
    return fail(PA_ERR_OVERFLOW, "decode grid too large");
  const int32_t ranges = balanced_ranges(num_seqs, g.num_kv_heads, max_context_len, partition_size);
  float* ws = nullptr;
  if (nparts > 1 || ranges > 0) {
    const size_t need = decode_ws_bytes(num_seqs, num_q_heads, g.num_kv_heads, g.head_dim,
                                        max_context_len, partition_size);
    if (!workspace || workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given (ptr %p)", need,
                  workspace_bytes, workspace);
    ws = (float*)workspace;
  }
  pa::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.ws = ws;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_partitions = (int)nparts;
  a.partition_blocks = part / PA_BLOCK_SIZE;
  a.scale = scale;
  a.num_ranges = ranges;
  a.max_ctx = max_context_len;
  a.new_k = new_k;
  a.new_v = new_v;
  a.new_slots = new_slots;
  hipError_t e = pa::launch_decode(a, g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

// ---------------------------------------------------------------------------
// The library's own decode scratch for pa_decode_append_noalloc: a file-scope
// device array, one copy per GPU, held until the process ends.  Host code
// never passes its name to a kernel (on the host that name is only a
// stand-in); it uses the device address hipGetSymbolAddress returns, looked
// up once per device with that device current.
constexpr size_t kScratchBytes = (size_t)PA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

int scratch_ptr(float** out) {
  static std::mutex mu;
  static float* ptrs[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(PA_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    ptrs[dev] = (float*)p;
  }
  *out = ptrs[dev];
  return PA_OK;
}

}  // namespace

PA_API int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                     int32_t num_q_heads, float scale, int32_t partition_size, void* workspace,
                     size_t workspace_bytes, const pa_cache_desc* desc, void* stream) {
  return decode_call(out, q, nullptr, nullptr, nullptr, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                     scale, partition_size, workspace, workspace_bytes, desc, stream);
}

PA_API int pa_decode_append(void* out, const void* q, const void* k, const void* v,
                            const int64_t* slot_mapping, void* k_cache, void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t max_context_len,
                            int32_t num_seqs, int32_t num_q_heads, float scale,
                            int32_t partition_size, void* workspace, size_t workspace_bytes,
                            const pa_cache_desc* desc, void* stream) {
  if (num_seqs > 0 && (!k || !v || !slot_mapping))
    return fail(PA_ERR_NULL, "k, v and slot_mapping must be non-NULL");
  return decode_call(out, q, k, v, slot_mapping, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                     scale, partition_size, workspace, workspace_bytes, desc, stream);
}

PA_API int pa_decode_append_noalloc(void* out, const void* q, const void* k, const void* v,
                                    const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t max_context_len,
                                    int32_t num_seqs, int32_t num_q_heads, float scale,
                                    int32_t partition_size, const pa_cache_desc* desc,
                                    void* stream) {
  if (num_seqs > 0 && (!k || !v || !slot_mapping))
    return fail(PA_ERR_NULL, "k, v and slot_mapping must be non-NULL");
  pa::CacheGeom g;
  int st = check_desc(desc, &g);
  if (st != PA_OK) return st;
  if (num_seqs <= 0 || num_q_heads <= 0 || max_context_len < 0)
    return decode_call(out, q, k, v, slot_mapping, k_cache, v_cache, block_tables,
                       max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                       scale, partition_size, nullptr, 0, desc, stream);
  if (partition_size > 0 && partition_size % PA_BLOCK_SIZE != 0)
    return fail(PA_ERR_SHAPE, "partition_size %d is not a multiple of 16", (int)partition_size);
  const size_t need = decode_ws_bytes(num_seqs, num_q_heads, g.num_kv_heads, g.head_dim,
                                      max_context_len, partition_size);
  if (need > kScratchBytes)
    return fail(PA_ERR_WORKSPACE,
                "pa_decode_append_noalloc: this call needs %zu bytes of scratch, the library's "
                "static scratch holds %zu (use pa_decode_append with a workspace)",
                need, kScratchBytes);
  float* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != PA_OK) return st;
  return decode_call(out, q, k, v, slot_mapping, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                     scale, partition_size, ws, kScratchBytes, desc, stream);
}

namespace {

// Launch plan of a shared-prefix decode (host side, from host bounds only).
struct SharedPrefixPlan {
  int32_t prefix_partition;  // tokens per prefix partition
  int32_t prefix_parts;      // partitions of the longest prefix
  int32_t own_partition;     // tokens per partition of a sequence's own blocks
  int32_t own_parts;
  int32_t stride;            // partial slots per (seq, q head) row
};

#ifndef PA_SP_WG_PER_CU
#define PA_SP_WG_PER_CU 2
#endif

SharedPrefixPlan plan_shared_prefix(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx,
                                    int32_t group_size, int32_t max_prefix) {
  SharedPrefixPlan pl;
  // prefix: split towards PA_SP_WG_PER_CU workgroups per compute unit, in
  // pieces of at least 256 keys.  The prefix workgroups of parallel sampling
  // (a few query rows each) take the narrow variant, two of which share a
  // compute unit; on the 32 x 4 shared-prefix batch with caches evicted,
  // two per compute unit (2048-token prefixes in two parts) measured 75.1 us
  // against 77.9 us for one and 79.0 us for four.
  const int64_t units = (int64_t)(num_seqs / group_size) * num_kv_heads;
  const int64_t slots = (int64_t)device_cu_count() * PA_SP_WG_PER_CU;
  const int64_t splits = units >= slots ? 1 : (slots + units - 1) / units;
  int64_t pp = (max_prefix + splits - 1) / splits;
  pp = (pp + 63) / 64 * 64;
  if (pp < 256) pp = 256;
  pl.prefix_partition = (int32_t)pp;
  pl.prefix_parts = max_prefix > 0 ? (int32_t)((max_prefix + pp - 1) / pp) : 0;
  // a sequence's own blocks: the plain decode rule over the longest context
  pl.own_partition = resolve_partition(num_seqs, num_kv_heads, max_ctx, 0);
  pl.own_parts = (int32_t)(((int64_t)max_ctx + pl.own_partition - 1) / pl.own_partition);
  if (pl.own_parts < 1) pl.own_parts = 1;
  pl.stride = pl.prefix_parts + pl.own_parts;
  return pl;
}

}  // namespace

PA_API size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                      int32_t num_kv_heads, int32_t head_dim,
                                                      int32_t max_context_len, int32_t group_size,
                                                      int32_t max_prefix_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len < 0 || group_size < 1 || num_seqs % group_size != 0 || max_prefix_len < 0 ||
      max_prefix_len % PA_BLOCK_SIZE != 0 || max_prefix_len > max_context_len)
    return 0;
  const SharedPrefixPlan pl =
      plan_shared_prefix(num_seqs, num_kv_heads, max_context_len, group_size, max_prefix_len);
  return pa::shared_prefix_ws_floats((int64_t)num_seqs * num_q_heads, pl.stride, head_dim) *
         sizeof(float);
}

PA_API int pa_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
                                   float scale, const int32_t* prefix_lens, int32_t group_size,
                                   int32_t max_prefix_len, void* workspace, size_t workspace_bytes,
                                   const pa_cache_desc* desc, void* stream) {
  pa::CacheGeom g;
  int st = check_desc(desc, &g);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 1 || num_q_heads < 1)
    return fail(PA_ERR_SHAPE, "num_seqs %d, max_context_len %d, max_blocks_per_seq %d, num_q_heads %d",
                (int)num_seqs, (int)max_context_len, (int)max_blocks_per_seq, (int)num_q_heads);
  if (num_q_heads % g.num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                (int)num_q_heads, g.num_kv_heads);
  if (group_size < 1 || num_seqs % group_size != 0)
    return fail(PA_ERR_SHAPE, "num_seqs %d is not a multiple of group_size %d", (int)num_seqs,
                (int)group_size);
  if (max_prefix_len < 0 || max_prefix_len % PA_BLOCK_SIZE != 0 || max_prefix_len > max_context_len)
    return fail(PA_ERR_SHAPE, "max_prefix_len %d must be a multiple of 16 in [0, max_context_len %d]",
                (int)max_prefix_len, (int)max_context_len);
  const int group = num_q_heads / g.num_kv_heads;
  if (!pa::shared_prefix_supported(g.elem_bytes, g.head_dim, group, group_size))
    return fail(PA_ERR_UNSUPPORTED,
                "shared-prefix decode dtype=%d head_dim=%d group=%d group_size=%d is not built",
                (int)desc->dtype, g.head_dim, group, (int)group_size);
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !prefix_lens)
    return fail(PA_ERR_NULL, "out, q, k_cache, v_cache, block_tables, context_lens and prefix_lens "
                             "must be non-NULL");
  const SharedPrefixPlan pl =
      plan_shared_prefix(num_seqs, g.num_kv_heads, max_context_len, group_size, max_prefix_len);
  if ((int64_t)pl.own_parts * num_seqs * g.num_kv_heads >= ((int64_t)1 << 31) ||
      (int64_t)pl.prefix_parts * num_seqs * g.num_kv_heads >= ((int64_t)1 << 31) ||
      (int64_t)num_seqs * num_q_heads >= ((int64_t)1 << 31))
    return fail(PA_ERR_OVERFLOW, "shared-prefix decode grid too large");
  const size_t need =
      pa::shared_prefix_ws_floats((int64_t)num_seqs * num_q_heads, pl.stride, g.head_dim) * sizeof(float);
  if (!workspace || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given (ptr %p)", need,
                workspace_bytes, workspace);
  pa::SharedPrefixArgs a;
  a.d.out = out;
  a.d.q = q;
  a.d.k_cache = k_cache;
  a.d.v_cache = v_cache;
  a.d.block_tables = block_tables;
  a.d.context_lens = context_lens;
  a.d.ws = (float*)workspace;
  a.d.max_blocks_per_seq = max_blocks_per_seq;
  a.d.num_seqs = num_seqs;
  a.d.num_q_heads = num_q_heads;
  a.d.num_partitions = pl.own_parts;
  a.d.partition_blocks = pl.own_partition / PA_BLOCK_SIZE;
  a.d.scale = scale;
  a.prefix_lens = prefix_lens;
  a.group_size = group_size;
  a.prefix_partition = pl.prefix_partition;
  a.prefix_parts = pl.prefix_parts;
  a.ws_stride = pl.stride;
  hipError_t e = pa::launch_prefix_partials(a, g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "shared-prefix launch");
  e = pa::launch_decode_own_and_merge(a, g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "shared-prefix decode launch");
  return ok();
}

namespace {

#ifndef PA_PF_SPLIT_FACTOR
#define PA_PF_SPLIT_FACTOR 1
#endif
#ifndef PA_PF_SPLIT_MIN_KEYS
#define PA_PF_SPLIT_MIN_KEYS 512
#endif

// Keys per part of a split prefill call, or 0 for no split.  Automatic:
// only the narrow variant (a few query rows per request: speculative
// verification, short chunks) is split, and only when its (request, kv
// head) workgroups do not fill the resident slots (two per compute unit):
// then each context is cut into parts so that the slots fill.  A batch that
// already fills them is not split: on the 64-request verification batch
// (contexts U[128, 4096)) parts of 512 to 2048 keys measured equal or
// slower than whole contexts.  The wide variant keeps its compute units
// busy on the matrix cores and is not split.
int32_t prefill_part_keys(int32_t num_reqs, int32_t num_kv_heads, int32_t max_q_len, int32_t group,
                          int32_t max_ctx, int32_t req) {
  if (req < 0 || max_ctx <= 0) return 0;
  if (req > 0) return req;
  if (!pa::prefill_narrow(max_q_len, group)) return 0;
  const int64_t qt = pa::prefill_tile_queries(max_q_len, group);
  const int64_t units = (int64_t)num_reqs * num_kv_heads * ((max_q_len + qt - 1) / qt);
  const int64_t slots = 2 * (int64_t)device_cu_count();
  const int64_t target = (PA_PF_SPLIT_FACTOR * slots + units - 1) / (units > 0 ? units : 1);
  if (target <= 1) return 0;
  int64_t part = ((max_ctx + target - 1) / target + 63) / 64 * 64;
  if (part < PA_PF_SPLIT_MIN_KEYS) part = PA_PF_SPLIT_MIN_KEYS;
  return part >= max_ctx ? 0 : (int32_t)part;
}

size_t prefill_ws_bytes(int32_t total_q_tokens, int32_t num_q_heads, int32_t head_dim,
                        int32_t max_ctx, int32_t part) {
  if (part <= 0) return 0;
  const int64_t parts = ((int64_t)max_ctx + part - 1) / part;
  if (parts <= 1) return 0;
  return pa::prefill_ws_floats((int64_t)total_q_tokens * num_q_heads, (int)parts, head_dim) *
         sizeof(float);
}

}  // namespace

PA_API size_t pa_prefill_chunk_workspace_bytes(int32_t num_reqs, int32_t total_q_tokens,
                                               int32_t max_q_len, int32_t max_context_len,
                                               int32_t num_q_heads, int32_t num_kv_heads,
                                               int32_t head_dim, int32_t partition_size) {
  if (num_reqs <= 0 || total_q_tokens <= 0 || max_q_len <= 0 || max_context_len <= 0 ||
      num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0)
    return 0;
  if (partition_size > 0 && partition_size % 64 != 0) return 0;
  const int32_t part = prefill_part_keys(num_reqs, num_kv_heads, max_q_len,
                                         num_q_heads / num_kv_heads, max_context_len,
                                         partition_size);
  return prefill_ws_bytes(total_q_tokens, num_q_heads, head_dim, max_context_len, part);
}

PA_API int pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* query_start_loc, const int32_t* context_lens,
                            int32_t num_reqs, int32_t total_q_tokens, int32_t max_q_len,
                            int32_t max_context_len, int32_t num_q_heads, float scale,
                            int32_t partition_size, void* workspace, size_t workspace_bytes,
                            const pa_cache_desc* desc, void* stream) {
  pa::CacheGeom g;
  int st = check_desc(desc, &g);
  if (st != PA_OK) return st;
  if (num_reqs < 0 || total_q_tokens < 0 || max_q_len < 0 || max_context_len < 0 ||
      max_blocks_per_seq < 1 || num_q_heads < 1)
    return fail(PA_ERR_SHAPE,
                "num_reqs %d, total_q_tokens %d, max_q_len %d, max_context_len %d, "
                "max_blocks_per_seq %d, num_q_heads %d",
                (int)num_reqs, (int)total_q_tokens, (int)max_q_len, (int)max_context_len,
                (int)max_blocks_per_seq, (int)num_q_heads);
  if (num_q_heads % g.num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                (int)num_q_heads, g.num_kv_heads);
  const int group = num_q_heads / g.num_kv_heads;
  if (!pa::prefill_supported(g.elem_bytes, g.head_dim, group))
    return fail(PA_ERR_UNSUPPORTED, "prefill variant dtype=%d head_dim=%d group=%d is not built",
                (int)desc->dtype, g.head_dim, group);
  if (partition_size > 0 && partition_size % 64 != 0)
    return fail(PA_ERR_SHAPE, "partition_size %d is not a multiple of 64", (int)partition_size);
  if (num_reqs == 0 || total_q_tokens == 0 || max_q_len == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start_loc || !context_lens)
    return fail(PA_ERR_NULL, "prefill pointers must be non-NULL");
  // automatic with no workspace: unsplit
  const int32_t part =
      (partition_size == 0 && !workspace)
          ? 0
          : prefill_part_keys(num_reqs, g.num_kv_heads, max_q_len, group, max_context_len,
                              partition_size);
  const int64_t parts = part > 0 ? ((int64_t)max_context_len + part - 1) / part : 1;
  const int64_t qt = pa::prefill_tile_queries(max_q_len, group);
  if ((max_q_len + qt - 1) / qt * (int64_t)num_reqs * g.num_kv_heads * parts >= ((int64_t)1 << 31) ||
      (int64_t)num_reqs * max_q_len * num_q_heads >= ((int64_t)1 << 31) ||
      (int64_t)total_q_tokens * num_q_heads * g.head_dim * (parts > 1 ? parts : 1) >= ((int64_t)1 << 40))
    return fail(PA_ERR_OVERFLOW, "prefill grid too large");
  pa::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.query_start_loc = query_start_loc;
  a.context_lens = context_lens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_reqs = num_reqs;
  a.total_q_tokens = total_q_tokens;
  a.max_q_len = max_q_len;
  a.num_q_heads = num_q_heads;
  a.scale = scale;
  if (parts > 1) {
    const size_t need = prefill_ws_bytes(total_q_tokens, num_q_heads, g.head_dim, max_context_len, part);
    if (!workspace || workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "prefill workspace of %zu bytes needed, %zu given (ptr %p)",
                  need, workspace_bytes, workspace);
    a.max_parts = (int)parts;
    a.part_keys = part;
    a.ws = (float*)workspace;
  }
  hipError_t e = pa::launch_prefill(a, g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

PA_API int pa_bw_probe(const void* buf, size_t bytes, const int32_t* tile_order, int32_t num_tiles,
                       uint32_t* sink, void* stream) {
  if (num_tiles < 0) return fail(PA_ERR_SHAPE, "num_tiles %d < 0", (int)num_tiles);
  if (num_tiles == 0) return ok();
  if (!buf || !tile_order || !sink) return fail(PA_ERR_NULL, "buf, tile_order and sink must be non-NULL");
  if (bytes < 4096) return fail(PA_ERR_SHAPE, "buffer of %zu bytes holds no 4 KiB tile", bytes);
  if (bytes / 4096 >= ((size_t)1 << 31)) return fail(PA_ERR_OVERFLOW, "buffer too large");
  hipError_t e = pa::launch_bw_probe(buf, bytes, tile_order, num_tiles, sink, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "probe launch");
  return ok();
}

PA_API size_t pa_rejection_sample_workspace_bytes(int32_t num_reqs, int32_t vocab) {
  if (num_reqs <= 0 || vocab < 1 || vocab > PA_MAX_VOCAB) return 0;
  return pa::spec_verify_workspace_bytes(num_reqs, vocab);
}

PA_API int pa_rejection_sample(const float* target_probs, const float* draft_probs,
                               const int32_t* draft_tokens, const float* uniforms,
                               int32_t num_reqs, int32_t num_draft, int32_t vocab,
                               int32_t* out_tokens, int32_t* num_out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (num_reqs < 0 || num_draft < 0 || vocab < 1)
    return fail(PA_ERR_SHAPE, "num_reqs %d, num_draft %d, vocab %d", (int)num_reqs, (int)num_draft,
                (int)vocab);
  if (num_draft > PA_MAX_DRAFT)
    return fail(PA_ERR_UNSUPPORTED, "num_draft %d (at most %d)", (int)num_draft, PA_MAX_DRAFT);
  if (vocab > PA_MAX_VOCAB)
    return fail(PA_ERR_UNSUPPORTED, "vocab %d (at most %d)", (int)vocab, PA_MAX_VOCAB);
  if ((int64_t)num_reqs * (num_draft + 1) * vocab >= ((int64_t)1 << 40))
    return fail(PA_ERR_OVERFLOW, "probability arrays too large");
  if (num_reqs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_reqs %d (at most 65535)", (int)num_reqs);
  if (num_reqs == 0) return ok();
  if (!target_probs || !uniforms || !out_tokens || !num_out || (num_draft > 0 && !draft_tokens))
    return fail(PA_ERR_NULL, "target_probs, draft_tokens, uniforms, out_tokens and num_out must be non-NULL");
  const size_t need = pa::spec_verify_workspace_bytes(num_reqs, vocab);
  if (!workspace || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given (ptr %p)", need,
                workspace_bytes, workspace);
  pa::SpecVerifyArgs a;
  a.target_probs = target_probs;
  a.draft_probs = draft_probs;
  a.draft_tokens = draft_tokens;
  a.uniforms = uniforms;
  a.out_tokens = out_tokens;
  a.num_out = num_out;
  a.workspace = workspace;
  a.num_reqs = num_reqs;
  a.k = num_draft;
  a.vocab = vocab;
  hipError_t e = pa::launch_spec_verify(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rejection sampling launch");
  return ok();
}

// ---- block pool (host only)

struct pa_block_pool {
  pa::BlockPool pool;
  explicit pa_block_pool(int32_t n) : pool(n) {}
};

namespace {
int pool_status(int s, int64_t req) {
  switch (s) {
    case 0: return ok();
    case -1: return fail(PA_ERR_NO_REQUEST, "unknown request %lld", (long long)req);
    case -2: return fail(PA_ERR_REQUEST_EXISTS, "request id %lld is in use", (long long)req);
    default: return fail(PA_ERR_NO_BLOCKS, "not enough free blocks for request %lld", (long long)req);
  }
}
}  // namespace

PA_API pa_block_pool* pa_pool_create(int32_t num_blocks) {
  if (num_blocks < 2 || (int64_t)num_blocks * PA_BLOCK_SIZE >= ((int64_t)1 << 31)) {
    fail(PA_ERR_SHAPE, "num_blocks %d (2 .. 2^27-1)", (int)num_blocks);
    return nullptr;
  }
  try {
    pa_block_pool* p = new pa_block_pool(num_blocks);
    ok();
    return p;
  } catch (...) {
    fail(PA_ERR_OVERFLOW, "out of host memory for %d blocks", (int)num_blocks);
    return nullptr;
  }
}

PA_API void pa_pool_destroy(pa_block_pool* pool) { delete pool; }

PA_API int32_t pa_pool_num_free(const pa_block_pool* pool) {
  return pool ? pool->pool.num_free() : 0;
}

PA_API int pa_pool_add_request(pa_block_pool* pool, int64_t req, const int32_t* prompt, int32_t n,
                               int32_t* num_cached) {
  if (!pool || !num_cached || (n > 0 && !prompt)) return fail(PA_ERR_NULL, "pool, prompt and num_cached must be non-NULL");
  if (n < 0) return fail(PA_ERR_SHAPE, "prompt length %d", (int)n);
  return pool_status(pool->pool.add_request(req, prompt, n, num_cached), req);
}

PA_API int pa_pool_allocate_slots(pa_block_pool* pool, int64_t req, const int32_t* tokens, int32_t n,
                                  int64_t* slot_mapping, int32_t* copy, int32_t* num_copies) {
  if (!pool || !copy || !num_copies || (n > 0 && (!tokens || !slot_mapping)))
    return fail(PA_ERR_NULL, "pool, tokens, slot_mapping, copy and num_copies must be non-NULL");
  if (n < 0) return fail(PA_ERR_SHAPE, "token count %d", (int)n);
  const int32_t have = pool->pool.num_tokens(req);
  if (have >= 0 && (int64_t)have + n >= ((int64_t)1 << 31) - PA_BLOCK_SIZE)
    return fail(PA_ERR_OVERFLOW, "request %lld would exceed 2^31 tokens", (long long)req);
  return pool_status(pool->pool.allocate_slots(req, tokens, n, slot_mapping, copy, num_copies), req);
}

PA_API int pa_pool_fork(pa_block_pool* pool, int64_t parent, int64_t child) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  const int s = pool->pool.fork(parent, child);
  return pool_status(s, s == -2 ? child : parent);
}

PA_API int pa_pool_free_request(pa_block_pool* pool, int64_t req) {
  if (!pool) return fail(PA_ERR_NULL, "pool is NULL");
  return pool_status(pool->pool.free_request(req), req);
}

PA_API int pa_pool_block_table(const pa_block_pool* pool, int64_t req, int32_t* row,
                               int32_t capacity, int32_t* num_blocks) {
  if (!pool || !num_blocks || (capacity > 0 && !row))
    return fail(PA_ERR_NULL, "pool, row and num_blocks must be non-NULL");
  const std::vector<int32_t>* t = pool->pool.table(req);
  if (!t) return fail(PA_ERR_NO_REQUEST, "unknown request %lld", (long long)req);
  *num_blocks = (int32_t)t->size();
  for (int32_t i = 0; i < capacity && i < (int32_t)t->size(); ++i) row[i] = (*t)[i];
  return ok();
}

PA_API int pa_pool_num_tokens(const pa_block_pool* pool, int64_t req, int32_t* num_tokens) {
  if (!pool || !num_tokens) return fail(PA_ERR_NULL, "pool and num_tokens must be non-NULL");
  const int32_t n = pool->pool.num_tokens(req);
  if (n < 0) return fail(PA_ERR_NO_REQUEST, "unknown request %lld", (long long)req);
  *num_tokens = n;
  return ok();
}

PA_API int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                          const pa_cache_desc* desc, void* stream) {
  pa::CacheGeom g;
  int st = check_desc(desc, &g);
  if (st != PA_OK) return st;
  if (num_pairs < 0 || num_pairs >= (1 << 30)) return fail(PA_ERR_SHAPE, "num_pairs %d", (int)num_pairs);
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !pairs) return fail(PA_ERR_NULL, "k_cache, v_cache and pairs must be non-NULL");
  hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, pairs, num_pairs, g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
  return ok();
}

PA_API const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_SHAPE: return "invalid shape";
    case PA_ERR_DTYPE: return "invalid dtype";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_OVERFLOW: return "size overflow";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks";
    case PA_ERR_NO_REQUEST: return "unknown request";
    case PA_ERR_REQUEST_EXISTS: return "request id in use";
    default: return "unknown status";
  }
}

PA_API const char* pa_last_error(void) { return g_last_error.c_str(); }
