/*
 * pa.h — C ABI of the MI355X (gfx950) paged-attention library libpa.so.
 *
 * The library implements the data-parallel hot path of PagedAttention as the
 * pages describe it:
 *   - the KV cache is cut into fixed blocks of 16 tokens that need not be
 *     contiguous, and a per-sequence block table maps logical to physical
 *     blocks ("vLLM: from PagedAttention to Speculative Decoding", 3.2;
 *     zihan-zhang.net vLLM study, 3.2);
 *   - kernels reach the scattered blocks through block_table (reads) and
 *     slot_mapping (writes); logical token i is in block block_table[i / 16]
 *     at offset i % 16 ("vLLM: from PagedAttention ...", 3.3);
 *   - attention is softmax(Q K^T / sqrt(d)) V under a causal mask
 *     (zihan-zhang.net vLLM study, 1.1.1), evaluated block by block with the
 *     online-softmax rescaling of FlashAttention (same page, 4.3.1).
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers.  The caller owns every buffer;
 *     the library never allocates, frees or synchronizes.  Work is enqueued
 *     on `stream` (a hipStream_t, NULL = the null stream) and the call returns
 *     before the GPU finishes.
 *   - q, k, v and out are dense row-major [tokens][heads][head_dim] in the
 *     cache dtype (fp32 or bf16; bf16 for PA_FP8_E4M3 pools); out has the
 *     dtype of q.
 *   - Block tables are int32 [rows][max_blocks_per_seq]; entries past a
 *     sequence's ceil(len / 16) blocks are never read.
 *   - Argument errors detected on the host return a negative pa_status and
 *     launch nothing; pa_last_error() then holds a description (per thread).
 *   - Values that live on the device (slots, block ids, lengths) are not
 *     checked on the host.  Kernels ignore slots outside the pool, treat
 *     block ids outside [0, num_blocks) as empty blocks and clamp lengths to
 *     what the table row and max_context_len cover, so a bad value gives a
 *     wrong result but never touches memory outside the caller's buffers.
 *
 * Pool layout (owned by the library; size it with pa_cache_bytes):
 *   K pool element (block b, kv head g, token offset o, dim x) at element index
 *       ((b * Hkv + g) * 16 + o) * D + x
 *   V pool element (b, g, o, x) at element index
 *       ((b * Hkv + g) * D + x) * 16 + o
 *   i.e. every (block, kv head) tile is one contiguous run (4 KiB for bf16
 *   with D = 128); K rows are token-major (one token's D values together), V
 *   rows are dim-major (one dim's 16 tokens together).  The pages print three
 *   different block-internal orders; this one is chosen so that every tile
 *   read is whole 128-byte lines on gfx950 and every 16-byte piece of a tile
 *   is directly a matrix-core operand fragment (K: 8 dims of one token,
 *   V: 8 tokens of one dim).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 3
#define PA_BLOCK_SIZE 16

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* sizes inconsistent or out of range */
  PA_ERR_DTYPE = -3,       /* unknown dtype */
  PA_ERR_UNSUPPORTED = -4, /* valid but not built: head_dim, GQA group, block size */
  PA_ERR_WORKSPACE = -5,   /* workspace missing or too small */
  PA_ERR_OVERFLOW = -6,    /* a size product does not fit the index types */
  PA_ERR_HIP = -7,         /* the HIP runtime reported an error */
  PA_ERR_NO_BLOCKS = -8,   /* block pool: not enough free blocks (nothing changed) */
  PA_ERR_NO_REQUEST = -9,  /* block pool: unknown request id */
  PA_ERR_REQUEST_EXISTS = -10 /* block pool: request id already in use */
} pa_status;

/* Pool element types.  PA_FP8_E4M3 pools hold one 8-bit code per element
 * (E4M3 of the OCP 8-bit floating-point format: 1 sign bit, 4 exponent bits
 * with bias 7, 3 mantissa bits, no infinities, largest magnitude 448) and
 * one fp32 scale per pool; the activations that meet such a pool (k and v
 * rows written, q, out) are bf16.  The pages name an fp8 KV cache for its
 * doubled capacity and halved attention bytes (zihan-zhang.net vLLM study,
 * 4.2.1) without fixing a format or scaling; these are the readings taken. */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

/* Describes one layer's K and V pools (both have the same shape). */
typedef struct {
  int32_t num_blocks;   /* physical blocks in the pool, >= 1 */
  int32_t block_size;   /* must be PA_BLOCK_SIZE (16) */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t dtype;        /* a pa_dtype */
  float k_scale;        /* PA_FP8_E4M3 only (finite, > 0): K code c stands for
                           value(c) * k_scale; ignored for other dtypes */
  float v_scale;        /* the same for the V pool */
} pa_cache_desc;

/* PA_ABI_VERSION of the built library. */
int pa_abi_version(void);

/* Bytes of ONE pool (K or V) for `desc`; 0 if desc is invalid. */
size_t pa_cache_bytes(const pa_cache_desc* desc);

/*
 * pa_reshape_and_cache — scatter new K/V rows into the pools
 * ("vLLM: from PagedAttention ...", 3.3: kernels address scattered blocks
 * through slot_mapping).
 *
 *   k, v          device, [num_tokens][Hkv][D] in the cache dtype (bf16 for
 *                 PA_FP8_E4M3 pools)
 *   slot_mapping  device int64 [num_tokens]; token i goes to block
 *                 slot / 16, offset slot % 16.  A negative slot marks a
 *                 padding token and writes nothing.  Slots at or beyond
 *                 num_blocks * 16 are ignored.  Two tokens with the same slot
 *                 in one call give an unspecified winner.
 *   k_cache, v_cache  device pools laid out as described above.
 * For bf16 and fp32 pools the copy is bit-exact (no value conversion).  For
 * PA_FP8_E4M3 pools each value x is stored as the E4M3 code nearest to
 * x / scale (the quotient one correctly rounded fp32 division), ties to the
 * even code; magnitudes beyond 448, infinities included, saturate to 448 with
 * x's sign, and a NaN gives code 0x7F with x's sign bit.  num_tokens == 0 is
 * a no-op.
 */
int pa_reshape_and_cache(const void* k, const void* v, const int64_t* slot_mapping,
                         int32_t num_tokens, void* k_cache, void* v_cache,
                         const pa_cache_desc* desc, void* stream);

/*
 * Partition size pa_decode uses for `partition_size_request`
 * (0 = automatic, < 0 = one partition per sequence, > 0 = that many tokens,
 * a multiple of 16).  Returns the resolved size in tokens, 0 when the call
 * runs the work-balanced schedule instead (an automatic call with fewer
 * than 4 (sequence, kv head) pairs per compute unit, at most 1024 sequences
 * and a context that would be split: the blocks of all sequences are cut
 * into equal ranges, one per resident workgroup, and the pieces of a
 * sequence are merged), or a negative pa_status.  The automatic choice
 * depends on the current device's compute unit count and on the shape.
 */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                                 int32_t partition_size_request);

/*
 * Workspace bytes pa_decode (and pa_decode_append) needs for these sizes and
 * this partition request (the same request later passed to pa_decode), on
 * the current device: the work-balanced schedule's workspace grows with the
 * device's compute unit count (2 partial states per (kv head, range, q head
 * of the group), ranges = 4 * CUs / num_kv_heads at most), independent of
 * the context lengths.  0 means no workspace is needed (every sequence fits
 * one partition).  pa_decode rechecks the size on the device it launches on
 * and returns PA_ERR_WORKSPACE when it is too small.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size_request);

/*
 * pa_decode — one query token per sequence attends to its whole paged context
 * (zihan-zhang.net vLLM study, 1.1.1 and 3.2: per block, look up the physical
 * block, score the 16 keys, then weight the 16 values; 4.3.1: online softmax).
 *
 *   out            device [num_seqs][num_q_heads][D], dtype of the cache
 *                  (bf16 for PA_FP8_E4M3 pools)
 *   q              device [num_seqs][num_q_heads][D], same dtype as out
 *   block_tables   device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens   device int32 [num_seqs]; counts the newest token, whose K/V
 *                  must already be in the pools (write it with
 *                  pa_reshape_and_cache earlier on the same stream).  A length
 *                  of 0 yields a zero output row.
 *   max_context_len  host bound on every context_lens entry (sizes the grid)
 *   scale          multiplies Q.K (normally 1/sqrt(D)), fp32
 *   partition_size 0 = automatic split-K, < 0 = no split, > 0 = tokens per
 *                  partition (multiple of 16).  Long contexts are split into
 *                  partitions whose partial softmax states are merged by a
 *                  second kernel with the same rescaling identity.  The
 *                  automatic choice may be the work-balanced schedule (see
 *                  pa_decode_partition_size), whose pieces are merged the
 *                  same way.
 *   workspace      device scratch of pa_decode_workspace_bytes(...) bytes
 *                  (may be NULL when that is 0).  Contents need no
 *                  initialisation and are overwritten; two calls in flight at
 *                  the same time must not share a workspace.
 * Query head h reads kv head h / (num_q_heads / Hkv).  Supported:
 * D in {64, 128}, num_q_heads / Hkv in {1, 2, 4, 8} (PA_FP8_E4M3 pools:
 * D = 128).  Accumulation is fp32.  With PA_FP8_E4M3 pools every code is
 * widened exactly to bf16 and attention runs over value(code) * scale: the
 * K scale is folded into `scale`, the V scale into the final normalisation.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
              int32_t num_q_heads, float scale, int32_t partition_size, void* workspace,
              size_t workspace_bytes, const pa_cache_desc* desc, void* stream);

/*
 * pa_decode_append — one decode step of a layer in one launch: the cache
 * write of every sequence's newest token (pa_reshape_and_cache of k, v,
 * slot_mapping with num_tokens = num_seqs) fused with pa_decode over the
 * updated pools (zihan-zhang.net vLLM study, 3.2: each step appends the new
 * token's K/V to its sequence's last block, then attends over all blocks).
 *
 *   k, v           device [num_seqs][Hkv][D], the q dtype (bf16 for
 *                  PA_FP8_E4M3 pools, encoded as pa_reshape_and_cache does):
 *                  row s is sequence s's newest token
 *   slot_mapping   device int64 [num_seqs]; slot of row s, negative = none
 *   context_lens   count the newest token (position context_lens[s] - 1)
 * The other arguments, the workspace rules and the supported variants are
 * pa_decode's.  Contract: for every s with slot_mapping[s] >= 0,
 * context_lens[s] >= 1 and slot_mapping[s] is position context_lens[s] - 1
 * of the sequence, i.e. block_tables[s][(ctx-1)/16] * 16 + (ctx-1) % 16, and
 * no other row's context holds that slot.  Then the pools end bit-identical
 * to pa_reshape_and_cache's and out equals pa_decode's over them up to the
 * order of fp32 sums (the newest token's K/V are taken from k, v instead of
 * being read back; its softmax term is added after the other tokens').
 * Rows whose context length is 0 (or negative) are not written.  Outside the
 * contract the pools are written as pa_reshape_and_cache writes them (slots
 * in range) but out is unspecified.
 */
int pa_decode_append(void* out, const void* q, const void* k, const void* v,
                     const int64_t* slot_mapping, void* k_cache, void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                     int32_t num_q_heads, float scale, int32_t partition_size, void* workspace,
                     size_t workspace_bytes, const pa_cache_desc* desc, void* stream);

/*
 * pa_decode_append_noalloc — pa_decode_append for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without the
 * workspace, the same kernels and the same result (bitwise equal to
 * pa_decode_append's for the same inputs).  The split-K partial states go to
 * a scratch array inside the library, PA_NOALLOC_SCRATCH_BYTES bytes per GPU,
 * held by every GPU the library runs on until the process ends; the call
 * itself allocates nothing.  A call whose workspace
 * (pa_decode_workspace_bytes) exceeds that size returns PA_ERR_WORKSPACE and
 * launches nothing.  Every call on one GPU shares that GPU's scratch: calls
 * that overlap on one GPU (two streams, or two threads) race and must be
 * ordered by the caller.  The scratch needs no initial contents; each call
 * overwrites what it reads.
 */
#define PA_NOALLOC_SCRATCH_BYTES (16u << 20)
int pa_decode_append_noalloc(void* out, const void* q, const void* k, const void* v,
                             const int64_t* slot_mapping, void* k_cache, void* v_cache,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t max_context_len,
                             int32_t num_seqs, int32_t num_q_heads, float scale,
                             int32_t partition_size, const pa_cache_desc* desc, void* stream);

/*
 * pa_decode_shared_prefix — pa_decode for sequences that share a prompt
 * prefix (parallel sampling: several samples of one prompt point their block
 * tables at the same prompt blocks; zihan-zhang.net vLLM study, 3.2.2, and
 * plumephp.com vLLM deep dive, 4.2).  Same inputs and result as pa_decode
 * (within rounding), but every shared block is read once per group instead
 * of once per sequence.
 *
 *   group_size     sequences g*group_size .. g*group_size+group_size-1 form
 *                  group g (num_seqs must be a multiple of it)
 *   prefix_lens    device int32 [num_seqs / group_size]: the group's shared
 *                  tokens, a multiple of 16 and at most every member's
 *                  context; the first prefix_lens[g] / 16 entries of the
 *                  members' block tables must be equal.  Values out of that
 *                  contract give unspecified output (no out-of-range access).
 *   max_prefix_len host bound on every prefix_lens entry (multiple of 16,
 *                  at most max_context_len; sizes the grid)
 *   workspace      device scratch of pa_decode_shared_prefix_workspace_bytes
 *                  bytes; same rules as pa_decode's.
 * The other arguments are pa_decode's.  Supported: bf16 pools with D in
 * {64, 128} and PA_FP8_E4M3 pools with D = 128,
 * num_q_heads / Hkv in {1, 2, 4, 8}, group_size * (num_q_heads / Hkv) <= 256.
 * The prefix part runs on bf16 MFMA (P rounded to bf16, as in
 * pa_prefill_chunk); each sequence's own blocks run through the decode
 * kernel; one merge kernel combines the partial softmax states.
 */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t max_context_len, int32_t group_size,
                                               int32_t max_prefix_len);
int pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t max_context_len,
                            int32_t num_seqs, int32_t num_q_heads, float scale,
                            const int32_t* prefix_lens, int32_t group_size,
                            int32_t max_prefix_len, void* workspace, size_t workspace_bytes,
                            const pa_cache_desc* desc, void* stream);

/*
 * Block pool — the host-side bookkeeping that produces block tables and
 * slot_mapping (zihan-zhang.net vLLM study, 3.2.2 sharing and copy-on-write,
 * 3.6 prefix caching, 5.5 the block pool; plumephp.com vLLM deep dive, 4.2).
 *
 * A pool of num_blocks blocks of 16 tokens; block 0 is a placeholder that is
 * never handed out.  Requests are named by caller-chosen int64 ids.
 *   - Blocks are shared by reference count (pa_pool_fork: parallel sampling).
 *   - A request that writes into a partly filled block others still hold
 *     first gets a copy (copy-on-write): pa_pool_allocate_slots returns the
 *     (src, dst) pair, which the caller applies with pa_copy_blocks before
 *     writing the new tokens with pa_reshape_and_cache.
 *   - Full blocks are indexed by a prefix-cumulative hash of their tokens;
 *     pa_pool_add_request reuses the cached blocks of a prompt up to the
 *     first miss (and never the block holding its last token).
 *   - Freed blocks keep their index entry and join the tail of a free queue;
 *     allocation takes the least recently used block and drops its old entry.
 * All pool calls are host-only (no GPU work) and not thread-safe per pool.
 * Host pointers throughout.
 */
typedef struct pa_block_pool pa_block_pool;

/* A new pool (NULL if num_blocks < 2 or out of memory).  Free with
 * pa_pool_destroy. */
pa_block_pool* pa_pool_create(int32_t num_blocks);
void pa_pool_destroy(pa_block_pool* pool);
/* Blocks in the free queue (unreferenced; they may still be cached). */
int32_t pa_pool_num_free(const pa_block_pool* pool);
/* Registers request `req` with its prompt (n token ids); *num_cached gets
 * the number of leading prompt tokens already held by cached blocks (a
 * multiple of 16); they need no slots.  PA_ERR_REQUEST_EXISTS if the id is
 * in use. */
int pa_pool_add_request(pa_block_pool* pool, int64_t req, const int32_t* prompt, int32_t n,
                        int32_t* num_cached);
/* Slots for the request's next n tokens, whose ids are tokens[0..n-1] (the
 * rest of a prompt past its cached part, or newly sampled tokens):
 * slot_mapping[i] = block * 16 + offset, in pa_reshape_and_cache's format.
 * copy[0..1] receives a (src, dst) copy-on-write pair when *num_copies is 1.
 * PA_ERR_NO_BLOCKS leaves the pool unchanged. */
int pa_pool_allocate_slots(pa_block_pool* pool, int64_t req, const int32_t* tokens, int32_t n,
                           int64_t* slot_mapping, int32_t* copy, int32_t* num_copies);
/* `child` shares every block of `parent` (reference counts + 1). */
int pa_pool_fork(pa_block_pool* pool, int64_t parent, int64_t child);
/* Releases the request's blocks (last block first). */
int pa_pool_free_request(pa_block_pool* pool, int64_t req);
/* The request's block table: row[0..*num_blocks-1] (at most capacity
 * entries written; *num_blocks is the full count), and its token count. */
int pa_pool_block_table(const pa_block_pool* pool, int64_t req, int32_t* row, int32_t capacity,
                        int32_t* num_blocks);
int pa_pool_num_tokens(const pa_block_pool* pool, int64_t req, int32_t* num_tokens);

/*
 * pa_copy_blocks — copies every kv head's K and V of block pairs[2i] to
 * block pairs[2i+1], raw bits (the copy-on-write copy, zihan-zhang.net vLLM
 * study, 3.2.2).  pairs: device int32 [num_pairs][2].  Pairs naming a block
 * outside the pool, or src == dst, are skipped; a block must not be both a
 * destination and a source in one call.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                   const pa_cache_desc* desc, void* stream);

/*
 * pa_prefill_chunk — causal attention of query chunks against paged KV
 * (zihan-zhang.net vLLM study, 3.5: a long prompt is processed chunk by chunk;
 * batch metadata flattens all requests' tokens into one launch).
 *
 *   q, out           device [total_q_tokens][num_q_heads][D], bf16 (pools bf16,
 *                    or PA_FP8_E4M3 with D = 128)
 *   query_start_loc  device int32 [num_reqs + 1]; request r owns query rows
 *                    query_start_loc[r] .. query_start_loc[r+1]-1 (n_r rows)
 *   context_lens     device int32 [num_reqs]; ctx_r counts the chunk, whose
 *                    K/V must already be in the pools.  Query i of request r
 *                    sits at position ctx_r - n_r + i and sees keys 0..that
 *                    position.
 *   block_tables     device int32 [num_reqs][max_blocks_per_seq]
 *   max_q_len        host bound on every n_r (sizes the grid)
 *   max_context_len  host bound on every ctx_r (sizes a split; a context
 *                    beyond it is cut to the bound when the call is split)
 *   partition_size   split-K over the keys: 0 = automatic (only with a
 *                    workspace; NULL workspace = no split), < 0 = no split,
 *                    > 0 = keys per part (a multiple of 64).  Parts of one
 *                    query tile leave partial softmax states that a second
 *                    kernel merges with the online-softmax rescale (zihan-
 *                    zhang.net vLLM study, 4.3.1), as pa_decode's split-K.
 *                    The automatic rule splits only calls of a few rows per
 *                    request (speculative verification), whose long
 *                    contexts would otherwise stream through one workgroup.
 *   workspace        device scratch of pa_prefill_chunk_workspace_bytes(...)
 *                    bytes for the same sizes and partition_size, or NULL;
 *                    a split call with a smaller one returns
 *                    PA_ERR_WORKSPACE.  Contents need no initialisation; two
 *                    calls in flight at once must not share one.
 * Uses bf16 MFMA for Q K^T and P V with fp32 accumulation and an fp32
 * online-softmax state; P is rounded to bf16 before the P V product.  fp8
 * codes are widened exactly to bf16 after the LDS read; the K scale is folded
 * into `scale` and the V scale into the normalisation.  With k + 1 rows per
 * request this is the verification attention of speculative decoding
 * (zihan-zhang.net vLLM study, 4.1.1: the target scores the k drafted
 * positions in one pass).
 */
size_t pa_prefill_chunk_workspace_bytes(int32_t num_reqs, int32_t total_q_tokens,
                                        int32_t max_q_len, int32_t max_context_len,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t partition_size);
int pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* query_start_loc, const int32_t* context_lens,
                     int32_t num_reqs, int32_t total_q_tokens, int32_t max_q_len,
                     int32_t max_context_len, int32_t num_q_heads, float scale,
                     int32_t partition_size, void* workspace, size_t workspace_bytes,
                     const pa_cache_desc* desc, void* stream);

/*
 * pa_rejection_sample — the verification step of speculative decoding
 * (zihan-zhang.net vLLM study, 4.1.1; vLLM: from PagedAttention to
 * Speculative Decoding, 5.3-5.4).  A drafter proposed num_draft = k tokens per
 * request; the target model scored the k + 1 positions in one pass (its
 * attention: pa_prefill_chunk with k + 1 query rows per request).  Candidate
 * x_i is kept with probability min(1, p_i(x_i) / q_i(x_i)); the first
 * rejection ends the round with a token drawn from the normalised
 * (p_i - q_i)_+; if all k are kept a bonus token is drawn from p_k.  The
 * emitted tokens follow the target distribution exactly.
 *
 *   target_probs  device fp32 [num_reqs][k+1][vocab]: p_0 .. p_k
 *   draft_probs   device fp32 [num_reqs][k][vocab]: q_0 .. q_{k-1}, or NULL
 *                 when drafts carry no distribution (q_i one-hot at x_i)
 *   draft_tokens  device int32 [num_reqs][k]; a token outside [0, vocab) is
 *                 never kept
 *   uniforms      device fp32 [num_reqs][k+1], in [0, 1): u_i decides
 *                 candidate i (kept iff u_i * q_i(x_i) <= p_i(x_i), exactly),
 *                 u_k draws the final token.  u_i = 1 gives the deterministic
 *                 rule "keep iff p(x) >= q(x)".
 *   out_tokens    device int32 [num_reqs][k+1]: the kept drafts, then the
 *                 drawn token, then -1 padding
 *   num_out       device int32 [num_reqs]: tokens emitted (kept + 1)
 *   workspace     device scratch of pa_rejection_sample_workspace_bytes(
 *                 num_reqs, vocab) bytes (one 64-bit weight sum per request
 *                 and 256-entry vocabulary segment); needs no initialisation;
 *                 two calls in flight at the same time must not share it
 * The final token is drawn by inverse CDF with u_k over integer weights
 * floor(max(r_j, 0) * 2^32), r_j = p_j - q_j in fp32 (NaN counts as 0), so the
 * choice is exact and independent of summation order; an empty residual draws
 * from p_i instead, and an all-zero p_k gives token -1.  Probabilities need
 * not be normalised.  Supported: k <= 32, vocab <= 2^21, num_reqs <= 65535.
 */
#define PA_MAX_DRAFT 32
#define PA_MAX_VOCAB (1 << 21)
size_t pa_rejection_sample_workspace_bytes(int32_t num_reqs, int32_t vocab);
int pa_rejection_sample(const float* target_probs, const float* draft_probs,
                        const int32_t* draft_tokens, const float* uniforms, int32_t num_reqs,
                        int32_t num_draft, int32_t vocab, int32_t* out_tokens, int32_t* num_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_bw_probe — measurement helper, not part of attention: reads num_tiles
 * 4 KiB tiles of `buf` once each, tile tile_order[i] for i = 0..num_tiles-1,
 * with the same non-temporal 16-byte loads the decode kernel uses for K/V
 * tiles.  Timing it gives the read bandwidth the device sustains for
 * scattered 4 KiB tiles, the practical ceiling beside the published HBM peak
 * (decode is bound by the bytes it moves: zihan-zhang.net vLLM study, 1.4).
 *
 *   buf         device buffer of `bytes` bytes (>= 4096)
 *   tile_order  device int32 [num_tiles]; values are clamped into the buffer
 *   sink        device uint32 [1]; written only for one improbable data value
 * Enqueued on `stream`; nothing is returned but the status.
 */
int pa_bw_probe(const void* buf, size_t bytes, const int32_t* tile_order, int32_t num_tiles,
                uint32_t* sink, void* stream);

/* Static description of a status code. */
const char* pa_status_string(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
