/*
 * pkv.h -- C ABI of libpkv: attention over a paged KV cache on AMD MI355X
 * (gfx950), plus the host-side block pool and sequence bookkeeping.
 *
 * Pages this interface follows (cited by title and section):
 *   [KV-prep]  "LLM Inference: KV Cache, Batching & Scheduling" (cariara.com)
 *   [KV-news]  "LLM Inference Engineering: Overcoming the KV-Cache Bottleneck
 *              and Maximizing Production Throughput" (wpnews.pro summary)
 *   [KV-blog]  the adilsher.pro blog post of the same title
 *
 * Conventions for every call below:
 *   - Device pointers are caller-owned, contiguous and 16-byte aligned; the
 *     library never allocates, frees or retains device memory.
 *   - Kernel calls enqueue on `stream` (a hipStream_t; NULL = the default
 *     stream) and return without synchronising.  A fault in a kernel shows up
 *     at the caller's next synchronisation.
 *   - Only host scalars and pointers are validated.  Contents of device
 *     arrays (block ids, slots, lengths) are preconditions; kernels never
 *     read or write outside the buffers the sizes describe: a block id
 *     outside [0, num_blocks) contributes nothing, a slot outside the cache
 *     is not written, and a context length is clamped to
 *     block_table_stride * block_size.
 *   - Return value: PKV_OK (0) or a negative PKV_E* code; pkv_last_error()
 *     then holds a message for the calling thread.
 *   - Debug build (libpkv_debug.so, built from the same sources with
 *     PKV_DEBUG defined; same symbols, same results): every call that
 *     enqueues device work also synchronises `stream` before it returns and
 *     then reports what the kernels found.  PKV_EHIP if the stream's work
 *     failed; PKV_EINVAL, naming each violation, if a kernel met a block id
 *     outside [0, num_blocks), a decode context length outside
 *     [0, min(block_table_stride * block_size, max_context_len)], a prefill
 *     context length outside [its chunk's length, block_table_stride *
 *     block_size], an append slot at or beyond num_blocks * block_size, or a
 *     copy id at or beyond its cache's block count; then, on the id lists
 *     read back to the host, if two rows map to one append slot, two copied
 *     pairs share a destination block, or an in-place copy (same caches)
 *     has a block that is both a source and a destination.  Negative slots
 *     and copy ids are padding there too and are not reported.  The check
 *     reads and clears flag words of the current GPU that all calls share,
 *     so debug calls must not overlap (one thread, one stream at a time),
 *     and they cannot be captured into a graph.  The release build
 *     (libpkv.so) does none of this.
 *   - Element types: q, k, v and the caches share one dtype (PKV_F32 or
 *     PKV_BF16); index arrays are int32.
 *
 * Cache layout (the pages fix none; this library's reading).  Each of
 * k_cache and v_cache holds num_blocks x num_kv_heads tiles; tile (block b,
 * KV head g) is one contiguous run of block_size * head_dim elements
 * starting at element (b * num_kv_heads + g) * block_size * head_dim.  A slot
 * s names block s / block_size, token offset s % block_size.  Inside a tile
 * the elements are NOT row-major.  With bs = block_size, D = head_dim and
 * E = 16 / element size (8 for bf16, 4 for f32), element (token t, dim d)
 * sits at tile offset
 *     K:  ((d / E) * bs + t) * E + d % E
 *         (each token's dims in 16-byte chunks, chunk-major: chunk c of all
 *         bs tokens, then chunk c + 1, ...)
 *     V:  ((t / 4) * D + d) * 4 + t % 4
 *         (4 consecutive tokens of one dim side by side, then the next dim)
 * pkv_k_elem_offset / pkv_v_elem_offset below give the full element offset.
 * pkv_append and pkv_append_decode write this layout; a cache filled any
 * other way must follow it.  Query head h reads KV head
 * h / (num_q_heads / num_kv_heads).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define PKV_OK 0
#define PKV_EINVAL (-1)       /* null pointer, bad size, misaligned pointer, short workspace */
#define PKV_EUNSUPPORTED (-2) /* dtype / head_dim / block_size / group combination not built */
#define PKV_ENOBLOCKS (-3)    /* block pool exhausted; the pool is left unchanged */
#define PKV_ESTATE (-4)       /* bookkeeping misuse: unknown id, double release, write into a shared block */
#define PKV_EHIP (-5)         /* HIP launch or runtime error */

/* Element types. */
#define PKV_F32 0
#define PKV_BF16 1

/* Shape of one layer's cache.  block_size: 16 or 32 ([KV-news] section 2,
 * [KV-prep] "PagedAttention and vLLM").  head_dim: 64 or 128. */
typedef struct pkv_cache_desc {
    int32_t num_blocks;   /* physical blocks in each of k_cache, v_cache */
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t head_dim;
    int32_t dtype;        /* PKV_F32 or PKV_BF16 */
} pkv_cache_desc;

/* Element offset of (block, KV head, token offset t, dim d) in k_cache,
 * resp. v_cache, for the layout above (no range checks). */
static inline int64_t pkv_k_elem_offset(const pkv_cache_desc *c, int32_t block, int32_t head,
                                        int32_t t, int32_t d)
{
    const int64_t bs = c->block_size, D = c->head_dim;
    const int64_t E = c->dtype == PKV_F32 ? 4 : 8;
    return ((int64_t)block * c->num_kv_heads + head) * bs * D + ((d / E) * bs + t) * E + d % E;
}
static inline int64_t pkv_v_elem_offset(const pkv_cache_desc *c, int32_t block, int32_t head,
                                        int32_t t, int32_t d)
{
    const int64_t bs = c->block_size, D = c->head_dim;
    return ((int64_t)block * c->num_kv_heads + head) * bs * D + ((int64_t)(t / 4) * D + d) * 4 +
           t % 4;
}

/* Static text for a return code. */
const char *pkv_strerror(int code);
/* Detail message of the calling thread's last failed call ("" if none). */
const char *pkv_last_error(void);
/* ABI version of this header (bumped on incompatible change). */
int pkv_abi_version(void);
#define PKV_ABI_VERSION 2

/* ------------------------------------------------------------------------
 * KV append ([KV-prep] "The KV cache": the new token's K and V are appended
 * each step).
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim], cache dtype
 *   slot_mapping  [num_tokens] int32; row t goes to slot slot_mapping[t];
 *                 a negative slot, or one at or past num_blocks * block_size,
 *                 skips the row.  Slots must be distinct.
 *   k_cache, v_cache  the caches described by `c`
 * Copies bits; no conversion.  num_tokens == 0 is a no-op.  Rows 4t .. 4t+3
 * mapped to 4 consecutive slots starting at a multiple of 4 (the rows of a
 * prompt or a prefill chunk) are written as whole cache lines; other rows
 * one by one.
 */
int pkv_append(const void *k, const void *v, const int32_t *slot_mapping, int32_t num_tokens,
               void *k_cache, void *v_cache, const pkv_cache_desc *c, void *stream);

/* ------------------------------------------------------------------------
 * Block copy.  Sequences with an identical prefix share its pages ([KV-news]
 * section 2, [KV-blog] "The Elegant Fix"); before one of them writes into a
 * shared, partially filled block it needs a private copy (copy-on-write, this
 * library's reading: the pages say nothing of writes to shared pages).  The
 * same call moves blocks to or from a second cache of the same block shape,
 * e.g. a swap area in pinned host memory.
 *
 *   src_k, src_v, src_c  source caches and their descriptor
 *   dst_k, dst_v, dst_c  destination caches (may be the source caches); the
 *                        descriptors must agree in num_kv_heads, block_size,
 *                        head_dim and dtype
 *   src_ids, dst_ids     [n] int32, device-readable: block dst_ids[i] of the
 *                        destination receives block src_ids[i] of the source
 *                        (K and V, every KV head and offset).  A pair with an
 *                        id outside its cache is skipped.  Destination blocks
 *                        must be distinct and, when the caches are the same,
 *                        disjoint from the source blocks.
 * Copies bits.  n == 0 is a no-op.
 */
int pkv_copy_blocks(const void *src_k, const void *src_v, const pkv_cache_desc *src_c,
                    void *dst_k, void *dst_v, const pkv_cache_desc *dst_c,
                    const int32_t *src_ids, const int32_t *dst_ids, int32_t n, void *stream);

/* ------------------------------------------------------------------------
 * Paged decode attention ([KV-prep] "The KV cache": the query attends the
 * keys and values of every prior position; [KV-news] section 2 and
 * [KV-prep] "PagedAttention and vLLM": those positions live in fixed-size
 * blocks that a per-sequence table maps from logical to physical).
 *
 * For sequence b and query head h (KV head g = h / G, G = num_q_heads /
 * num_kv_heads), with L = context_lens[b] and key/value j read from block
 * block_tables[b * block_table_stride + j / block_size], offset
 * j % block_size:
 *     out[b][h][:] = sum_j softmax_j(scale * q[b][h] . K_j) * V_j[:]
 * over j in [0, L); L == 0 gives zeros.  Accumulation is fp32.
 *
 *   q             [num_seqs][num_q_heads][head_dim], cache dtype
 *   block_tables  [num_seqs][block_table_stride] int32; entries past
 *                 ceil(L / block_size) are not read
 *   context_lens  [num_seqs] int32
 *   max_context_len  host-side upper bound of context_lens (sizes the split;
 *                 a longer device length is clamped to it)
 *   out           [num_seqs][num_q_heads][head_dim]; out_dtype PKV_F32 or
 *                 PKV_BF16 (round to nearest even)
 *   num_splits    workgroups per KV head; 0 = library choice
 *                 (pkv_decode_num_splits).  The blocks of all sequences are
 *                 laid end to end and cut into num_splits equal ranges, so
 *                 every workgroup reads the same number of K/V bytes; a
 *                 sequence cut between ranges is finished by a log-sum-exp
 *                 merge pass (a second, small launch).  The result depends on num_splits only through
 *                 fp32 rounding, and is bitwise reproducible for a given
 *                 (context_lens, num_splits).
 *   workspace     device scratch of at least pkv_decode_workspace_bytes(...)
 *                 bytes (never NULL for num_seqs > 0); its contents need no
 *                 initialisation and are overwritten.  Calls that share a
 *                 workspace must not run concurrently.
 * Sequences are processed in launches of at most 1024; num_seqs may be
 * larger.  Supported: dtype F32/BF16, head_dim 64/128, block_size 16/32,
 * G in {1, 2, 4, 8}.
 */
int32_t pkv_decode_num_splits(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                              const pkv_cache_desc *c);
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                  int32_t num_splits, const pkv_cache_desc *c);
int pkv_decode(const void *q, const void *k_cache, const void *v_cache,
               const int32_t *block_tables, int32_t block_table_stride,
               const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
               int32_t max_context_len, float scale, void *out, int32_t out_dtype,
               int32_t num_splits, void *workspace, size_t workspace_bytes,
               const pkv_cache_desc *c, void *stream);

/* ------------------------------------------------------------------------
 * pkv_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, computation and result as pkv_decode with the same
 * num_splits (bit for bit), without the workspace: the split partials live
 * in a scratch area inside the library, PKV_DECODE_NOALLOC_SCRATCH_BYTES on
 * each GPU it runs on, held until the process ends.  A call whose partials
 * need more (pkv_decode_workspace_bytes(...) above the limit) returns
 * PKV_EINVAL; pkv_decode with a caller workspace has no such limit.  The
 * scratch address is looked up once per device, on the first call with that
 * device current.  Every call on one GPU shares that GPU's scratch: calls
 * that overlap on one GPU (two streams, two host threads) race and give
 * wrong results; order them.  Nothing needs clearing between calls.
 */
#define PKV_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int pkv_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, int32_t block_table_stride,
                       const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_context_len, float scale, void *out, int32_t out_dtype,
                       int32_t num_splits, const pkv_cache_desc *c, void *stream);

/* ------------------------------------------------------------------------
 * Decode step with the append fused into the same launch.
 *
 * Same result, cache contents included, as
 *     pkv_append(k_new, v_new, slot_mapping, num_seqs, k_cache, v_cache, c)
 *     pkv_decode(q, k_cache, ..., context_lens, num_seqs, ...)
 * for a decode step in which sequence b appends one token (row b of k_new,
 * v_new: [num_seqs][num_kv_heads][head_dim]) at slot slot_mapping[b], and
 * that token is position context_lens[b] - 1 of the sequence (the slot the
 * block table maps that position to: a precondition).  A negative slot
 * appends nothing, and position L - 1 is then read from the cache.  The new
 * rows are written to the cache and, for the attention, taken from k_new /
 * v_new directly, so nothing in the launch reads what it writes.  One launch
 * fewer per step than the two calls ([KV-prep] "The KV cache": append, then
 * attend).  Other arguments, workspace and return codes as pkv_decode.
 */
int pkv_append_decode(const void *k_new, const void *v_new, const int32_t *slot_mapping,
                      const void *q, void *k_cache, void *v_cache, const int32_t *block_tables,
                      int32_t block_table_stride, const int32_t *context_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t max_context_len, float scale, void *out,
                      int32_t out_dtype, int32_t num_splits, void *workspace,
                      size_t workspace_bytes, const pkv_cache_desc *c, void *stream);

/* ------------------------------------------------------------------------
 * Cascade decode over a shared prefix ([KV-news] section 2 and [KV-blog]
 * "The Elegant Fix": sequences with an identical prefix share its pages;
 * [KV-prep] "Prefix caching").  Reading every shared block once per sharer
 * is what plain decode does; here the shared prefix's blocks are read once
 * for all sequences of the call.
 *
 * Sequence b attends prefix_len tokens held in prefix_blocks ([prefix_len /
 * block_size] int32, device) followed by its own context_lens[b] tokens in
 * block_tables[b] (which lists only its own blocks).  The result equals
 * pkv_decode over the concatenated block lists, up to rounding order.
 * prefix_len must be a whole number of blocks (0 allowed).  The prefix runs
 * as a non-causal MFMA pass over all sequences' queries, split over ranges
 * of prefix blocks; the suffixes as the split decode; the states are merged
 * by log-sum-exp.  bf16 caches only (PKV_EUNSUPPORTED otherwise).  Other
 * arguments as pkv_decode (max_context_len bounds context_lens); the
 * workspace (size from pkv_decode_cascade_workspace_bytes) needs no
 * initialisation, and calls sharing one must not overlap.
 *
 * Streams: the suffix decode runs on `stream`; the prefix pass runs beside
 * it on a stream the library creates once per device (default priority,
 * non-blocking), which first waits for all work enqueued on `stream` before
 * the call, and `stream` then waits for it before the state merge.  To the
 * caller the call is ordered on `stream` like any other, also under HIP
 * graph capture (the side branch is captured through the two events).
 * Host threads calling it on one device are serialised while they enqueue.
 */
size_t pkv_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                          int32_t prefix_len, int32_t max_context_len,
                                          const pkv_cache_desc *c);
int pkv_decode_cascade(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *prefix_blocks, int32_t prefix_len,
                       const int32_t *block_tables, int32_t block_table_stride,
                       const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_context_len, float scale, void *out, int32_t out_dtype,
                       void *workspace, size_t workspace_bytes, const pkv_cache_desc *c,
                       void *stream);

/* ------------------------------------------------------------------------
 * Causal chunked prefill ([KV-prep] "Chunked prefill": a prompt is split into
 * fixed-size chunks, e.g. 512 tokens, interleaved with decode; the split does
 * not change the result).
 *
 * Sequence b contributes C_b = query_start_loc[b+1] - query_start_loc[b]
 * query rows; its chunk's K/V is already appended, so context_lens[b] (L_b)
 * counts it.  Chunk row i (0 <= i < C_b) attends keys [0, L_b - C_b + i],
 * diagonal included.  QK^T and PV run on bf16 MFMA with fp32 accumulation.
 *
 *   q                [query_start_loc[num_seqs]][num_q_heads][head_dim] bf16
 *   query_start_loc  [num_seqs + 1] int32, non-decreasing, starts at 0
 *   max_query_len    host-side upper bound of C_b
 *   out              like q, out_dtype PKV_F32 or PKV_BF16
 *   workspace        caller-owned device memory of workspace_bytes bytes, no
 *                    initialisation needed; may be NULL.
 * Key splits.  When the grid (num_kv_heads x num_seqs x q-tiles workgroups)
 * has fewer workgroups than the device has compute units (a short chunk of
 * one or a few sequences), the keys of each workgroup are split k ways; every split writes an fp32 state (normalised output and
 * log2-sum-exp) into the workspace and a log-sum-exp merge writes out.  The
 * result equals the single pass up to fp32 rounding order.
 * pkv_prefill_workspace_bytes gives the bytes for the largest split the
 * library would choose for these sizes (0: it would not split); a NULL or
 * shorter workspace makes it split less or not at all.  Calls sharing a
 * workspace must not overlap.
 * Supported: dtype BF16 only (PKV_EUNSUPPORTED for F32), head_dim 64/128,
 * block_size 16/32, G in {1, 2, 4, 8}.
 */
size_t pkv_prefill_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t max_query_len,
                                   const pkv_cache_desc *c);
int pkv_prefill_chunk(const void *q, const int32_t *query_start_loc, int32_t num_seqs,
                      int32_t max_query_len, const void *k_cache, const void *v_cache,
                      const int32_t *block_tables, int32_t block_table_stride,
                      const int32_t *context_lens, int32_t max_context_len,
                      int32_t num_q_heads, float scale, void *out, int32_t out_dtype,
                      void *workspace, size_t workspace_bytes, const pkv_cache_desc *c,
                      void *stream);

/* ------------------------------------------------------------------------
 * Host block pool ([KV-prep] "PagedAttention and vLLM": pages are allocated
 * on demand and a finished request's pages return to the pool at once;
 * [KV-news] section 2 and [KV-blog] "The Elegant Fix": identical prefixes
 * share pages).  Single-threaded; the caller owns the handle.
 */
typedef struct pkv_pool pkv_pool;

/* seed 0: free list in ascending id order; otherwise a permutation drawn
 * from the seed.  Returns NULL on bad arguments or allocation failure. */
pkv_pool *pkv_pool_create(int32_t num_blocks, uint64_t seed);
void pkv_pool_destroy(pkv_pool *pool);
/* Pop n blocks from the front of the free list (refcount 1 each) into ids.
 * All-or-nothing: PKV_ENOBLOCKS leaves the pool unchanged. */
int pkv_pool_alloc(pkv_pool *pool, int32_t n, int32_t *ids);
/* Add one reference to each of n allocated blocks (PKV_ESTATE if any is
 * free or unknown; then nothing changes). */
int pkv_pool_share(pkv_pool *pool, int32_t n, const int32_t *ids);
/* Drop one reference from each of n blocks; a block reaching 0 returns to the
 * back of the free list, or, if the prefix cache holds it, to the back of the
 * cache's LRU list.  PKV_ESTATE if any id is free or unknown, or appears
 * more often than its refcount; then nothing changes. */
int pkv_pool_release(pkv_pool *pool, int32_t n, const int32_t *ids);
/* Blocks that can be handed out: the free list plus unreferenced blocks kept
 * by the prefix cache (those are reused, least recently released first, only
 * once the free list is empty). */
int32_t pkv_pool_num_free(const pkv_pool *pool);
/* Unreferenced blocks kept by the prefix cache. */
int32_t pkv_pool_num_cached(const pkv_pool *pool);
int32_t pkv_pool_num_blocks(const pkv_pool *pool);
/* Refcount of a block (0 = free or kept only by the prefix cache), or -1 for
 * an id outside the pool. */
int32_t pkv_pool_refcount(const pkv_pool *pool, int32_t id);

/* ------------------------------------------------------------------------
 * Sequence bookkeeping over a pool (continuous batching, [KV-prep]
 * "Continuous batching (Orca)": sequences join and leave at every step).
 * A sequence is a caller-chosen int64 id with a length and a list of block
 * ids.  The pool must outlive the set.
 */
typedef struct pkv_seqs pkv_seqs;

typedef struct pkv_seqs_stats {
    int32_t num_seqs;
    int64_t blocks_referenced;   /* sum over sequences of their block counts */
    int32_t blocks_in_use;       /* pool blocks with refcount > 0 */
    int64_t tokens;              /* sum of lengths */
    int64_t slots_unused;        /* reserved but unused slots in last blocks
                                    ([KV-prep] "internal fragmentation") */
} pkv_seqs_stats;

pkv_seqs *pkv_seqs_create(pkv_pool *pool, int32_t block_size);
void pkv_seqs_destroy(pkv_seqs *seqs);
/* New empty sequence; PKV_ESTATE if the id exists. */
int pkv_seqs_add(pkv_seqs *seqs, int64_t seq_id);
/* New sequence whose first num_tokens positions share the physical blocks of
 * sequence src_id (num_tokens a multiple of block_size and <= its length):
 * the blocks gain a reference and are read-only for both. */
int pkv_seqs_add_shared(pkv_seqs *seqs, int64_t seq_id, int64_t src_id, int32_t num_tokens);
/* Extend a sequence by n tokens; slots[0..n) receive their slots.  New blocks
 * come from the pool when a block boundary is crossed; all-or-nothing
 * (PKV_ENOBLOCKS).  PKV_ESTATE if a slot would land in a block with
 * refcount > 1. */
int pkv_seqs_append(pkv_seqs *seqs, int64_t seq_id, int32_t n, int32_t *slots);
/* One token for each of n sequences (a decode step); slots[i] for seq_ids[i].
 * All-or-nothing across the batch. */
int pkv_seqs_append_batch(pkv_seqs *seqs, int32_t n, const int64_t *seq_ids, int32_t *slots);
/* New sequence holding all of src_id's blocks, the partially filled last one
 * included (parallel sampling, beam search): every block gains a reference.
 * The first append of either sequence into the shared last block must go
 * through pkv_seqs_append_cow. */
int pkv_seqs_fork(pkv_seqs *seqs, int64_t seq_id, int64_t src_id);
/* pkv_seqs_append / pkv_seqs_append_batch with copy-on-write: a sequence
 * whose slot would land in a shared, partially filled last block first gets
 * a fresh block in its place, and the pair (old, new) is written to
 * copy_src[c], copy_dst[c] (room for 1 pair, resp. n pairs); *num_copies
 * receives the count.  The caller copies those blocks (pkv_copy_blocks)
 * before the new tokens are written.  In a batch, copies are decided in
 * order: if every holder of a shared block is in the batch, the last one
 * keeps the original.  Allocation is all-or-nothing (PKV_ENOBLOCKS). */
int pkv_seqs_append_cow(pkv_seqs *seqs, int64_t seq_id, int32_t n, int32_t *slots,
                        int32_t *copy_src, int32_t *copy_dst, int32_t *num_copies);
int pkv_seqs_append_batch_cow(pkv_seqs *seqs, int32_t n, const int64_t *seq_ids, int32_t *slots,
                              int32_t *copy_src, int32_t *copy_dst, int32_t *num_copies);

/* Prefix cache ([KV-prep] "Prefix caching": a prefix shared by many requests
 * is computed once and later requests pay only for the tokens after it).
 * Full blocks are registered under a chained key of their token ids (the key
 * of block j covers tokens [0, (j+1) * block_size)); a lookup compares the
 * stored ids, so a hash collision never returns wrong data.
 *
 * pkv_seqs_add_cached: new sequence for a prompt of n token ids; it takes
 * the longest run of registered blocks matching the prompt's leading whole
 * blocks, at most (n - 1) / block_size of them so that at least one token is
 * left to compute.  Returns the number of tokens reused (the new sequence's
 * length, a multiple of block_size) or a negative code.
 * pkv_seqs_cache: register the sequence's full blocks holding tokens[0, n)
 * (n <= its length; a partial last block is not registered).  The caller
 * states that those blocks hold the KV of exactly these token ids.  A block
 * registered earlier under other contents is re-registered. */
int32_t pkv_seqs_add_cached(pkv_seqs *seqs, int64_t seq_id, const int32_t *tokens, int32_t n);
int pkv_seqs_cache(pkv_seqs *seqs, int64_t seq_id, const int32_t *tokens, int32_t n);
/* Swap ([KV-prep] "The KV cache": running out of KV memory stalls new
 * requests or forces preemption of running ones; this is the preemption that
 * keeps the KV instead of recomputing it).  `host` is a second pool whose ids
 * name blocks of a host-side cache of the same block shape (e.g. pinned host
 * memory); it must outlive the sequences swapped into it.
 *
 * pkv_seqs_swap_out: the blocks the sequence holds alone (refcount 1) get a
 * host slot each and their device blocks return to the device pool; shared
 * blocks stay resident and referenced.  Pair k is (dev_ids[k], host_ids[k]),
 * *n pairs (cap >= the sequence's block count always suffices).  The caller
 * copies those blocks device -> host (pkv_copy_blocks) on the stream before
 * any later work that may write the freed device blocks.  All-or-nothing:
 * PKV_ENOBLOCKS if the host pool is short.
 * pkv_seqs_swap_in: fresh device blocks for the swapped blocks, pairs
 * (host_ids[k], dev_ids[k]) to copy host -> device, host slots released.
 * All-or-nothing: PKV_ENOBLOCKS if the device pool is short.
 * While swapped out a sequence can only be swapped in, released, queried for
 * its length or block list (host slots in place of the moved blocks) and
 * counted; every other call on it returns PKV_ESTATE.  Recompute-style
 * preemption needs no call of its own: release the sequence and admit it
 * again later (pkv_seqs_add_cached reuses whatever stayed cached). */
int pkv_seqs_swap_out(pkv_seqs *seqs, int64_t seq_id, pkv_pool *host, int32_t cap,
                      int32_t *dev_ids, int32_t *host_ids, int32_t *n);
int pkv_seqs_swap_in(pkv_seqs *seqs, int64_t seq_id, int32_t cap, int32_t *host_ids,
                     int32_t *dev_ids, int32_t *n);
/* 1 if swapped out, 0 if resident, -1 if unknown. */
int pkv_seqs_is_swapped(const pkv_seqs *seqs, int64_t seq_id);
/* Remove a sequence and drop its block references at once (host slots of a
 * swapped-out sequence return to its host pool). */
int pkv_seqs_release(pkv_seqs *seqs, int64_t seq_id);
/* Length of a sequence, or -1 if unknown. */
int32_t pkv_seqs_len(const pkv_seqs *seqs, int64_t seq_id);
/* Copy up to cap block ids of a sequence into ids; returns the count, or a
 * negative code. */
int32_t pkv_seqs_block_ids(const pkv_seqs *seqs, int64_t seq_id, int32_t cap, int32_t *ids);
/* Fill block_tables[i][0..stride) (padding -1) and context_lens[i] for the
 * listed sequences, ready to copy to the device.  PKV_EINVAL if a sequence
 * needs more than stride blocks. */
int pkv_seqs_fill(const pkv_seqs *seqs, int32_t n, const int64_t *seq_ids,
                  int32_t *block_tables, int32_t stride, int32_t *context_lens);
int pkv_seqs_stats_get(const pkv_seqs *seqs, pkv_seqs_stats *out);

/* ------------------------------------------------------------------------
 * Token-budget step scheduler ([KV-prep] "Continuous batching (Orca)":
 * sequences join and leave every step; "Chunked prefill": prompts are split
 * into fixed-size chunks, e.g. 512 tokens, that share steps with decode
 * tokens; "The KV cache" warning: when KV memory runs out new requests stall
 * or running ones are preempted).  The scheduler owns the sequences it
 * creates in `seqs` (ids are the request ids); single-threaded.
 *
 * Each step, under token_budget tokens: finished sequences of the previous
 * step are released; every running sequence whose prompt is complete gets
 * one decode token (admission order); the rest of the budget goes to prefill
 * chunks of at most chunk_tokens, first to running sequences still
 * prefilling, then to queued requests admitted first come first served (at
 * most max_running sequences run).  If the pool cannot hold the plan, queued
 * requests stall; if running sequences alone do not fit, the most recently
 * admitted is preempted by recompute (blocks released, back to the front of
 * the queue with its progress reset).  The step's slots are allocated from
 * the pool (pkv_seqs_append); the caller then appends the rows (pkv_append),
 * runs pkv_prefill_chunk over the chunks and pkv_decode over the decode
 * sequences, with block tables from pkv_seqs_fill.
 *
 * A request generates max_new_tokens tokens: the first when its prompt's
 * last chunk is processed (listed in first_ids: the time-to-first-token
 * event), then one per decode step.  It is listed in finished_ids in the
 * step that produces its last token and released at the next step.
 */
typedef struct pkv_sched pkv_sched;

typedef struct pkv_step_plan {
    /* Caller-provided arrays: max_running entries each, except chunk_slots
     * (token_budget entries). */
    int64_t *decode_ids;      /* sequences with one decode token this step */
    int32_t *decode_slots;    /* the slot of that token */
    int64_t *chunk_ids;       /* sequences with a prefill chunk this step */
    int32_t *chunk_prior;     /* prompt tokens already in the cache before the chunk */
    int32_t *chunk_len;       /* chunk tokens */
    int32_t *chunk_slots;     /* slots of all chunk tokens, chunk after chunk */
    int64_t *first_ids;       /* prompt completed this step (first token) */
    int64_t *finished_ids;    /* last token produced this step */
    int64_t *preempted_ids;   /* preempted (recompute) while planning this step */
    /* Counts written by pkv_sched_step. */
    int32_t n_decode, n_chunks, n_chunk_tokens, n_first, n_finished, n_preempted;
} pkv_step_plan;

pkv_sched *pkv_sched_create(pkv_pool *pool, pkv_seqs *seqs, int32_t block_size,
                            int32_t token_budget, int32_t chunk_tokens, int32_t max_running);
void pkv_sched_destroy(pkv_sched *sched);
/* Queue a request; PKV_ESTATE if the id is queued or is a sequence of seqs. */
int pkv_sched_submit(pkv_sched *sched, int64_t req_id, int32_t prompt_len,
                     int32_t max_new_tokens);
int pkv_sched_step(pkv_sched *sched, pkv_step_plan *plan);
int32_t pkv_sched_num_waiting(const pkv_sched *sched);
int32_t pkv_sched_num_running(const pkv_sched *sched);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
