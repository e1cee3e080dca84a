// Internal declarations shared by the libpkv translation units (not installed).
#pragma once

#include <cstddef>
#include <cstdint>
#include <functional>

#include "pkv.h"

namespace pkv {

// Debug builds (PKV_DEBUG, libpkv_debug.so): the kernels record the device
// preconditions they find violated in a word per kernel module (bits
// below; the release build handles the same inputs silently: blocks read
// as zeros, lengths clamped, slots and pairs skipped), and every entry
// point that enqueued work synchronises its stream and turns a set word
// into PKV_EINVAL, a device error into PKV_EHIP (debug_finish).
constexpr uint32_t kDbgBlockId = 1u;   // block id outside the pool
constexpr uint32_t kDbgLength = 2u;    // context length outside its bound, or a chunk longer
constexpr uint32_t kDbgSlot = 4u;      // append slot beyond the cache
constexpr uint32_t kDbgCopyId = 8u;    // block copy id outside its cache
#ifdef PKV_DEBUG
// Each returns and clears its module's word on the current device.
uint32_t append_debug_take();
uint32_t copy_debug_take();
uint32_t decode_debug_take();
uint32_t prefill_debug_take();
int debug_finish(int rc, void *stream, const char *who);
// Host-side checks of the distinctness preconditions, on the id lists read
// back after the call: append slots in [0, cap) distinct; copy destinations
// of the pairs copied distinct and, in place, none of them also a source.
int debug_slots(int rc, const int32_t *slots, int64_t n, int64_t cap, void *stream,
                const char *who);
int debug_copy_ids(int rc, const int32_t *src_ids, const int32_t *dst_ids, int64_t n,
                   int64_t src_nb, int64_t dst_nb, bool in_place, void *stream, const char *who);
#define PKV_FINISH(rc, stream, who) pkv::debug_finish((rc), (stream), (who))
#define PKV_CHECK_SLOTS(rc, ...) pkv::debug_slots((rc), __VA_ARGS__)
#define PKV_CHECK_COPY_IDS(rc, ...) pkv::debug_copy_ids((rc), __VA_ARGS__)
#else
#define PKV_FINISH(rc, stream, who) (rc)
#define PKV_CHECK_SLOTS(rc, ...) (rc)
#define PKV_CHECK_COPY_IDS(rc, ...) (rc)
#endif

// Record a failure for pkv_last_error() and return `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Sequences per decode launch: the kernel keeps the batch's block prefix
// sums in LDS; larger batches go in several launches.
constexpr int32_t kDecodeMaxSeqs = 1024;

// Launch arguments of the decode kernels, already validated by the C ABI.
struct DecodeLaunch {
    const void *q;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    int32_t table_stride;
    const int32_t *context_lens;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_blocks;
    int32_t block_size;
    int32_t head_dim;
    int32_t dtype;
    int32_t max_context_len;   // device lengths are clamped to this
    int32_t num_splits;        // workgroups per KV head
    float scale;
    void *out;
    int32_t out_dtype;
    int32_t *ws_pref;          // [Bc + 1] block prefix sums
    float *ws_o;               // [Hkv][W + Bc][G][D] partial outputs
    float *ws_ml;              // [Hkv][W + Bc][G][2] running max (log2 units) and sum
    const void *k_new;         // fused append (NULL: plain decode): [B][Hkv][D]
    const void *v_new;
    const int32_t *slots;      // [B]
    void *k_cache_w;           // writable views of the caches for the fused append
    void *v_cache_w;
    void *stream;
    float *lse = nullptr;      // optional [B][Hq] log2-sum-exp of the scaled scores
};
int launch_decode(const DecodeLaunch &a);
// Device address of the current device's pkv_decode_noalloc scratch
// (PKV_DECODE_NOALLOC_SCRATCH_BYTES), looked up on the first call per device.
int decode_noalloc_scratch(void **ptr);
// Runs on_main(stream) and on_side(side) so that the two may execute
// concurrently: the side stream (one per device, the library's) first waits
// for everything enqueued on `stream` so far, and `stream` then waits for
// everything launched on the side stream, so later work on `stream` sees
// both.  Host callers on one device are serialised for the sequence.
// Returns the first failing branch's code (the join is enqueued anyway).
int launch_forked(void *stream, const std::function<int(void *)> &on_main,
                  const std::function<int(void *)> &on_side);
// Cost of a sequence boundary in a decode workgroup's range, in blocks.
int32_t decode_piece_cost(int32_t block_size, int32_t head_dim, int32_t elem_size);
// out[r][d] = sum_k o[k][r][d] 2^(lse[k][r] - M) / sum_k 2^(lse[k][r] - M),
// M = max_k lse[k][r] (zeros where every state is empty), r < rows; with
// row_tokens set, only rows r < row_tokens[0] * heads are merged (the rest of
// the states' rows are padding and out holds no such rows).
int launch_merge_states(const float *o, const float *lse, int32_t k, int64_t rows,
                        int32_t head_dim, void *out, int32_t out_dtype, void *stream,
                        const int32_t *row_tokens = nullptr, int32_t heads = 0);
// Compute units of the current device (256 if it cannot be queried).
int32_t device_cu_count();

struct AppendLaunch {
    const void *k;
    const void *v;
    const int32_t *slots;
    int32_t num_tokens;
    void *k_cache;
    void *v_cache;
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t block_size;
    int32_t head_dim;
    int32_t elem_size;
    void *stream;
};
int launch_append(const AppendLaunch &a);

struct CopyLaunch {
    const void *src_k;
    const void *src_v;
    int32_t src_num_blocks;
    void *dst_k;
    void *dst_v;
    int32_t dst_num_blocks;
    const int32_t *src_ids;
    const int32_t *dst_ids;
    int32_t n;
    int64_t block_bytes;   // multiple of 16, < 2^31
    void *stream;
};
int launch_copy_blocks(const CopyLaunch &a);

struct PrefillLaunch {
    const void *q;
    const int32_t *query_start;
    int32_t num_seqs;
    int32_t max_query_len;
    const void *k_cache;
    const void *v_cache;
    const int32_t *block_tables;
    int32_t table_stride;
    const int32_t *context_lens;
    int32_t max_context_len;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_blocks;
    int32_t block_size;
    int32_t head_dim;
    float scale;
    void *out;
    int32_t out_dtype;
    void *stream;
    int32_t causal = 1;        // 0: every row attends all keys of its sequence
    int32_t q_shared = 0;      // 1: every sequence reads queries from rows 0..C-1
    float *lse = nullptr;      // optional [rows][Hq] log2-sum-exp of the scaled scores
    int32_t key_splits = 1;    // > 1: split k writes its fp32 state at out + k * split_rows * D
    int64_t split_rows = 0;    //      and its log2-sum-exp at lse + k * split_rows
    // syn_rows > 0: sequence s is range s of one block list (block_tables,
    // stride syn_nbk, syn_nb blocks in all): syn_rows query rows from row
    // s * syn_rows, min(syn_nbk, syn_nb - s * syn_nbk) blocks of keys;
    // query_start and context_lens are not read.
    int32_t syn_rows = 0, syn_nbk = 0, syn_nb = 0;
};
int launch_prefill(const PrefillLaunch &a);
// Query rows (GQA-packed (token, head) pairs) one prefill workgroup holds.
int32_t prefill_rows_per_workgroup();

}  // namespace pkv
