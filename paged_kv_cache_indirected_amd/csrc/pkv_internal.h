// Internal declarations shared by the libpkv translation units (not installed).
#pragma once

#include <cstddef>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Record a failure for pkv_last_error() and return `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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
    int32_t partition_blocks;  // blocks of context per workgroup
    int32_t max_partitions;    // grid extent over partitions
    float scale;
    void *out;
    int32_t out_dtype;
    float *ws_o;               // [B][Hq][max_partitions][D] un-normalised partial outputs
    float *ws_ml;              // [B][Hq][max_partitions][2] running max (log2 units) and sum
    void *stream;
};
int launch_decode(const DecodeLaunch &a);

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
};
int launch_prefill(const PrefillLaunch &a);

}  // namespace pkv
