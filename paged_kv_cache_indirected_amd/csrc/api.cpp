// C ABI entry points of libpkv: argument validation, launch geometry and
// workspace sizing.  Every step of the computation runs in the HIP kernels;
// this file only checks host scalars and pointers and picks launch shapes.
#include <algorithm>
#include <cmath>

#include "pkv_internal.h"

using pkv::fail;

namespace {

int check_desc(const pkv_cache_desc *c, const char *who)
{
    if (!c)
        return fail(PKV_EINVAL, "%s: null cache descriptor", who);
    if (c->num_blocks <= 0 || c->num_kv_heads <= 0)
        return fail(PKV_EINVAL, "%s: num_blocks %d and num_kv_heads %d must be positive", who,
                    c->num_blocks, c->num_kv_heads);
    if (c->dtype != PKV_F32 && c->dtype != PKV_BF16)
        return fail(PKV_EUNSUPPORTED, "%s: dtype %d", who, c->dtype);
    if (c->head_dim != 64 && c->head_dim != 128)
        return fail(PKV_EUNSUPPORTED, "%s: head_dim %d (64 or 128)", who, c->head_dim);
    if (c->block_size != 16 && c->block_size != 32)
        return fail(PKV_EUNSUPPORTED, "%s: block_size %d (16 or 32)", who, c->block_size);
    if ((int64_t)c->num_blocks * c->block_size > INT32_MAX)
        return fail(PKV_EINVAL, "%s: num_blocks * block_size exceeds int32 slots", who);
    return PKV_OK;
}

int elem_size(int32_t dtype) { return dtype == PKV_F32 ? 4 : 2; }

int check_ptr(const void *p, const char *what, const char *who)
{
    if (!p)
        return fail(PKV_EINVAL, "%s: %s is NULL", who, what);
    if (!pkv::aligned16(p))
        return fail(PKV_EINVAL, "%s: %s is not 16-byte aligned", who, what);
    return PKV_OK;
}

int check_heads(int32_t hq, const pkv_cache_desc *c, const char *who)
{
    if (hq <= 0 || hq % c->num_kv_heads != 0)
        return fail(PKV_EINVAL, "%s: num_q_heads %d is not a positive multiple of num_kv_heads %d",
                    who, hq, c->num_kv_heads);
    const int32_t G = hq / c->num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(PKV_EUNSUPPORTED, "%s: query group %d (1, 2, 4 or 8)", who, G);
    return PKV_OK;
}

// Decode split: W workgroups per KV head cut the batch's blocks into equal
// ranges.  W = one resident workgroup per CU for the KV heads together
// (kGroupsPerCU): more ranges only add pieces to merge and per-piece
// start-up, fewer leave CUs idle.  Measured on the Llama-70B-shaped batch
// with the current kernel: 32 per KV head 56.8 us per call, 24 to 64 per KV
// head 57.6 to 68.7 us; on the 256-sequence continuous-batching step 32 per
// KV head 0.215 ms against 0.227 to 0.260 ms.
constexpr int kGroupsPerCU = 1;

int64_t blocks_bound(int32_t num_seqs, int32_t max_ctx, const pkv_cache_desc *c)
{
    const int64_t bc = num_seqs < pkv::kDecodeMaxSeqs ? num_seqs : pkv::kDecodeMaxSeqs;
    const int64_t ctx = max_ctx > 0 ? max_ctx : 0;
    return bc * ((ctx + c->block_size - 1) / c->block_size);
}

int32_t auto_splits(int32_t num_seqs, int32_t max_ctx, const pkv_cache_desc *c)
{
    (void)num_seqs;
    (void)max_ctx;
    int64_t w = ((int64_t)pkv::device_cu_count() * kGroupsPerCU + c->num_kv_heads - 1) /
                c->num_kv_heads;
    w = w < 1 ? 1 : (w > 65535 ? 65535 : w);
    return (int32_t)w;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: block prefix sums [Bc + 1] int32, then partial outputs
// [W + Bc][Hq][D] and (m, l) [W + Bc][Hq][2] fp32, Bc = min(B, kDecodeMaxSeqs).
struct WsLayout {
    size_t pref, o, ml, total;
};

WsLayout ws_layout(int32_t B, int32_t hq, int32_t W, int32_t D)
{
    const size_t bc = (size_t)(B < pkv::kDecodeMaxSeqs ? B : pkv::kDecodeMaxSeqs);
    const size_t pieces = (size_t)W + bc;
    WsLayout l;
    l.pref = 0;
    l.o = align256((bc + 1) * sizeof(int32_t));
    l.ml = l.o + align256(pieces * hq * D * sizeof(float));
    l.total = l.ml + pieces * hq * 2 * sizeof(float);
    return l;
}

// Key splits of a chunked prefill.  The grid has Hkv * S * q-tiles
// workgroups; when that is fewer than the device's CUs (a short chunk of one
// or a few sequences), CUs sit idle for the whole call.  Splitting each
// workgroup's keys k ways (each split writes an fp32 state and its
// log2-sum-exp, merged afterwards) gives about one workgroup per CU, keeping
// at least 8 key tiles of 64 per split.  Larger grids are not split: a CU
// left with one workgroup in a partly full last round runs it about twice as
// fast, so the tail costs less than the states' traffic and the merge.
// max_ctx < 0: no bound from the context (the workspace size query).
int32_t prefill_key_splits(int32_t S, int32_t hq, int32_t maxq, int64_t max_ctx,
                           const pkv_cache_desc *c)
{
    if (S <= 0 || maxq <= 0 || hq <= 0 || !c || c->num_kv_heads <= 0)
        return 1;
    const int64_t tq = pkv::prefill_rows_per_workgroup() / (hq / c->num_kv_heads);
    const int64_t nqt = (maxq + tq - 1) / tq;
    const int64_t items = (int64_t)c->num_kv_heads * S * nqt;
    int64_t ks = (int64_t)pkv::device_cu_count() / items;
    if (max_ctx >= 0)
        ks = std::min<int64_t>(ks, (max_ctx + 63) / 64 / 8);
    ks = std::min<int64_t>(ks, 16);
    ks = std::min<int64_t>(ks, 65535 / std::max<int64_t>(nqt, 1));
    return (int32_t)std::max<int64_t>(ks, 1);
}

// Prefill split states: fp32 outputs [ks][S * maxq * Hq][D], then
// log2-sum-exp [ks][S * maxq * Hq].
struct PrefillWs {
    int64_t rows;
    size_t o, lse, total;
};

PrefillWs prefill_layout(int32_t S, int32_t hq, int32_t maxq, int32_t D, int32_t ks)
{
    PrefillWs l;
    l.rows = (int64_t)S * maxq * hq;
    l.o = 0;
    l.lse = align256((size_t)ks * l.rows * D * sizeof(float));
    l.total = l.lse + align256((size_t)ks * l.rows * sizeof(float));
    return l;
}

}  // namespace

extern "C" int pkv_append(const void *k, const void *v, const int32_t *slot_mapping,
                          int32_t num_tokens, void *k_cache, void *v_cache,
                          const pkv_cache_desc *c, void *stream)
{
    static const char *who = "pkv_append";
    pkv::clear_error();
    int rc = check_desc(c, who);
    if (rc)
        return rc;
    if (num_tokens < 0)
        return fail(PKV_EINVAL, "%s: num_tokens %d", who, num_tokens);
    if (num_tokens == 0)
        return PKV_OK;
    if ((rc = check_ptr(k, "k", who)) || (rc = check_ptr(v, "v", who)) ||
        (rc = check_ptr(k_cache, "k_cache", who)) || (rc = check_ptr(v_cache, "v_cache", who)))
        return rc;
    if (!slot_mapping)
        return fail(PKV_EINVAL, "%s: slot_mapping is NULL", who);
    pkv::AppendLaunch a{k, v, slot_mapping, num_tokens, k_cache, v_cache, c->num_blocks,
                        c->num_kv_heads, c->block_size, c->head_dim, elem_size(c->dtype), stream};
    rc = PKV_FINISH(pkv::launch_append(a), stream, who);
    return PKV_CHECK_SLOTS(rc, slot_mapping, num_tokens,
                           (int64_t)c->num_blocks * c->block_size, stream, who);
}

extern "C" int pkv_copy_blocks(const void *src_k, const void *src_v, const pkv_cache_desc *src_c,
                               void *dst_k, void *dst_v, const pkv_cache_desc *dst_c,
                               const int32_t *src_ids, const int32_t *dst_ids, int32_t n,
                               void *stream)
{
    static const char *who = "pkv_copy_blocks";
    pkv::clear_error();
    int rc;
    if ((rc = check_desc(src_c, who)) || (rc = check_desc(dst_c, who)))
        return rc;
    if (src_c->num_kv_heads != dst_c->num_kv_heads || src_c->block_size != dst_c->block_size ||
        src_c->head_dim != dst_c->head_dim || src_c->dtype != dst_c->dtype)
        return fail(PKV_EINVAL, "%s: source and destination blocks differ in shape or dtype", who);
    if (n < 0)
        return fail(PKV_EINVAL, "%s: n %d", who, n);
    if (n == 0)
        return PKV_OK;
    if ((rc = check_ptr(src_k, "src_k", who)) || (rc = check_ptr(src_v, "src_v", who)) ||
        (rc = check_ptr(dst_k, "dst_k", who)) || (rc = check_ptr(dst_v, "dst_v", who)))
        return rc;
    if (!src_ids || !dst_ids)
        return fail(PKV_EINVAL, "%s: block id list is NULL", who);
    const int64_t block_bytes = (int64_t)src_c->num_kv_heads * src_c->block_size *
                                src_c->head_dim * elem_size(src_c->dtype);
    if (block_bytes > INT32_MAX / 2)
        return fail(PKV_EINVAL, "%s: block of %lld bytes is too large", who,
                    (long long)block_bytes);
    pkv::CopyLaunch a{src_k, src_v, src_c->num_blocks, dst_k, dst_v, dst_c->num_blocks,
                      src_ids, dst_ids, n, block_bytes, stream};
    rc = PKV_FINISH(pkv::launch_copy_blocks(a), stream, who);
    return PKV_CHECK_COPY_IDS(rc, src_ids, dst_ids, n, src_c->num_blocks, dst_c->num_blocks,
                              src_k == dst_k || src_v == dst_v, stream, who);
}

extern "C" int32_t pkv_decode_num_splits(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t max_context_len, const pkv_cache_desc *c)
{
    (void)num_q_heads;
    if (check_desc(c, "pkv_decode_num_splits") || num_seqs < 0)
        return 0;
    return auto_splits(num_seqs, max_context_len, c);
}

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t max_context_len, int32_t num_splits,
                                             const pkv_cache_desc *c)
{
    if (check_desc(c, "pkv_decode_workspace_bytes") || num_seqs <= 0 || num_q_heads <= 0 ||
        num_splits < 0)
        return 0;
    const int32_t W = num_splits > 0 ? num_splits : auto_splits(num_seqs, max_context_len, c);
    return ws_layout(num_seqs, num_q_heads, W, c->head_dim).total;
}

namespace {

// Validation and launch shared by pkv_decode and pkv_append_decode (k_new
// NULL for the plain decode).
int decode_call(const char *who, const void *q, const void *k_cache, const void *v_cache,
                const int32_t *block_tables, int32_t block_table_stride,
                const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                int32_t max_context_len, float scale, void *out, int32_t out_dtype,
                int32_t num_splits, void *workspace, size_t workspace_bytes,
                const pkv_cache_desc *c, void *stream, const void *k_new, const void *v_new,
                const int32_t *slots, float *lse = nullptr, bool launch = true)
{
    int rc = check_desc(c, who);
    if (rc || (rc = check_heads(num_q_heads, c, who)))
        return rc;
    if (num_seqs < 0)
        return fail(PKV_EINVAL, "%s: num_seqs %d", who, num_seqs);
    if (out_dtype != PKV_F32 && out_dtype != PKV_BF16)
        return fail(PKV_EINVAL, "%s: out_dtype %d", who, out_dtype);
    if (!std::isfinite(scale))
        return fail(PKV_EINVAL, "%s: scale is not finite", who);
    if (num_seqs == 0)
        return PKV_OK;
    if (block_table_stride <= 0 || max_context_len < 0 ||
        (int64_t)max_context_len > (int64_t)block_table_stride * c->block_size)
        return fail(PKV_EINVAL,
                    "%s: max_context_len %d must lie in [0, block_table_stride %d * block_size]",
                    who, max_context_len, block_table_stride);
    if (blocks_bound(num_seqs, max_context_len, c) +
            (int64_t)pkv::decode_piece_cost(c->block_size, c->head_dim, elem_size(c->dtype)) *
                pkv::kDecodeMaxSeqs > INT32_MAX)
        return fail(PKV_EINVAL, "%s: %d sequences of up to %d tokens exceed 2^31 blocks per launch",
                    who, num_seqs, max_context_len);
    if (num_splits < 0 || num_splits > 65535)
        return fail(PKV_EINVAL, "%s: num_splits %d (0 .. 65535)", who, num_splits);
    if ((rc = check_ptr(q, "q", who)) || (rc = check_ptr(k_cache, "k_cache", who)) ||
        (rc = check_ptr(v_cache, "v_cache", who)) || (rc = check_ptr(out, "out", who)))
        return rc;
    if (!block_tables || !context_lens)
        return fail(PKV_EINVAL, "%s: block_tables or context_lens is NULL", who);
    if (k_new || v_new || slots) {
        if ((rc = check_ptr(k_new, "k_new", who)) || (rc = check_ptr(v_new, "v_new", who)))
            return rc;
        if (!slots)
            return fail(PKV_EINVAL, "%s: slot_mapping is NULL", who);
    }
    const int32_t W = num_splits > 0 ? num_splits : auto_splits(num_seqs, max_context_len, c);
    const WsLayout lay = ws_layout(num_seqs, num_q_heads, W, c->head_dim);
    if ((rc = check_ptr(workspace, "workspace", who)))
        return rc;
    if (workspace_bytes < lay.total)
        return fail(PKV_EINVAL, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes,
                    lay.total);
    if (!launch)
        return PKV_OK;
    pkv::DecodeLaunch d{};
    d.q = q;
    d.k_cache = k_cache;
    d.v_cache = v_cache;
    d.block_tables = block_tables;
    d.table_stride = block_table_stride;
    d.context_lens = context_lens;
    d.num_seqs = num_seqs;
    d.num_q_heads = num_q_heads;
    d.num_kv_heads = c->num_kv_heads;
    d.num_blocks = c->num_blocks;
    d.block_size = c->block_size;
    d.head_dim = c->head_dim;
    d.dtype = c->dtype;
    d.max_context_len = max_context_len;
    d.num_splits = W;
    d.scale = scale;
    d.out = out;
    d.out_dtype = out_dtype;
    char *ws = static_cast<char *>(workspace);
    d.ws_pref = reinterpret_cast<int32_t *>(ws + lay.pref);
    d.ws_o = reinterpret_cast<float *>(ws + lay.o);
    d.ws_ml = reinterpret_cast<float *>(ws + lay.ml);
    d.k_new = k_new;
    d.v_new = v_new;
    d.slots = slots;
    d.k_cache_w = const_cast<void *>(k_cache);
    d.v_cache_w = const_cast<void *>(v_cache);
    d.stream = stream;
    d.lse = lse;
    return pkv::launch_decode(d);
}

// Cascade decode: prefix splits, then the suffix decode's own workspace.
int32_t cascade_splits(int32_t B, int32_t hq, int32_t nb, const pkv_cache_desc *c)
{
    if (nb <= 0 || B <= 0)
        return 0;
    const int64_t tq = pkv::prefill_rows_per_workgroup() / (hq / c->num_kv_heads);  // tokens per prefill tile
    const int64_t per = (int64_t)c->num_kv_heads * ((B + tq - 1) / tq);
    int64_t ks = (pkv::device_cu_count() + per - 1) / per;
    ks = ks < 1 ? 1 : (ks > nb ? nb : ks);
    ks = ks > 4096 ? 4096 : ks;
    const int64_t nbk = (nb + ks - 1) / ks;
    return (int32_t)((nb + nbk - 1) / nbk);
}

struct CascadeWs {
    size_t o, lse, dws, total;
};

CascadeWs cascade_layout(int32_t B, int32_t hq, int32_t D, int32_t ks, int32_t W)
{
    const size_t rows = (size_t)B * hq, states = (size_t)ks + 1;
    CascadeWs l;
    l.o = 0;
    l.lse = l.o + align256(states * rows * D * sizeof(float));
    l.dws = l.lse + align256(states * rows * sizeof(float));
    l.total = l.dws + ws_layout(B, hq, W, D).total;
    return l;
}

}  // namespace

extern "C" int pkv_decode(const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *block_tables, int32_t block_table_stride,
                          const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                          int32_t max_context_len, float scale, void *out, int32_t out_dtype,
                          int32_t num_splits, void *workspace, size_t workspace_bytes,
                          const pkv_cache_desc *c, void *stream)
{
    pkv::clear_error();
    const int rc = decode_call("pkv_decode", q, k_cache, v_cache, block_tables,
                               block_table_stride, context_lens, num_seqs, num_q_heads,
                               max_context_len, scale, out, out_dtype, num_splits, workspace,
                               workspace_bytes, c, stream, nullptr, nullptr, nullptr);
    return PKV_FINISH(rc, stream, "pkv_decode");
}

extern "C" int pkv_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_tables, int32_t block_table_stride,
                                  const int32_t *context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_context_len, float scale,
                                  void *out, int32_t out_dtype, int32_t num_splits,
                                  const pkv_cache_desc *c, void *stream)
{
    static const char *who = "pkv_decode_noalloc";
    pkv::clear_error();
    int rc = check_desc(c, who);
    if (rc || (rc = check_heads(num_q_heads, c, who)))
        return rc;
    if (num_seqs > 0 && num_splits >= 0 && num_splits <= 65535) {
        const int32_t W = num_splits > 0 ? num_splits : auto_splits(num_seqs, max_context_len, c);
        const size_t need = ws_layout(num_seqs, num_q_heads, W, c->head_dim).total;
        if (need > PKV_DECODE_NOALLOC_SCRATCH_BYTES)
            return fail(PKV_EINVAL,
                        "%s: %d sequences x %d query heads with %d splits need %zu bytes of "
                        "partials, above the %zu-byte no-allocation scratch; use pkv_decode with "
                        "a workspace", who, num_seqs, num_q_heads, W, need,
                        (size_t)PKV_DECODE_NOALLOC_SCRATCH_BYTES);
    }
    // Every host-side check first (a stand-in workspace pointer that is never
    // used), so that a rejected call touches no device state.
    alignas(16) static char stand_in;
    rc = decode_call(who, q, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                     num_seqs, num_q_heads, max_context_len, scale, out, out_dtype, num_splits,
                     &stand_in, PKV_DECODE_NOALLOC_SCRATCH_BYTES, c, stream, nullptr, nullptr,
                     nullptr, nullptr, false);
    if (rc || num_seqs == 0)
        return rc;
    void *ws = nullptr;
    if ((rc = pkv::decode_noalloc_scratch(&ws)))
        return rc;
    rc = decode_call(who, q, k_cache, v_cache, block_tables, block_table_stride, context_lens,
                     num_seqs, num_q_heads, max_context_len, scale, out, out_dtype, num_splits,
                     ws, PKV_DECODE_NOALLOC_SCRATCH_BYTES, c, stream, nullptr, nullptr, nullptr);
    return PKV_FINISH(rc, stream, who);
}

extern "C" int pkv_append_decode(const void *k_new, const void *v_new,
                                 const int32_t *slot_mapping, const void *q, void *k_cache,
                                 void *v_cache, const int32_t *block_tables,
                                 int32_t block_table_stride, const int32_t *context_lens,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                 float scale, void *out, int32_t out_dtype, int32_t num_splits,
                                 void *workspace, size_t workspace_bytes, const pkv_cache_desc *c,
                                 void *stream)
{
    pkv::clear_error();
    if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
        return fail(PKV_EINVAL, "pkv_append_decode: k_new, v_new or slot_mapping is NULL");
    const int rc = decode_call("pkv_append_decode", q, k_cache, v_cache, block_tables,
                               block_table_stride, context_lens, num_seqs, num_q_heads,
                               max_context_len, scale, out, out_dtype, num_splits, workspace,
                               workspace_bytes, c, stream, k_new, v_new, slot_mapping);
    return PKV_CHECK_SLOTS(PKV_FINISH(rc, stream, "pkv_append_decode"), slot_mapping, num_seqs,
                           c ? (int64_t)c->num_blocks * c->block_size : 0, stream,
                           "pkv_append_decode");
}

extern "C" size_t pkv_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                     int32_t prefix_len, int32_t max_context_len,
                                                     const pkv_cache_desc *c)
{
    if (check_desc(c, "pkv_decode_cascade_workspace_bytes") || num_seqs <= 0 ||
        check_heads(num_q_heads, c, "pkv_decode_cascade_workspace_bytes") || prefix_len < 0)
        return 0;
    const int32_t ks = cascade_splits(num_seqs, num_q_heads, prefix_len / c->block_size, c);
    const int32_t W = auto_splits(num_seqs, max_context_len, c);
    return cascade_layout(num_seqs, num_q_heads, c->head_dim, ks, W).total;
}

extern "C" int pkv_decode_cascade(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *prefix_blocks, int32_t prefix_len,
                                  const int32_t *block_tables, int32_t block_table_stride,
                                  const int32_t *context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_context_len, float scale,
                                  void *out, int32_t out_dtype, void *workspace,
                                  size_t workspace_bytes, const pkv_cache_desc *c, void *stream)
{
    static const char *who = "pkv_decode_cascade";
    pkv::clear_error();
    int rc = check_desc(c, who);
    if (rc || (rc = check_heads(num_q_heads, c, who)))
        return rc;
    if (c->dtype != PKV_BF16)
        return fail(PKV_EUNSUPPORTED, "%s: bf16 caches only", who);
    if (prefix_len < 0 || prefix_len % c->block_size != 0)
        return fail(PKV_EINVAL, "%s: prefix_len %d is not a whole number of blocks", who,
                    prefix_len);
    if (prefix_len > 0 && !prefix_blocks)
        return fail(PKV_EINVAL, "%s: prefix_blocks is NULL", who);
    if (num_seqs < 0)
        return fail(PKV_EINVAL, "%s: num_seqs %d", who, num_seqs);
    if (num_seqs == 0)
        return PKV_OK;
    if ((int64_t)num_seqs * num_q_heads > INT32_MAX / 2)
        return fail(PKV_EINVAL, "%s: too many rows", who);
    const int32_t nb = prefix_len / c->block_size;
    const int32_t ks = cascade_splits(num_seqs, num_q_heads, nb, c);
    const int32_t W = auto_splits(num_seqs, max_context_len, c);
    const CascadeWs lay = cascade_layout(num_seqs, num_q_heads, c->head_dim, ks, W);
    if ((rc = check_ptr(workspace, "workspace", who)))
        return rc;
    if (workspace_bytes < lay.total)
        return fail(PKV_EINVAL, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes,
                    lay.total);
    if ((rc = check_ptr(out, "out", who)))
        return rc;
    if (out_dtype != PKV_F32 && out_dtype != PKV_BF16)
        return fail(PKV_EINVAL, "%s: out_dtype %d", who, out_dtype);
    char *ws = static_cast<char *>(workspace);
    const int64_t rows = (int64_t)num_seqs * num_q_heads;
    float *o_all = reinterpret_cast<float *>(ws + lay.o);
    float *lse_all = reinterpret_cast<float *>(ws + lay.lse);
    // The suffixes: a plain split decode writing a normalised fp32 state.
    auto suffixes = [&](void *st) {
        return decode_call(who, q, k_cache, v_cache, block_tables, block_table_stride,
                           context_lens, num_seqs, num_q_heads, max_context_len, scale,
                           o_all + (size_t)ks * rows * c->head_dim, PKV_F32, W, ws + lay.dws,
                           workspace_bytes - lay.dws, c, st, nullptr, nullptr, nullptr,
                           lse_all + (size_t)ks * rows);
    };
    // The shared prefix once for all sequences: ks pseudo-sequences, one per
    // range of prefix blocks, each holding every sequence's queries (read
    // from the same rows) and attending its whole range; the kernel derives
    // each one's query rows and key count itself.
    auto prefix = [&](void *st) {
        const int32_t nbk = (nb + ks - 1) / ks;
        pkv::PrefillLaunch p{q, nullptr, ks, num_seqs, k_cache, v_cache, prefix_blocks, nbk,
                             nullptr, nbk * c->block_size, num_q_heads, c->num_kv_heads,
                             c->num_blocks, c->block_size, c->head_dim, scale, o_all, PKV_F32,
                             st};
        p.causal = 0;
        p.q_shared = 1;
        p.lse = lse_all;
        p.syn_rows = num_seqs;
        p.syn_nbk = nbk;
        p.syn_nb = nb;
        return pkv::launch_prefill(p);
    };
    // The two passes write disjoint states and read only q and the caches:
    // the suffix decode (HBM-bound, the longer one) is launched first on the
    // caller's stream and the prefix pass (MFMA-bound) beside it on the
    // library's side stream, so that they share the CUs.  On 128 sequences
    // over a 2048-token prefix, calls back to back: 69-71 us against
    // 76-77 us one after the other.
    rc = ks > 0 ? pkv::launch_forked(stream, suffixes, prefix) : suffixes(stream);
    if (rc != PKV_OK)
        return rc;
    return PKV_FINISH(pkv::launch_merge_states(o_all, lse_all, ks + 1, rows, c->head_dim, out,
                                               out_dtype, stream),
                      stream, who);
}

extern "C" size_t pkv_prefill_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                              int32_t max_query_len, const pkv_cache_desc *c)
{
    if (!c || c->dtype != PKV_BF16 || c->num_kv_heads <= 0 || num_q_heads <= 0 ||
        num_q_heads % c->num_kv_heads || (c->head_dim != 64 && c->head_dim != 128))
        return 0;
    const int32_t ks = prefill_key_splits(num_seqs, num_q_heads, max_query_len, -1, c);
    if (ks <= 1)
        return 0;
    return prefill_layout(num_seqs, num_q_heads, max_query_len, c->head_dim, ks).total;
}

extern "C" int pkv_prefill_chunk(const void *q, const int32_t *query_start_loc, int32_t num_seqs,
                                 int32_t max_query_len, const void *k_cache, const void *v_cache,
                                 const int32_t *block_tables, int32_t block_table_stride,
                                 const int32_t *context_lens, int32_t max_context_len,
                                 int32_t num_q_heads, float scale, void *out, int32_t out_dtype,
                                 void *workspace, size_t workspace_bytes, const pkv_cache_desc *c,
                                 void *stream)
{
    static const char *who = "pkv_prefill_chunk";
    pkv::clear_error();
    int rc = check_desc(c, who);
    if (rc || (rc = check_heads(num_q_heads, c, who)))
        return rc;
    if (c->dtype != PKV_BF16)
        return fail(PKV_EUNSUPPORTED, "%s: the MFMA path takes bf16 only", who);
    if (num_seqs < 0 || num_seqs > 65535)
        return fail(PKV_EINVAL, "%s: num_seqs %d (0 .. 65535)", who, num_seqs);
    if (out_dtype != PKV_F32 && out_dtype != PKV_BF16)
        return fail(PKV_EINVAL, "%s: out_dtype %d", who, out_dtype);
    if (!std::isfinite(scale))
        return fail(PKV_EINVAL, "%s: scale is not finite", who);
    if (num_seqs == 0 || max_query_len == 0)
        return PKV_OK;
    if (max_query_len < 0 || block_table_stride <= 0 || max_context_len < 0 ||
        (int64_t)max_context_len > (int64_t)block_table_stride * c->block_size)
        return fail(PKV_EINVAL, "%s: bad max_query_len %d / max_context_len %d / stride %d", who,
                    max_query_len, max_context_len, block_table_stride);
    if ((rc = check_ptr(q, "q", who)) || (rc = check_ptr(k_cache, "k_cache", who)) ||
        (rc = check_ptr(v_cache, "v_cache", who)) || (rc = check_ptr(out, "out", who)))
        return rc;
    if (!query_start_loc || !block_tables || !context_lens)
        return fail(PKV_EINVAL, "%s: query_start_loc, block_tables or context_lens is NULL", who);
    pkv::PrefillLaunch p{q, query_start_loc, num_seqs, max_query_len, k_cache, v_cache,
                         block_tables, block_table_stride, context_lens, max_context_len,
                         num_q_heads, c->num_kv_heads, c->num_blocks, c->block_size, c->head_dim,
                         scale, out, out_dtype, stream};
    // Key splits when the workspace holds their states (fewer if it is
    // short; none without one).
    int32_t ks = workspace ? prefill_key_splits(num_seqs, num_q_heads, max_query_len,
                                                max_context_len, c)
                           : 1;
    while (ks > 1 &&
           prefill_layout(num_seqs, num_q_heads, max_query_len, c->head_dim, ks).total >
               workspace_bytes)
        --ks;
    if (ks <= 1)
        return PKV_FINISH(pkv::launch_prefill(p), stream, who);
    if ((rc = check_ptr(workspace, "workspace", who)))
        return rc;
    const PrefillWs lay = prefill_layout(num_seqs, num_q_heads, max_query_len, c->head_dim, ks);
    float *so = reinterpret_cast<float *>(static_cast<char *>(workspace) + lay.o);
    float *sl = reinterpret_cast<float *>(static_cast<char *>(workspace) + lay.lse);
    p.out = so;
    p.out_dtype = PKV_F32;
    p.lse = sl;
    p.key_splits = ks;
    p.split_rows = lay.rows;
    if ((rc = pkv::launch_prefill(p)))
        return rc;
    return PKV_FINISH(pkv::launch_merge_states(so, sl, ks, lay.rows, c->head_dim, out, out_dtype,
                                               stream, query_start_loc + num_seqs, num_q_heads),
                      stream, who);
}
