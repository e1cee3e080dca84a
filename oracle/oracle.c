/*
 * oracle.c -- plain, slow, fp64 CPU reference for paged-KV attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no code, header, table or helper
 * with the HIP path.
 *
 * Pages followed (cited by title and section):
 *   [KV-prep]  "LLM Inference: KV Cache, Batching & Scheduling"
 *              (cariara.com interview-prep page)
 *   [KV-news]  "LLM Inference Engineering: Overcoming the KV-Cache Bottleneck
 *              and Maximizing Production Throughput" (wpnews.pro summary)
 *   [KV-blog]  the adilsher.pro blog post of the same title
 *
 * What it computes.  Paging only changes WHERE key/value rows live; the
 * attention result is the plain definition over the logically contiguous
 * sequence ([KV-prep] "The KV cache": attention needs the keys and values of
 * all prior positions; [KV-news] section 2 and [KV-prep] "PagedAttention and
 * vLLM": blocks are mapped, not moved).  So the oracle never sees a block
 * table, slot or physical block id for attention: it takes, per sequence, the
 * K and V rows in append order.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - attention is softmax(scale * q . k) . v with `scale` passed in;
 *   - query head h reads KV head g = floor(h / G), G = Hq / Hkv (the pages give
 *     only "KV heads (GQA) 8", [KV-prep] "The KV cache" table);
 *   - an empty context gives a zero output row;
 *   - prefill row i of a chunk of C rows whose sequence holds L keys (the chunk
 *     already appended) attends keys [0, L - C + i], diagonal included;
 *   - the cache holds, per tensor, num_blocks x num_kv_heads tiles, each the
 *     block_size x head_dim elements of one KV head's share of a block, and
 *     slot s names block s / block_size, offset s % block_size; a negative
 *     slot is padding and writes nothing.  Inside a tile (bs tokens, D dims,
 *     E = 16 / element size dims per 16-byte chunk) K element (t, d) sits at
 *     ((d / E) * bs + t) * E + d % E and V element (t, d) at
 *     ((t / 4) * D + d) * 4 + t % 4.
 *
 * Precision: inputs are upcast exactly (fp32 -> double; bf16 -> fp32 by a
 * 16-bit shift -> double).  All arithmetic is IEEE double with sums taken
 * sequentially in index order; exp is libm's.  Build without -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Exact upcast of one stored element to double. */
static double elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    uint32_t u = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Attention of one query row over `nkeys` logically contiguous key/value rows.
 *   qbase/qoff : the query row is q[qoff .. qoff + D)
 *   kv rows    : key row j of KV head g is k[(row0 + j) * Hkv * D + g * D + d]
 *   w          : optional, receives the nkeys softmax weights
 * Follows the plain definition: logits s_j = scale * sum_d q_d k_jd; subtract
 * the maximum; exponentiate; normalise by the sum; weighted sum of value rows.
 */
static void attend_row(const void *q, int64_t qoff, const void *k, const void *v,
                       int64_t row0, int nkeys, int Hkv, int g, int D, int dtype,
                       double scale, double *out, double *s, double *w)
{
    if (nkeys <= 0) {
        for (int d = 0; d < D; ++d)
            out[d] = 0.0;
        return;
    }
    double m = -INFINITY;
    for (int j = 0; j < nkeys; ++j) {
        int64_t kb = (row0 + j) * (int64_t)Hkv * D + (int64_t)g * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += elem(q, dtype, qoff + d) * elem(k, dtype, kb + d);
        s[j] = scale * dot;
        if (s[j] > m)
            m = s[j];
    }
    double z = 0.0;
    for (int j = 0; j < nkeys; ++j) {
        s[j] = exp(s[j] - m);
        z += s[j];
    }
    for (int j = 0; j < nkeys; ++j)
        s[j] = s[j] / z;
    if (w)
        memcpy(w, s, sizeof(double) * (size_t)nkeys);
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int j = 0; j < nkeys; ++j) {
            int64_t vb = (row0 + j) * (int64_t)Hkv * D + (int64_t)g * D;
            acc += s[j] * elem(v, dtype, vb + d);
        }
        out[d] = acc;
    }
}

static int check_heads(int Hq, int Hkv, int D)
{
    return !(Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0);
}

/*
 * Decode ([KV-prep] "The KV cache": the new token attends every prior
 * position, its own K/V appended first).
 *   q        [B][Hq][D]
 *   k, v     [rows][Hkv][D]; sequence b owns rows seq_start[b] .. seq_start[b+1]
 *   out      [B][Hq][D] doubles
 *   pairs    optional list of npairs (b, h) pairs (2*npairs ints) to compute;
 *            NULL computes every (b, h).  Rows not computed are left untouched.
 *   nthreads OpenMP threads (<= 0: runtime default)
 * Returns 0, or -1 on bad arguments.
 */
int oracle_decode(int B, int Hq, int Hkv, int D, int dtype, const void *q,
                  const void *k, const void *v, const int64_t *seq_start,
                  double scale, double *out, const int32_t *pairs, int npairs,
                  int nthreads)
{
    if (B < 0 || !check_heads(Hq, Hkv, D) || (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return -1;
    const int G = Hq / Hkv;
    int64_t maxlen = 0;
    for (int b = 0; b < B; ++b) {
        int64_t L = seq_start[b + 1] - seq_start[b];
        if (L < 0)
            return -1;
        if (L > maxlen)
            maxlen = L;
    }
    const int64_t total = pairs ? npairs : (int64_t)B * Hq;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
    int bad = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < total; ++t) {
            if (!s)
                continue;
            int b = pairs ? pairs[2 * t] : (int)(t / Hq);
            int h = pairs ? pairs[2 * t + 1] : (int)(t % Hq);
            if (b < 0 || b >= B || h < 0 || h >= Hq) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int64_t L = seq_start[b + 1] - seq_start[b];
            attend_row(q, ((int64_t)b * Hq + h) * D, k, v, seq_start[b], (int)L, Hkv,
                       h / G, D, dtype, scale, out + ((int64_t)b * Hq + h) * D, s, NULL);
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/* Softmax weights of one decode row (b, h): w[0 .. L_b).  Test hook for the
 * normalisation invariant. */
int oracle_decode_weights(int B, int Hq, int Hkv, int D, int dtype, const void *q,
                          const void *k, const void *v, const int64_t *seq_start,
                          double scale, int b, int h, double *w, double *out_row)
{
    if (b < 0 || b >= B || h < 0 || !check_heads(Hq, Hkv, D) || h >= Hq)
        return -1;
    int64_t L = seq_start[b + 1] - seq_start[b];
    double *s = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    if (!s)
        return -1;
    attend_row(q, ((int64_t)b * Hq + h) * D, k, v, seq_start[b], (int)L, Hkv, h / (Hq / Hkv),
               D, dtype, scale, out_row, s, w);
    free(s);
    return 0;
}

/*
 * Chunked prefill ([KV-prep] "Chunked prefill": the prompt is split into
 * fixed-size chunks; splitting changes scheduling, not the result).
 *   q          [sum C][Hq][D]; chunk rows of sequence b are
 *              query_start[b] .. query_start[b+1]
 *   k, v       logical rows per sequence as in oracle_decode; the sequence's
 *              rows already include the chunk (L_b = seq_start[b+1]-seq_start[b])
 *   out        [sum C][Hq][D] doubles
 *   Row i of chunk b (C_b rows) attends keys 0 .. L_b - C_b + i inclusive.
 *   rows       optional list of nrows (token row, h) pairs to compute; NULL = all
 */
int oracle_prefill(int S, int Hq, int Hkv, int D, int dtype, const void *q,
                   const int32_t *query_start, const void *k, const void *v,
                   const int64_t *seq_start, double scale, double *out,
                   const int32_t *rows, int nrows, int nthreads)
{
    if (S < 0 || !check_heads(Hq, Hkv, D) || (dtype != ORACLE_F32 && dtype != ORACLE_BF16))
        return -1;
    const int G = Hq / Hkv;
    int64_t maxlen = 0;
    for (int b = 0; b < S; ++b) {
        int64_t L = seq_start[b + 1] - seq_start[b];
        int64_t C = (int64_t)query_start[b + 1] - query_start[b];
        if (L < 0 || C < 0 || C > L)
            return -1;
        if (L > maxlen)
            maxlen = L;
    }
    const int64_t T = query_start[S];
    const int64_t total = rows ? nrows : T * Hq;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
    int bad = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < total; ++t) {
            if (!s)
                continue;
            int64_t r = rows ? rows[2 * t] : t / Hq;
            int h = rows ? rows[2 * t + 1] : (int)(t % Hq);
            if (r < 0 || r >= T || h < 0 || h >= Hq) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int b = 0; /* the sequence that owns token row r */
            while (b + 1 < S && query_start[b + 1] <= r)
                ++b;
            int64_t L = seq_start[b + 1] - seq_start[b];
            int64_t C = (int64_t)query_start[b + 1] - query_start[b];
            int64_t i = r - query_start[b];
            int64_t nkeys = L - C + i + 1;
            attend_row(q, (r * Hq + h) * D, k, v, seq_start[b], (int)nkeys, Hkv, h / G, D,
                       dtype, scale, out + (r * Hq + h) * D, s, NULL);
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * KV append ([KV-prep] "The KV cache": the cache appends the new token's K
 * and V each step).  For every t with s = slots[t] >= 0 and every KV head g,
 * the D elements of k[t][g][:] are copied, bit for bit, to
 *   k_cache[s / bs][g][s % bs][:]   (and likewise v into v_cache).
 * Every other byte of the caches is left as it was.
 * Returns 0, or -1 if a slot is out of range (nothing written then).
 */
int oracle_append(const void *k, const void *v, const int32_t *slots, int T, int Hkv, int D,
                  int elem_size, int bs, int64_t num_blocks, void *k_cache, void *v_cache)
{
    if (T < 0 || Hkv <= 0 || D <= 0 || bs <= 0 || (elem_size != 2 && elem_size != 4))
        return -1;
    const int E = 16 / elem_size;
    if (D % E != 0 || bs % 4 != 0)
        return -1;
    for (int t = 0; t < T; ++t)
        if (slots[t] >= 0 && (int64_t)slots[t] >= num_blocks * bs)
            return -1;
    const size_t tile = (size_t)bs * (size_t)D;          /* elements per (block, head) tile */
    for (int t = 0; t < T; ++t) {
        int64_t s = slots[t];
        if (s < 0)
            continue;
        int64_t blk = s / bs, off = s % bs;
        for (int g = 0; g < Hkv; ++g) {
            size_t base = ((size_t)blk * Hkv + g) * tile;
            for (int d = 0; d < D; ++d) {
                size_t src = ((size_t)t * Hkv + g) * D + d;
                size_t kdst = base + ((size_t)(d / E) * bs + off) * E + d % E;
                size_t vdst = base + ((size_t)(off / 4) * D + d) * 4 + off % 4;
                memcpy((char *)k_cache + kdst * elem_size, (const char *)k + src * elem_size,
                       elem_size);
                memcpy((char *)v_cache + vdst * elem_size, (const char *)v + src * elem_size,
                       elem_size);
            }
        }
    }
    return 0;
}

/*
 * Block copy (sharing of identical prefixes, [KV-news] section 2 and
 * [KV-blog] "The Elegant Fix"; the copy made before a sharer writes into a
 * shared block is this library's reading, the pages are silent on writes to
 * shared pages).  For pair i, every (KV head, offset) row of block
 * dst_ids[i] in each destination tensor becomes the same row of block
 * src_ids[i] in the source tensor.  A pair naming a block outside its cache
 * is skipped.  Pairs are applied in order.
 */
int oracle_copy_blocks(const void *src_k, const void *src_v, int64_t src_nb, void *dst_k,
                       void *dst_v, int64_t dst_nb, const int32_t *src_ids,
                       const int32_t *dst_ids, int n, int Hkv, int bs, int D, int elem_size)
{
    if (n < 0 || Hkv <= 0 || bs <= 0 || D <= 0 || (elem_size != 2 && elem_size != 4))
        return -1;
    const size_t row = (size_t)D * (size_t)elem_size;
    for (int i = 0; i < n; ++i) {
        const int64_t s = src_ids[i], d = dst_ids[i];
        if (s < 0 || s >= src_nb || d < 0 || d >= dst_nb)
            continue;
        for (int g = 0; g < Hkv; ++g)
            for (int o = 0; o < bs; ++o) {
                size_t from = (((size_t)s * Hkv + g) * bs + o) * row;
                size_t to = (((size_t)d * Hkv + g) * bs + o) * row;
                memcpy((char *)dst_k + to, (const char *)src_k + from, row);
                memcpy((char *)dst_v + to, (const char *)src_v + from, row);
            }
    }
    return 0;
}

/*
 * Per-layer KV-cache bytes ([KV-prep] "The KV cache", memory-cost formula):
 * two tensors (K and V) x tokens x KV heads x head_dim x element size.
 */
int64_t oracle_kv_bytes_per_layer(int64_t seq_len, int64_t num_kv_heads, int64_t head_dim,
                                  int64_t elem_size)
{
    return 2 * seq_len * num_kv_heads * head_dim * elem_size;
}
