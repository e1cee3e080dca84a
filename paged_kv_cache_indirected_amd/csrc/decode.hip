// Paged decode attention for gfx950 (CDNA4): split-context partition pass
// plus a log-sum-exp merge pass.
//
// What is computed ("LLM Inference: KV Cache, Batching & Scheduling",
// sections "The KV cache" and "PagedAttention and vLLM"; the "LLM Inference
// Engineering" summary, section 2): for sequence b and query head h, softmax
// attention of q[b][h] over the K/V rows of all L_b prior positions, where
// position j lives in physical block block_tables[b][j / bs] at offset
// j % bs.  Query head h reads KV head h / G.
//
// Design (one workgroup = one (KV head g, context partition, sequence b)):
//   * 4 waves; wave w takes blocks w, w+4, ... of the partition.  A wave is
//     R rows of LPT lanes; lane (row r, i) loads the 16-byte chunk i of token
//     rows r, r+R, ... of each K and V block tile.  Per load instruction the
//     wave reads one contiguous KiB of the tile: whole-block, coalesced
//     16-byte loads straight from HBM into registers.
//   * GQA packing: each lane keeps its 16-byte slice of q for all G query
//     heads of the group, so every K/V byte read from HBM serves the G heads.
//   * QK^T: per lane, partial dot products over its slice (bf16 pairs via
//     v_dot2_f32_bf16, fp32 accumulation), then a cross-lane reduction by
//     recursive halving with DPP row_mirror / row_half_mirror / quad_perm
//     exchanges: lane i holds q heads in an order permuted by its own lane
//     bits, so at every halving step the half a lane keeps and the half it
//     sends sit in the same registers on every lane, and each step costs one
//     DPP add per kept value.  Afterwards each lane owns the full scores of
//     G / 2^S heads for its row's tokens.
//   * Online softmax per (row, head) stream in log2 units (exp2 on the
//     hardware exp unit); masking by select, never by multiplying, so NaN
//     poison in unused slots never reaches the result.
//   * PV: lane (r, i) accumulates o[h][its 8 (bf16) or 4 (fp32) dims] for all
//     G heads with p broadcast from the owning lane by DPP row_newbcast.
//   * End of partition: the NW * R streams merge through LDS; a partition
//     that covers the whole context writes the normalised output, others
//     write (o, m, l) partials that the merge pass combines in partition
//     order (deterministic: the result depends on logical positions and the
//     partition size only, never on physical block ids).
//   * Grid (Hkv, partitions, B) with the KV head fastest, so workgroups of
//     one KV head land on one XCD and blocks shared between sequences stay in
//     that XCD's L2.
#include <hip/hip_runtime.h>

#include <utility>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int NW = 4;                 // waves per workgroup
constexpr int kThreads = NW * 64;
constexpr float kLazyMax = 8.0f;      // running-max slack, log2 units
constexpr int kRsrcWord3 = 0x00020000; // raw buffer resource: 32-bit data format, no swizzle

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct Args {
    const void *q;
    const void *kc;
    const void *vc;
    const int32_t *tables;
    const int32_t *lens;
    void *out;
    float *ws_o;
    float *ws_ml;
    int32_t stride;
    int32_t B, Hq, Hkv, num_blocks;
    int32_t part_blocks, max_parts;
    int32_t out_dtype;
    float scale_log2;                 // scale * log2(e)
};

__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// Value held by lane (i ^ C) inside groups of C + 1 lanes.
template <int C>
__device__ __forceinline__ float xmirror(float v)
{
    if constexpr (C == 1)
        return __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    else if constexpr (C == 3)
        return __builtin_amdgcn_update_dpp(0.0f, v, 0x1B, 0xF, 0xF, false);   // quad_perm 3,2,1,0
    else if constexpr (C == 7)
        return __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    else if constexpr (C == 15)
        return __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xF, 0xF, false);  // row_mirror
    else {
        static_assert(C == 31, "mirror width");
        // ds_swizzle bit mode: and 0x1f, or 0, xor 0x1f (within 32 lanes)
        return __builtin_bit_cast(float,
                                  __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x7C1F));
    }
}

// Value held by lane SRC of this lane's group of LPT lanes.
template <int LPT, int SRC>
__device__ __forceinline__ float bcast(float v)
{
    if constexpr (LPT == 16)
        return __builtin_amdgcn_update_dpp(0.0f, v, 0x150 + SRC, 0xF, 0xF, false);  // row_newbcast
    else if constexpr (LPT == 8)
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                     (SRC << 5) | 0x18));
    else {
        static_assert(LPT == 32, "group width");
        return __builtin_bit_cast(float,
                                  __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), SRC << 5));
    }
}

template <int DT, int D, int BS, int G>
struct Shape {
    static constexpr int ES = DT == PKV_F32 ? 4 : 2;   // element bytes
    static constexpr int CH = 16 / ES;                 // elements per 16-byte chunk
    static constexpr int LPT = D / CH;                 // lanes per token row
    static constexpr int R = 64 / LPT;                 // token rows per wave
    static constexpr int SUBTOK = BS < 4 * R ? BS : 4 * R;   // tokens per pipelined sub-tile
    static constexpr int NSUBT = BS / SUBTOK;          // sub-tiles per block
    static constexpr int TPR = SUBTOK / R;             // tokens per row per sub-tile (<= 4)
    static constexpr int LL = ilog2(LPT);
    static constexpr int LG = ilog2(G);
    static constexpr int S = LG < LL ? LG : LL;        // halving steps
    static constexpr int GH = G >> S;                  // heads a lane owns after reduction
    static constexpr int NSUB = NW * R;                // softmax streams per workgroup
    static_assert(TPR >= 1 && (1 << LL) == LPT && (1 << LG) == G, "shape");
};

// Recursive halving of the G x TPR partial scores across the LPT lanes of a
// row; step s keeps heads [0, G >> (s+1)) and adds the partner's copy of the
// same heads, which the partner holds in registers h ^ X.
template <int s, int S, int LL, int LG, int G, int TPR>
__device__ __forceinline__ void halve(float (&acc)[G][TPR])
{
    if constexpr (s < S) {
        constexpr int X = ((1 << (LG - s)) - 1) ^ ((1 << (LG - S)) - 1);
        constexpr int C = (1 << (LL - s)) - 1;
#pragma unroll
        for (int h = 0; h < (G >> (s + 1)); ++h)
#pragma unroll
            for (int t = 0; t < TPR; ++t)
                acc[h][t] += xmirror<C>(acc[h ^ X][t]);
        halve<s + 1, S, LL, LG, G, TPR>(acc);
    }
}

// Plain butterfly over the lane bits the halving did not use.
template <int bit, int GH, int G, int TPR>
__device__ __forceinline__ void butterfly(float (&acc)[G][TPR])
{
    if constexpr (bit >= 0) {
        constexpr int C = (1 << (bit + 1)) - 1;
#pragma unroll
        for (int h = 0; h < GH; ++h)
#pragma unroll
            for (int t = 0; t < TPR; ++t)
                acc[h][t] += xmirror<C>(acc[h][t]);
        butterfly<bit - 1, GH, G, TPR>(acc);
    }
}

// Partial dot product of one 16-byte chunk of q and of k.
template <int DT>
__device__ __forceinline__ float chunk_dot(const uint4 &q, const uint4 &k)
{
    if constexpr (DT == PKV_BF16) {
        float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x),
                                                  __builtin_bit_cast(bf16x2_t, k.x), 0.0f, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y),
                                            __builtin_bit_cast(bf16x2_t, k.y), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z),
                                            __builtin_bit_cast(bf16x2_t, k.z), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w),
                                            __builtin_bit_cast(bf16x2_t, k.w), a, false);
        return a;
    } else {
        float a = as_f32(q.x) * as_f32(k.x);
        a = __builtin_fmaf(as_f32(q.y), as_f32(k.y), a);
        a = __builtin_fmaf(as_f32(q.z), as_f32(k.z), a);
        a = __builtin_fmaf(as_f32(q.w), as_f32(k.w), a);
        return a;
    }
}

// The 16-byte chunk of v as CH floats.
template <int DT>
__device__ __forceinline__ void chunk_to_f32(const uint4 &v, float (&f)[16 / (DT == PKV_F32 ? 4 : 2)])
{
    if constexpr (DT == PKV_BF16) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            f[2 * c] = as_f32(w[c] << 16);
            f[2 * c + 1] = as_f32(w[c] & 0xFFFF0000u);
        }
    } else {
        f[0] = as_f32(v.x);
        f[1] = as_f32(v.y);
        f[2] = as_f32(v.z);
        f[3] = as_f32(v.w);
    }
}

__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_out(void *out, int32_t dtype, int64_t idx, float x)
{
    if (dtype == PKV_F32)
        static_cast<float *>(out)[idx] = x;
    else
        static_cast<uint16_t *>(out)[idx] = bf16_rne(x);
}

// Context length of sequence b clamped to what its table row can address,
// and the number of partitions it spans (at least 1, at most max_parts).
template <int BS>
__device__ __forceinline__ void seq_extent(const Args &a, int b, int &L, int &nblk, int &np)
{
    L = a.lens[b];
    const int cap = a.stride * BS;
    L = L < 0 ? 0 : (L > cap ? cap : L);
    nblk = (L + BS - 1) / BS;
    np = (nblk + a.part_blocks - 1) / a.part_blocks;
    np = np < 1 ? 1 : (np > a.max_parts ? a.max_parts : np);
}

template <int DT, int D, int BS, int G>
__global__ __launch_bounds__(kThreads, 2) void k_decode(Args a)
{
    using Sh = Shape<DT, D, BS, G>;
    constexpr int CH = Sh::CH, LPT = Sh::LPT, R = Sh::R, TPR = Sh::TPR;
    constexpr int SUBTOK = Sh::SUBTOK, NSUBT = Sh::NSUBT;
    constexpr int LL = Sh::LL, LG = Sh::LG, S = Sh::S, GH = Sh::GH, NSUB = Sh::NSUB;
    constexpr int TILE = BS * D * Sh::ES;              // bytes of one (block, head) tile

    __shared__ float lds_o[NSUB * G * D];
    __shared__ float lds_m[NSUB * G];
    __shared__ float lds_l[NSUB * G];

    const int g = blockIdx.x, part = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane / LPT, li = lane % LPT;

    int L, nblk, np;
    seq_extent<BS>(a, b, L, nblk, np);
    if (part >= np)
        return;
    const int j0 = part * a.part_blocks;
    const int j1 = min(j0 + a.part_blocks, nblk);

    // This lane's q slices, heads permuted by its own lane bits: slot h holds
    // query head g*G + (h ^ hm).
    const int hm = (li >> (LL - S)) << (LG - S);
    const int hq0 = g * G;
    uint4 qr[G];
    {
        const uint4 *qp = static_cast<const uint4 *>(a.q) + ((int64_t)b * a.Hq + hq0) * LPT + li;
#pragma unroll
        for (int h = 0; h < G; ++h)
            qr[h] = qp[(h ^ hm) * LPT];
    }

    float o[G][CH];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < CH; ++c)
            o[h][c] = 0.0f;
    float m[GH], l[GH];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
    }

    const int32_t *bt = a.tables + (int64_t)b * a.stride;
    const int64_t blk_bytes = (int64_t)a.Hkv * TILE;
    const char *kbase = static_cast<const char *>(a.kc) + (int64_t)g * TILE;
    const char *vbase = static_cast<const char *>(a.vc) + (int64_t)g * TILE;
    const uint32_t lane_off = (uint32_t)lane * 16u;

    auto blk_of = [&](int e) { return j0 + w + (e / NSUBT) * NW; };

    // Issue the 2 * TPR 16-byte loads of one sub-tile through a buffer
    // resource whose base is the wave-uniform tile address (scalar
    // registers) and this lane's fixed 32-bit offset.  A block id outside the
    // pool gets an empty resource, so its loads return zeros without touching
    // memory; every load is unconditional and the wait counts stay exact.
    auto issue = [&](int e, int id, uint4 (&kr)[TPR], uint4 (&vr)[TPR]) {
        const bool ok = (unsigned)id < (unsigned)a.num_blocks;
        const int64_t off = (int64_t)(ok ? id : 0) * blk_bytes + (e % NSUBT) * (TPR * 1024);
        const int nrec = ok ? TPR * 1024 : 0;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kbase + off), 0, nrec, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vbase + off), 0, nrec, kRsrcWord3);
#pragma unroll
        for (int t = 0; t < TPR; ++t) {
            kr[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rk, (int)(lane_off + t * 1024u), 0, 0));
            vr[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rv, (int)(lane_off + t * 1024u), 0, 0));
        }
    };

    // One sub-tile: QK^T, online softmax update, PV.
    auto process = [&](int e, int id, const uint4 (&kr)[TPR], uint4 (&vr)[TPR]) {
        const int j = blk_of(e);
        const bool ok = (unsigned)id < (unsigned)a.num_blocks;
        float acc[G][TPR];
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int t = 0; t < TPR; ++t)
                acc[h][t] = chunk_dot<DT>(qr[h], kr[t]);
        halve<0, S, LL, LG, G, TPR>(acc);
        butterfly<LL - S - 1, GH, G, TPR>(acc);

        // Scores in log2 units; positions past the context are masked.  The
        // running max only moves when a block's max exceeds it by more than
        // 2^8: exponentials stay <= 256, and the rescale of o is skipped
        // unless some stream of the wave moved.
        const int pos0 = j * BS + (e % NSUBT) * SUBTOK + r;
        float p[GH][TPR], alpha[GH];
        bool grew = false;
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            float mb = -INFINITY;
#pragma unroll
            for (int t = 0; t < TPR; ++t) {
                const bool live = ok && (pos0 + t * R < L);
                const float sc = live ? acc[h][t] * a.scale_log2 : -INFINITY;
                p[h][t] = sc;
                mb = fmaxf(mb, sc);
            }
            const bool up = mb > m[h] + kLazyMax;
            const float mn = up ? mb : m[h];
            alpha[h] = up ? __builtin_amdgcn_exp2f(m[h] - mn) : 1.0f;
            grew |= up;
            const bool dead = (mn == -INFINITY);
            float sum = 0.0f;
#pragma unroll
            for (int t = 0; t < TPR; ++t) {
                p[h][t] = dead ? 0.0f : __builtin_amdgcn_exp2f(p[h][t] - mn);
                sum += p[h][t];
            }
            l[h] = __builtin_fmaf(l[h], alpha[h], sum);
            m[h] = mn;
        }

        // Rescale the accumulators of every head by its owner's alpha.
        if (__builtin_amdgcn_ballot_w64(grew) != 0) {
            [&]<int... H>(std::integer_sequence<int, H...>) {
                (([&] {
                     constexpr int src = (H >> (LG - S)) << (LL - S);
                     const float ah = bcast<LPT, src>(alpha[H & (GH - 1)]);
#pragma unroll
                     for (int c = 0; c < CH; ++c)
                         o[H][c] *= ah;
                 }()),
                 ...);
            }(std::make_integer_sequence<int, G>{});
        }

        // The context's last block may hold unused slots, and a bad id reads
        // block 0: such V must not reach the sum (0 * NaN would).
        if (j == nblk - 1 || !ok) {
#pragma unroll
            for (int t = 0; t < TPR; ++t)
                if (!ok || pos0 + t * R >= L)
                    vr[t] = make_uint4(0, 0, 0, 0);
        }

        // PV with p broadcast from the lane that owns the head.
#pragma unroll
        for (int t = 0; t < TPR; ++t) {
            float vf[CH];
            chunk_to_f32<DT>(vr[t], vf);
            [&]<int... H>(std::integer_sequence<int, H...>) {
                (([&] {
                     constexpr int src = (H >> (LG - S)) << (LL - S);
                     const float ph = bcast<LPT, src>(p[H & (GH - 1)][t]);
#pragma unroll
                     for (int c = 0; c < CH; ++c)
                         o[H][c] = __builtin_fmaf(ph, vf[c], o[H][c]);
                 }()),
                 ...);
            }(std::make_integer_sequence<int, G>{});
        }
    };

    // Wave w takes blocks j0 + w, j0 + w + NW, ..., each as NSUBT sub-tiles
    // (units e = 0 .. E-1).  The next unit's loads are in flight while the
    // current one is processed (ping-pong buffers; table ids read two units
    // ahead, clamped to the last unit, whose re-read is harmless).
    if (j0 + w < j1) {
        const int E = ((j1 - j0 - w + NW - 1) / NW) * NSUBT;
        auto id_of = [&](int e) { return bt[blk_of(e < E ? e : E - 1)]; };
        uint4 kA[TPR], vA[TPR], kB[TPR], vB[TPR];
        int e = 0;
        int id_cur = id_of(0);
        int id_nxt = id_of(1);
        issue(0, id_cur, kA, vA);
        for (;;) {
            issue(e + 1 < E ? e + 1 : E - 1, id_nxt, kB, vB);
            int id_nn = id_of(e + 2);
            process(e, id_cur, kA, vA);
            if (++e >= E)
                break;
            id_cur = id_nxt;
            id_nxt = id_nn;
            issue(e + 1 < E ? e + 1 : E - 1, id_nxt, kA, vA);
            id_nn = id_of(e + 2);
            process(e, id_cur, kB, vB);
            if (++e >= E)
                break;
            id_cur = id_nxt;
            id_nxt = id_nn;
        }
    }

    // Merge the NSUB streams of this workgroup through LDS.
    const int sub = w * R + r;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < CH; ++c)
            lds_o[(sub * G + h) * D + li * CH + c] = o[h][c];
    if ((li & ((1 << (LL - S)) - 1)) == 0) {
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            lds_m[sub * G + (hm | h)] = m[h];
            lds_l[sub * G + (hm | h)] = l[h];
        }
    }
    __syncthreads();

    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int h = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int s2 = 0; s2 < NSUB; ++s2)
            M = fmaxf(M, lds_m[s2 * G + h]);
        float Ls = 0.0f, O = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int s2 = 0; s2 < NSUB; ++s2) {
                const float ms = lds_m[s2 * G + h];
                const float f = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
                Ls = __builtin_fmaf(lds_l[s2 * G + h], f, Ls);
                O = __builtin_fmaf(lds_o[(s2 * G + h) * D + d], f, O);
            }
        }
        const int64_t row = (int64_t)b * a.Hq + hq0 + h;
        if (np == 1) {
            store_out(a.out, a.out_dtype, row * D + d, Ls > 0.0f ? O / Ls : 0.0f);
        } else {
            const int64_t pr = row * a.max_parts + part;
            a.ws_o[pr * D + d] = O;
            if (d == 0) {
                a.ws_ml[pr * 2] = M;
                a.ws_ml[pr * 2 + 1] = Ls;
            }
        }
    }
}

// Log-sum-exp merge of the partitions of every (sequence, query head):
// M = max_p m_p, L = sum_p l_p 2^(m_p - M), out = sum_p o_p 2^(m_p - M) / L,
// summed in partition order.
template <int D, int BS>
__global__ __launch_bounds__(256) void k_merge(Args a)
{
    const int b = blockIdx.y;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= a.Hq * D)
        return;
    int L, nblk, np;
    seq_extent<BS>(a, b, L, nblk, np);
    if (np <= 1)
        return;
    const int h = idx / D, d = idx % D;
    const int64_t row = (int64_t)b * a.Hq + h;
    const float *ml = a.ws_ml + row * a.max_parts * 2;
    const float *op = a.ws_o + row * a.max_parts * D + d;
    float M = -INFINITY;
    for (int p = 0; p < np; ++p)
        M = fmaxf(M, ml[2 * p]);
    float Ls = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
        for (int p = 0; p < np; ++p) {
            const float mp = ml[2 * p];
            const float f = (mp == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mp - M);
            Ls = __builtin_fmaf(ml[2 * p + 1], f, Ls);
            O = __builtin_fmaf(op[(int64_t)p * D], f, O);
        }
    }
    store_out(a.out, a.out_dtype, row * D + d, Ls > 0.0f ? O / Ls : 0.0f);
}

using KernelFn = void (*)(Args);

template <int DT, int D, int BS>
KernelFn pick_g(int G)
{
    switch (G) {
    case 1: return k_decode<DT, D, BS, 1>;
    case 2: return k_decode<DT, D, BS, 2>;
    case 4: return k_decode<DT, D, BS, 4>;
    case 8: return k_decode<DT, D, BS, 8>;
    default: return nullptr;
    }
}

template <int DT, int D>
KernelFn pick_bs(int BS, int G)
{
    return BS == 16 ? pick_g<DT, D, 16>(G) : (BS == 32 ? pick_g<DT, D, 32>(G) : nullptr);
}

template <int DT>
KernelFn pick_d(int D, int BS, int G)
{
    return D == 64 ? pick_bs<DT, 64>(BS, G) : (D == 128 ? pick_bs<DT, 128>(BS, G) : nullptr);
}

KernelFn pick_merge(int D, int BS)
{
    if (D == 64)
        return BS == 16 ? k_merge<64, 16> : k_merge<64, 32>;
    return BS == 16 ? k_merge<128, 16> : k_merge<128, 32>;
}

}  // namespace

int launch_decode(const DecodeLaunch &d)
{
    if (d.num_seqs == 0)
        return PKV_OK;
    const int G = d.num_q_heads / d.num_kv_heads;
    KernelFn fn = d.dtype == PKV_F32 ? pick_d<PKV_F32>(d.head_dim, d.block_size, G)
                                     : pick_d<PKV_BF16>(d.head_dim, d.block_size, G);
    if (!fn)
        return fail(PKV_EUNSUPPORTED, "pkv_decode: no kernel for head_dim %d, block %d, group %d",
                    d.head_dim, d.block_size, G);
    Args a;
    a.q = d.q;
    a.kc = d.k_cache;
    a.vc = d.v_cache;
    a.tables = d.block_tables;
    a.lens = d.context_lens;
    a.out = d.out;
    a.ws_o = d.ws_o;
    a.ws_ml = d.ws_ml;
    a.stride = d.table_stride;
    a.B = d.num_seqs;
    a.Hq = d.num_q_heads;
    a.Hkv = d.num_kv_heads;
    a.num_blocks = d.num_blocks;
    a.part_blocks = d.partition_blocks;
    a.max_parts = d.max_partitions;
    a.out_dtype = d.out_dtype;
    a.scale_log2 = d.scale * 1.4426950408889634f;
    hipStream_t st = reinterpret_cast<hipStream_t>(d.stream);
    hipLaunchKernelGGL(fn, dim3(d.num_kv_heads, d.max_partitions, d.num_seqs), dim3(kThreads), 0,
                       st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(PKV_EHIP, "pkv_decode: launch failed: %s", hipGetErrorString(e));
    if (d.max_partitions > 1) {
        const unsigned gx = (unsigned)((d.num_q_heads * d.head_dim + 255) / 256);
        hipLaunchKernelGGL(pick_merge(d.head_dim, d.block_size), dim3(gx, d.num_seqs), dim3(256), 0,
                           st, a);
        e = hipGetLastError();
        if (e != hipSuccess)
            return fail(PKV_EHIP, "pkv_decode: merge launch failed: %s", hipGetErrorString(e));
    }
    return PKV_OK;
}

}  // namespace pkv
