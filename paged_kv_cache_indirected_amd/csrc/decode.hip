// Paged decode attention for gfx950 (CDNA4): a work-balanced split pass plus
// a log-sum-exp merge pass.
//
// What is computed ("LLM Inference: KV Cache, Batching & Scheduling",
// sections "The KV cache" and "PagedAttention and vLLM"; the "LLM Inference
// Engineering" summary, section 2): for sequence b and query head h, softmax
// attention of q[b][h] over the K/V rows of all L_b prior positions, where
// position j lives in physical block block_tables[b][j / bs] at offset
// j % bs.  Query head h reads KV head h / G.
//
// Work split.  For each KV head the blocks of all sequences are laid end to
// end (sequence b owns positions pref[b] .. pref[b+1] of that line, pref
// being the prefix sum of ceil(L_b / bs)), and the line is cut into W equal
// ranges, one per workgroup.  Every workgroup therefore streams the same
// number of bytes whatever the length mix, so the grid drains together
// instead of waiting on the longest sequence (flash-decoding style split of
// the context, balanced over the whole batch).  A range that covers a
// sequence entirely writes its normalised output; the pieces of a sequence
// cut between workgroups are written as (o, m, l) partials that the merge
// pass combines in workgroup order.  (Merging in the split pass's last
// workgroup would need device-scope release/acquire fences, which write back
// and invalidate the L2 of every XCD and cost far more than a second
// launch.)  The result depends only on the lengths and W, never on physical
// block ids or scheduling.
//
// Inside a workgroup (one KV head g, one range):
//   * 4 waves; for each piece (the part of one sequence inside the range)
//     wave w takes blocks w, w+4, ... of the piece.  A wave is R rows of LPT
//     lanes; lane (row r, i) loads the 16-byte chunk i of token rows r,
//     r+R, ... of each K and V block tile: whole-block, coalesced 16-byte
//     loads straight from HBM into registers, the next sub-tile's loads in
//     flight while the current one is processed.
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
//   * End of a piece: the R row streams of a wave merge in registers with
//     cross-row lane swaps (v_permlane16/32_swap, DPP row_ror), the 4 waves
//     through a 16 KiB LDS buffer.
//   * Grid (Hkv, W) with the KV head fastest, so workgroups of one KV head
//     land on one XCD and blocks shared between sequences stay in its L2.
#include <hip/hip_runtime.h>

#include <utility>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int NW = 4;                 // waves per workgroup
constexpr int kThreads = NW * 64;
constexpr float kLazyMax = 8.0f;      // running-max slack, log2 units
constexpr int kRsrcWord3 = 0x00020000; // raw buffer resource: 32-bit data format, no swizzle
constexpr int kIdChunk = 512;         // block-table entries staged in LDS at a time

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct Args {
    const void *q;
    const void *kc;
    const void *vc;
    const int32_t *tables;
    const int32_t *lens;
    void *out;
    float *ws_o;                      // [Hkv][W + B][G][D] partial outputs
    float *ws_ml;                     // [Hkv][W + B][G][2] running max (log2 units), sum
    int32_t *ws_pref;                 // [B + 1] block prefix sums, for the merge pass
    const void *k_new;                // fused append: [B][Hkv][D] rows (NULL: none)
    const void *v_new;
    const int32_t *slots;             // fused append: slot of sequence b's new row
    void *kc_w;                       // the caches, written by the fused append
    void *vc_w;
    int32_t row_chunks;               // 16-byte chunks per K/V row (LPT)
    int32_t block_size;
    int32_t stride;
    int32_t B, Hq, Hkv, num_blocks;
    int32_t W;                        // workgroups per KV head
    int32_t max_len;                  // context lengths are clamped to this
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
    if constexpr (LPT == 16)   // row_newbcast; every lane is written, so no old value
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                                  0x150 + SRC, 0xF, 0xF, true));
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
        // First pair through the VOP3P form with an inline zero accumulator
        // (the compiler would otherwise zero a register for v_dot2c).
        float a;
        asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(a) : "v"(q.x), "v"(k.x));
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

// Combine v with the value of lane (l ^ X) (X = 8, 16 or 32) by + or max;
// both lanes of a pair get the same bits.
template <int X, bool MAX>
__device__ __forceinline__ float xrow(float v)
{
    float o;
    if constexpr (X == 8) {
        o = __builtin_amdgcn_update_dpp(0.0f, v, 0x128, 0xF, 0xF, false);   // row_ror:8
        return MAX ? fmaxf(v, o) : v + o;
    } else {
        const uint32_t u = __builtin_bit_cast(uint32_t, v);
        auto p = X == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
        const float a = __builtin_bit_cast(float, (uint32_t)p[0]);
        const float b = __builtin_bit_cast(float, (uint32_t)p[1]);
        return MAX ? fmaxf(a, b) : a + b;
    }
}

// Reduce over the R rows of a wave (rows differ in lane bits log2(LPT)..5).
template <int LPT, bool MAX>
__device__ __forceinline__ float rows_reduce(float v)
{
    if constexpr (LPT <= 8)
        v = xrow<8, MAX>(v);
    if constexpr (LPT <= 16)
        v = xrow<16, MAX>(v);
    if constexpr (LPT <= 32)
        v = xrow<32, MAX>(v);
    return v;
}

// Context length of sequence b, clamped to what its table row addresses and
// to the host's bound.
template <int BS>
__device__ __forceinline__ int clamp_len(const Args &a, int b)
{
    const int L = a.lens[b];
    const int cap = min(a.stride * BS, a.max_len);
    return L < 0 ? 0 : (L > cap ? cap : L);
}

// Workgroup whose range holds flattened block x: ranges are
// [floor(T w / W), floor(T (w+1) / W)).
__device__ __forceinline__ int owner(int64_t x, int64_t T, int W)
{
    return (int)(((x + 1) * W + T - 1) / T - 1);
}

// Whether workgroup w got no blocks (possible when W exceeds the batch's
// block count); it then wrote no piece.
__device__ __forceinline__ bool empty_range(int w, int64_t T, int W)
{
    return T * w / W == T * (w + 1) / W;
}

template <int DT, int D, int BS, int G>
__global__ __launch_bounds__(kThreads, 2) void k_decode(Args a)
{
    using Sh = Shape<DT, D, BS, G>;
    constexpr int CH = Sh::CH, LPT = Sh::LPT, R = Sh::R, TPR = Sh::TPR;
    constexpr int SUBTOK = Sh::SUBTOK, NSUBT = Sh::NSUBT;
    constexpr int LL = Sh::LL, LG = Sh::LG, S = Sh::S, GH = Sh::GH;
    constexpr int TILE = BS * D * Sh::ES;              // bytes of one (block, head) tile

    __shared__ int32_t lds_pref[kDecodeMaxSeqs + 1];
    __shared__ __attribute__((aligned(16))) uint4 lds_q[G * LPT];
    __shared__ __attribute__((aligned(16))) uint4 lds_new[2][LPT];   // fused append: K, V row
    __shared__ int32_t lds_ids[kIdChunk];
    __shared__ int32_t lds_wsum[NW];
    __shared__ float lds_o[NW][G * D];
    __shared__ float lds_m[NW][G];
    __shared__ float lds_l[NW][G];

    const int g = blockIdx.x, wg = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane / LPT, li = lane % LPT;

    // Prefix sums of the per-sequence block counts (the same in every
    // workgroup).
    int carry = 0;
    for (int base = 0; base < a.B; base += kThreads) {
        const int b = base + tid;
        int v = b < a.B ? (clamp_len<BS>(a, b) + BS - 1) / BS : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(v, off);
            if (lane >= off)
                v += t;
        }
        if (lane == 63)
            lds_wsum[w] = v;
        __syncthreads();
        int before = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int s = lds_wsum[i];
            before += i < w ? s : 0;
            tot += s;
        }
        if (b < a.B)
            lds_pref[b + 1] = carry + before + v;
        carry += tot;
        __syncthreads();
    }
    if (tid == 0)
        lds_pref[0] = 0;
    __syncthreads();
    const int T = lds_pref[a.B];
    const int hq0 = g * G;

    if (g == 0 && wg == 0)
        for (int i = tid; i <= a.B; i += kThreads)
            a.ws_pref[i] = lds_pref[i];

    const int64_t start = (int64_t)T * wg / a.W, end = (int64_t)T * (wg + 1) / a.W;
    if (start >= end)
        return;

    // First sequence with blocks in the range: the last b with pref[b] <= start.
    int b;
    {
        int lo = 0, hi = a.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (lds_pref[mid] <= start)
                lo = mid;
            else
                hi = mid - 1;
        }
        b = lo;
    }

    const int hm = (li >> (LL - S)) << (LG - S);   // this lane's head permutation
    const int64_t blk_bytes = (int64_t)a.Hkv * TILE;
    const char *kbase = static_cast<const char *>(a.kc) + (int64_t)g * TILE;
    const char *vbase = static_cast<const char *>(a.vc) + (int64_t)g * TILE;
    const uint32_t lane_off = (uint32_t)lane * 16u;

    int64_t x = start;
    while (x < end) {
        while (lds_pref[b + 1] <= x)
            ++b;
        const int sb = lds_pref[b], se = lds_pref[b + 1];
        const int j0 = (int)(x - sb);
        const int j1 = (int)((end < se ? end : (int64_t)se) - sb);
        const int L = clamp_len<BS>(a, b);
        const int nblk = se - sb;
        const int32_t *bt = a.tables + (int64_t)b * a.stride;

        // The group's q rows go to LDS (G * D elements); each lane reads its
        // slices from there when it needs them, heads permuted by its own
        // lane bits: slot h holds query head g*G + (h ^ hm).
        {
            const uint4 *qp = static_cast<const uint4 *>(a.q) + ((int64_t)b * a.Hq + hq0) * LPT;
            for (int i = tid; i < G * LPT; i += kThreads)
                lds_q[i] = qp[i];
        }
        // Fused append: the workgroup holding the sequence's last block
        // writes the step's new K/V row of this KV head to its slot, and
        // keeps it in LDS so that the attention reads position L-1 from it
        // rather than from the cache written in the same launch.
        const int nslot = (a.k_new && j1 == nblk) ? a.slots[b] : -1;
        const bool fresh = (unsigned)nslot < (unsigned)(a.num_blocks * BS);
        if (fresh && tid < 2 * LPT) {
            const int kv = tid / LPT, i = tid % LPT;
            const uint4 row = static_cast<const uint4 *>(kv ? a.v_new : a.k_new)
                [((int64_t)b * a.Hkv + g) * LPT + i];
            lds_new[kv][i] = row;
            const int64_t dst = (((int64_t)(nslot / BS) * a.Hkv + g) * BS + nslot % BS) * LPT + i;
            static_cast<uint4 *>(kv ? a.vc_w : a.kc_w)[dst] = row;
        }
        __syncthreads();

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

        int c0 = j0;                       // first block of the staged id chunk
        auto blk_of = [&](int e) { return c0 + w + (e / NSUBT) * NW; };

        // Issue the 2 * TPR 16-byte loads of one sub-tile through a buffer
        // resource whose base is the wave-uniform tile address (scalar
        // registers) and this lane's fixed 32-bit offset.  A block id outside
        // the pool gets an empty resource, so its loads return zeros without
        // touching memory; every load is unconditional and the wait counts
        // stay exact.
        auto issue = [&](int e, int id, uint4 (&kr)[TPR], uint4 (&vr)[TPR]) {
            const bool ok = (unsigned)id < (unsigned)a.num_blocks;
            const int64_t off = (int64_t)(ok ? id : 0) * blk_bytes + (e % NSUBT) * (TPR * 1024);
            const int nrec = ok ? TPR * 1024 : 0;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(kbase + off), 0, nrec, kRsrcWord3);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(vbase + off), 0, nrec, kRsrcWord3);
#pragma unroll
            for (int t = 0; t < TPR; ++t) {
                kr[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rk, (int)(lane_off + t * 1024u), 0, 0));
                vr[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rv, (int)(lane_off + t * 1024u), 0, 0));
            }
        };

        // One sub-tile: QK^T, online softmax update, PV.
        auto process = [&](int e, int id, uint4 (&kr)[TPR], uint4 (&vr)[TPR]) {
            const int j = blk_of(e);
            const bool ok = (unsigned)id < (unsigned)a.num_blocks;
            if (fresh && j == nblk - 1) {
                const int pl = j * BS + (e % NSUBT) * SUBTOK + r;   // position of token row 0
#pragma unroll
                for (int t = 0; t < TPR; ++t)
                    if (pl + t * R == L - 1) {
                        kr[t] = lds_new[0][li];
                        vr[t] = lds_new[1][li];
                    }
            }
            float acc[G][TPR];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const uint4 qh = lds_q[(h ^ hm) * LPT + li];
#pragma unroll
                for (int t = 0; t < TPR; ++t)
                    acc[h][t] = chunk_dot<DT>(qh, kr[t]);
            }
            halve<0, S, LL, LG, G, TPR>(acc);
            butterfly<LL - S - 1, GH, G, TPR>(acc);

            // Scores in log2 units; positions past the context are masked.
            // The running max only moves when a block's max exceeds it by
            // more than 2^8: exponentials stay <= 256, and the rescale of o
            // is skipped unless some stream of the wave moved.
            const int pos0 = j * BS + (e % NSUBT) * SUBTOK + r;
            const bool full = ok && (j + 1) * BS <= L;      // wave-uniform
            float p[GH][TPR], alpha[GH];
            bool grew = false;
#pragma unroll
            for (int h = 0; h < GH; ++h)
#pragma unroll
                for (int t = 0; t < TPR; ++t)
                    p[h][t] = acc[h][t] * a.scale_log2;
            if (!full) {
#pragma unroll
                for (int h = 0; h < GH; ++h)
#pragma unroll
                    for (int t = 0; t < TPR; ++t)
                        p[h][t] = (ok && pos0 + t * R < L) ? p[h][t] : -INFINITY;
            }
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                float mb = -INFINITY;
#pragma unroll
                for (int t = 0; t < TPR; ++t)
                    mb = fmaxf(mb, p[h][t]);
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

            // The context's last block may hold unused slots, and a bad id
            // reads as zeros: such V must not reach the sum (0 * NaN would).
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

        // Wave w takes blocks j0 + w, j0 + w + NW, ... of the piece, each as
        // NSUBT sub-tiles (units e = 0 .. E-1).  Three register buffers
        // rotate: the loads of units e+1 and e+2 are in flight while unit e
        // is processed.  Loads past the last unit go through an empty
        // resource (zeros, no memory access), so every iteration issues the
        // same loads and the compiler's wait counts stay exact.
        // The piece's block ids are staged through LDS in chunks, so the
        // loop issues no vector-memory reads besides the K/V tiles: a table
        // read would share the in-order load counter with them and waiting
        // for it would drain the prefetch.
        for (; c0 < j1; c0 += kIdChunk) {
          const int c1 = j1 - c0 < kIdChunk ? j1 : c0 + kIdChunk;
          for (int i = tid; i < c1 - c0; i += kThreads)
              lds_ids[i] = bt[c0 + i];
          __syncthreads();
          if (c0 + w < c1) {
            const int E = ((c1 - c0 - w + NW - 1) / NW) * NSUBT;
            auto id_of = [&](int e) {
                const int id = lds_ids[(e < E ? e : E - 1) / NSUBT * NW + w];
                return e < E ? id : -1;
            };
            uint4 kA[TPR], vA[TPR], kB[TPR], vB[TPR], kC[TPR], vC[TPR];
            int idA = id_of(0), idB = id_of(1), idC = id_of(2), idn;
            issue(0, idA, kA, vA);
            issue(1, idB, kB, vB);
            for (int e = 0;;) {
                issue(e + 2, idC, kC, vC);
                idn = id_of(e + 3);
                process(e, idA, kA, vA);
                if (++e >= E)
                    break;
                idA = idn;
                issue(e + 2, idA, kA, vA);
                idn = id_of(e + 3);
                process(e, idB, kB, vB);
                if (++e >= E)
                    break;
                idB = idn;
                issue(e + 2, idB, kB, vB);
                idn = id_of(e + 3);
                process(e, idC, kC, vC);
                if (++e >= E)
                    break;
                idC = idn;
            }
          }
          __syncthreads();
        }

        // Merge the R row streams of the wave in registers: per head, the
        // row's (m, l) from its owning lane, the wave max, then every row's
        // share rescaled and summed across rows.
        float mw[G], lw[G];
        [&]<int... H>(std::integer_sequence<int, H...>) {
            (([&] {
                 constexpr int src = (H >> (LG - S)) << (LL - S);
                 const float mr = bcast<LPT, src>(m[H & (GH - 1)]);
                 const float lr = bcast<LPT, src>(l[H & (GH - 1)]);
                 const float M = rows_reduce<LPT, true>(mr);
                 const float f = (mr == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mr - M);
                 lw[H] = rows_reduce<LPT, false>(lr * f);
                 mw[H] = M;
#pragma unroll
                 for (int c = 0; c < CH; ++c)
                     o[H][c] = rows_reduce<LPT, false>(o[H][c] * f);
             }()),
             ...);
        }(std::make_integer_sequence<int, G>{});

        if (r == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int c = 0; c < CH; ++c)
                    lds_o[w][h * D + li * CH + c] = o[h][c];
            if (li == 0) {
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    lds_m[w][h] = mw[h];
                    lds_l[w][h] = lw[h];
                }
            }
        }
        __syncthreads();

        // Merge the 4 waves; a sequence held whole by this range is final.
        const bool whole = owner(sb, T, a.W) == owner(se - 1, T, a.W);
        for (int idx = tid; idx < G * D; idx += kThreads) {
            const int h = idx / D, d = idx % D;
            float M = -INFINITY;
#pragma unroll
            for (int s2 = 0; s2 < NW; ++s2)
                M = fmaxf(M, lds_m[s2][h]);
            float Ls = 0.0f, O = 0.0f;
            if (M != -INFINITY) {
#pragma unroll
                for (int s2 = 0; s2 < NW; ++s2) {
                    const float ms = lds_m[s2][h];
                    const float f = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
                    Ls = __builtin_fmaf(lds_l[s2][h], f, Ls);
                    O = __builtin_fmaf(lds_o[s2][idx], f, O);
                }
            }
            if (whole) {
                store_out(a.out, a.out_dtype, ((int64_t)b * a.Hq + hq0 + h) * D + d,
                          Ls > 0.0f ? O / Ls : 0.0f);
            } else {
                const int64_t pr = ((int64_t)g * (a.W + a.B) + wg + b) * G + h;
                a.ws_o[pr * D + d] = O;
                if (d == 0) {
                    a.ws_ml[pr * 2] = M;
                    a.ws_ml[pr * 2 + 1] = Ls;
                }
            }
        }
        __syncthreads();
        x = sb + j1;
        ++b;
    }
}

// Log-sum-exp merge of the pieces of every (sequence, query head) cut
// between workgroups: M = max_p m_p, L = sum_p l_p 2^(m_p - M),
// out = sum_p o_p 2^(m_p - M) / L, summed in workgroup order over the
// workgroups whose ranges hold blocks of the sequence.  One workgroup per
// (sequence, query head), one thread per output element; the pieces of a
// sequence are consecutive in the workspace, and the loop over them is
// unrolled so their loads are in flight together.  Empty sequences get zeros
// here; sequences held whole by one workgroup were written by it.
template <int D>
__global__ __launch_bounds__(D) void k_merge(Args a)
{
    const int b = blockIdx.x, hq = blockIdx.y, d = threadIdx.x;
    const int G = a.Hq / a.Hkv;
    const int g = hq / G, h = hq - g * G;
    const int T = a.ws_pref[a.B];
    const int sb = a.ws_pref[b], se = a.ws_pref[b + 1];
    const int64_t oidx = ((int64_t)b * a.Hq + hq) * D + d;
    if (se == sb) {
        store_out(a.out, a.out_dtype, oidx, 0.0f);
        // Fused append of a sequence with no blocks: no split workgroup
        // visits it, so its new row is written here.
        if (a.k_new && h == 0 && d < 2 * a.row_chunks) {
            const int nslot = a.slots[b];
            const int bsz = a.stride > 0 ? a.block_size : 1;
            if ((unsigned)nslot < (unsigned)(a.num_blocks * bsz)) {
                const int kv = d / a.row_chunks, i = d % a.row_chunks;
                const uint4 row = static_cast<const uint4 *>(kv ? a.v_new : a.k_new)
                    [((int64_t)b * a.Hkv + g) * a.row_chunks + i];
                const int64_t dst = (((int64_t)(nslot / bsz) * a.Hkv + g) * bsz + nslot % bsz) *
                                        a.row_chunks + i;
                static_cast<uint4 *>(kv ? a.vc_w : a.kc_w)[dst] = row;
            }
        }
        return;
    }
    const int wf = owner(sb, T, a.W), wl = owner(se - 1, T, a.W);
    if (wf == wl)
        return;
    const bool sparse = T < a.W;   // only then can a range be empty
    // Piece (w + b) of KV head g, query head h within the group.
    const int64_t p0 = ((int64_t)g * (a.W + a.B) + b) * G + h;
    float M = -INFINITY;
#pragma unroll 8
    for (int w = wf; w <= wl; ++w)
        if (!sparse || !empty_range(w, T, a.W))
            M = fmaxf(M, a.ws_ml[(p0 + (int64_t)w * G) * 2]);
    float Ls = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
#pragma unroll 8
        for (int w = wf; w <= wl; ++w) {
            if (sparse && empty_range(w, T, a.W))
                continue;
            const int64_t pr = p0 + (int64_t)w * G;
            const float mp = a.ws_ml[pr * 2];
            const float f = (mp == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mp - M);
            Ls = __builtin_fmaf(a.ws_ml[pr * 2 + 1], f, Ls);
            O = __builtin_fmaf(a.ws_o[pr * D + d], f, O);
        }
    }
    store_out(a.out, a.out_dtype, oidx, Ls > 0.0f ? O / Ls : 0.0f);
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

}  // namespace

int32_t device_cu_count()
{
    constexpr int kMaxDev = 64;
    static int32_t cached[kMaxDev] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
        (void)hipGetLastError();
        return 256;
    }
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cached[dev] = n;
    }
    return cached[dev];
}

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
    KernelFn merge = d.head_dim == 64 ? k_merge<64> : k_merge<128>;
    hipStream_t st = reinterpret_cast<hipStream_t>(d.stream);
    const int esz = d.dtype == PKV_F32 ? 4 : 2;
    const int osz = d.out_dtype == PKV_F32 ? 4 : 2;
    // Sequences go in launches of at most kDecodeMaxSeqs (the prefix sums
    // live in LDS); the workspace is reused, launches being stream-ordered.
    for (int32_t b0 = 0; b0 < d.num_seqs; b0 += kDecodeMaxSeqs) {
        const int32_t nb = d.num_seqs - b0 < kDecodeMaxSeqs ? d.num_seqs - b0 : kDecodeMaxSeqs;
        Args a;
        a.q = static_cast<const char *>(d.q) + (int64_t)b0 * d.num_q_heads * d.head_dim * esz;
        a.kc = d.k_cache;
        a.vc = d.v_cache;
        a.tables = d.block_tables + (int64_t)b0 * d.table_stride;
        a.lens = d.context_lens + b0;
        a.out = static_cast<char *>(d.out) + (int64_t)b0 * d.num_q_heads * d.head_dim * osz;
        a.ws_o = d.ws_o;
        a.ws_ml = d.ws_ml;
        a.ws_pref = d.ws_pref;
        a.k_new = d.k_new ? static_cast<const char *>(d.k_new) +
                                (int64_t)b0 * d.num_kv_heads * d.head_dim * esz
                          : nullptr;
        a.v_new = d.v_new ? static_cast<const char *>(d.v_new) +
                                (int64_t)b0 * d.num_kv_heads * d.head_dim * esz
                          : nullptr;
        a.slots = d.slots ? d.slots + b0 : nullptr;
        a.kc_w = d.k_cache_w;
        a.vc_w = d.v_cache_w;
        a.row_chunks = d.head_dim * esz / 16;
        a.block_size = d.block_size;
        a.stride = d.table_stride;
        a.B = nb;
        a.Hq = d.num_q_heads;
        a.Hkv = d.num_kv_heads;
        a.num_blocks = d.num_blocks;
        a.W = d.num_splits;
        a.max_len = d.max_context_len;
        a.out_dtype = d.out_dtype;
        a.scale_log2 = d.scale * 1.4426950408889634f;
        hipLaunchKernelGGL(fn, dim3(d.num_kv_heads, d.num_splits), dim3(kThreads), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(PKV_EHIP, "pkv_decode: launch failed: %s", hipGetErrorString(e));
        hipLaunchKernelGGL(merge, dim3(nb, d.num_q_heads), dim3(d.head_dim), 0, st, a);
        e = hipGetLastError();
        if (e != hipSuccess)
            return fail(PKV_EHIP, "pkv_decode: merge launch failed: %s", hipGetErrorString(e));
    }
    return PKV_OK;
}

}  // namespace pkv
