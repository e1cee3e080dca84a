// Causal chunked prefill over the paged cache on gfx950 (CDNA4) MFMA.
//
// What is computed ("LLM Inference: KV Cache, Batching & Scheduling",
// sections "Chunked prefill" and "The KV cache"): a prompt is processed in
// fixed-size chunks interleaved with decode; chunking changes the schedule,
// not the result.  Sequence s holds L_s keys, its chunk of C_s tokens already
// appended, so chunk token i (0 <= i < C_s) attends keys 0 .. L_s - C_s + i,
// diagonal included.  Query head h reads KV head h / G.  Keys live in paged
// blocks (same page, "PagedAttention and vLLM"): key j of sequence s sits in
// block block_tables[s][j / bs] at offset j % bs.
//
// Design (one workgroup = 128 GQA-packed query rows of one (sequence, KV
// head); row r is chunk token r / G, query head g*G + r % G, so every K/V
// tile staged once serves all G heads of the group):
//   * 4 waves x 32 rows (NCT = 2 column tiles of 16; 48 rows per wave need
//     more than half the register file, and one wave per SIMD ran 1.6x
//     slower).  Keys are processed in tiles of 64.  The workgroup stages
//     each tile of K ([64][D], row-major) and V (per dim, the 8 keys of one
//     PV operand side by side) into LDS from the paged cache with coalesced
//     16-byte loads (1 KiB runs of a block's tile), double buffered: the
//     next tile's global loads are in flight while the current tile is
//     computed.
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = K from LDS, B = the wave's
//     Q rows held in registers for the whole kernel).  Computing the
//     transpose leaves each lane with 4 consecutive keys of one query column,
//     which is exactly the B-operand layout P^T needs for the PV product, so
//     P never leaves registers.
//   * Online softmax per query column in log2 units: tile max reduced over
//     the 4 lane groups of the column, lazy running max (rescale only when
//     the max grows by more than 2^8), masking by select on tiles that cross
//     the causal diagonal or the end of the context.
//   * O^T = V^T P^T on MFMA with fp32 accumulation.  P is split into
//     bf16 hi + lo parts (two MFMAs), so the weights keep ~16 significant
//     bits instead of bf16's 8; the PV error then stays far below the
//     2e-3 bar even on rows that attend a handful of keys.
//   * Grid (Hkv, q-tiles, sequences): the KV head is fastest so all q-tiles
//     of one (sequence, head) land on one XCD and share its L2; q-tiles run
//     last-to-first, the longest (most keys) first.
//   * The loop is software-pipelined inside each wave: the body for key
//     tile kt runs tile kt - 1's PV product beside tile kt's softmax and
//     P split, and tile kt + 1's S product beside the staging, in slots
//     whose order scheduling fences fix, so that the matrix cores have
//     vector work of the same wave beside them.  One LDS-only barrier per
//     tile.  Block ids stream through a ring in LDS, so tables of any
//     length work.
// Unused slots and keys past the context are staged as zeros and masked; a
// block id outside the pool is read as zeros without touching memory.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "pkv_internal.h"

#ifdef PKV_DEBUG
// Device preconditions found violated by this module's kernels (kDbg* bits).
static __device__ uint32_t dbg_word;
#define PKV_DBG_NOTE(bit) atomicOr(&dbg_word, (bit))
#else
#define PKV_DBG_NOTE(bit) ((void)0)
#endif

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int NW = 4;                  // waves per workgroup
constexpr int kThreads = NW * 64;
constexpr int KT = 64;                 // keys per tile
constexpr int NCT = 2;                 // 16-column MFMA tiles per wave
constexpr int WROWS = 16 * NCT;        // query rows per wave
constexpr int ROWS = NW * WROWS;       // query rows per workgroup
constexpr float kLazyMax = 8.0f;       // running-max slack, log2 units
constexpr int kIdChunk = 1024;         // slots of the LDS ring of block ids
constexpr int kRsrcWord3 = 0x00020000; // raw buffer resource: 32-bit data format, no swizzle

template <int D>
struct PShape {
    static constexpr int KSTR = D + 8;               // LDS row stride of K (elements)
    static constexpr int VPS = 8 * D;                // LDS stride of a V group pair (elements)
    static constexpr int KBUF = KT * KSTR;
    static constexpr int VBUF = (KT / 8) * VPS;
    static constexpr int NDS = D / 32;               // k-steps of S^T over head_dim
    static constexpr int NDT = D / 16;               // 16-row tiles of O^T
    static constexpr int CPR = D / 8;                // 16-byte chunks per K/V row
    static constexpr int KLD = KT * CPR / kThreads;  // K chunks staged per thread
    static constexpr int VK = KT * CPR / kThreads;   // V 16-byte units staged per thread
    static_assert(KLD * kThreads == KT * CPR && (VK == 2 || VK == 4), "staging shape");
};

struct PArgs {
    const uint16_t *q;
    const int32_t *qsl;
    const uint16_t *kc;
    const uint16_t *vc;
    const int32_t *tables;
    const int32_t *lens;
    void *out;
    int32_t stride, Hq, Hkv, num_blocks, n_qtiles, out_dtype;
    int32_t S;                        // sequences in the launch
    int32_t causal;                   // 0: every row attends all L keys of its sequence
    int32_t q_shared;                 // 1: every sequence reads its queries from rows 0..C-1
    float *lse;                       // optional [rows][Hq]: log2-sum-exp of the scaled scores
    float scale_log2;
    int32_t ks;                       // key splits: split k writes state k (fp32 out + lse)
    int64_t split_rows;               // rows of one split's state (out / lse stride)
    // syn_rows > 0: the sequences are the ranges of one block list (cascade
    // prefix): sequence s has syn_rows query rows from row s * syn_rows and
    // min(syn_nbk, syn_nb - s * syn_nbk) blocks of keys (qsl, lens unused).
    int32_t syn_rows, syn_nbk, syn_nb;
};

template <int BS>
__device__ __forceinline__ int seq_len(const PArgs &a, int s)
{
    return a.syn_rows > 0 ? min(a.syn_nbk, a.syn_nb - s * a.syn_nbk) * BS : a.lens[s];
}


__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x40);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Maximum that propagates NaN (IEEE 754-2019 maximum): gfx950 has it as a
// 3-input instruction that needs no quieting of its inputs, unlike fmaxf.
// A NaN score can only come from a NaN in the attended keys or the query,
// where the result is NaN either way (masked scores are -inf, never NaN).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Combine v with lane (l ^ X) (X = 16 or 32) by max; both lanes get the
// same bits.
template <int X>
__device__ __forceinline__ float xmax(float v)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    auto p = X == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                     : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return vmax(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
}
template <int X>
__device__ __forceinline__ float xsum(float v)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    auto p = X == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                     : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
}

// Workgroup barrier ordering LDS only (global loads in flight stay in flight).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The loop: the body for tile kt runs the PV product of tile kt - 1 beside
// the softmax of tile kt, and the S product of tile kt + 1 beside the P
// split of tile kt, so that the matrix cores and the vector units have
// independent work at every point.  K is staged two tiles ahead and V one
// (K tile t and V tile t in LDS buffer t & 1), through registers loaded one
// tile earlier.  The first tile's PV is that of an all-zero P over a
// zeroed V buffer.
template <int D, int BS, int G>
__global__ __launch_bounds__(kThreads, NCT == 2 ? 2 : 1) void k_prefill(PArgs a)
{
    using Sh = PShape<D>;
    constexpr int TQ = ROWS / G;                     // chunk tokens per workgroup
    constexpr int NDS = Sh::NDS, NDT = Sh::NDT, CPR = Sh::CPR, VK = Sh::VK;
    constexpr int KSTR = Sh::KSTR, VPS = Sh::VPS;
    constexpr int IDS = kIdChunk;                    // ring of block ids in LDS
    constexpr int IPT = KT / BS;                     // block ids per key tile

    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][Sh::KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][Sh::VBUF];
    __shared__ int32_t lds_ids[IDS];

    const int g = blockIdx.x;
    const int qt = a.n_qtiles - 1 - (int)blockIdx.y / a.ks;
    const int ksp = (int)blockIdx.y % a.ks;          // key split of this workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, quad = lane >> 4;

    // Sequences are taken longest context first (grid z is the rank), so the
    // heaviest workgroups start first and the light ones fill the tail.
    // Ranking is done for up to 64 sequences; beyond that, in order.
    int s = blockIdx.z;
    if (a.S <= 64) {
        const int i = lane < a.S ? lane : 0;
        const int wi = seq_len<BS>(a, i);
        int rank = 0;
        for (int j = 0; j < a.S; ++j) {
            const int wj = __builtin_amdgcn_readlane(wi, j);
            rank += (wj > wi || (wj == wi && j < i)) ? 1 : 0;
        }
        const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < a.S && rank == (int)blockIdx.z);
        s = hit ? __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit)) : blockIdx.z;
    }

    const int q0 = a.syn_rows > 0 ? s * a.syn_rows : a.qsl[s];
    const int C = a.syn_rows > 0 ? a.syn_rows : a.qsl[s + 1] - q0;
    int L = seq_len<BS>(a, s);
    const int cap = a.stride * BS;
    if (a.syn_rows == 0 && (L < 0 || L > cap || L < C))
        PKV_DBG_NOTE(kDbgLength);
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int p0 = L - C;                            // keys before the chunk
    const int tok0 = qt * TQ;
    if (tok0 >= C)
        return;
    const int tok_end = min(C, tok0 + TQ);
    const int kend = a.causal ? min(L, p0 + tok_end) : L;   // keys any row of this tile attends
    const int NT = kend > 0 ? (kend + KT - 1) / KT : 0;
    // Key split ksp takes tiles [t0, t1) of the NT; an empty split still
    // writes its (zero, -inf) state.
    const int t0 = (int)((int64_t)NT * ksp / a.ks);
    const int t1 = (int)((int64_t)NT * (ksp + 1) / a.ks);

    // This lane's two query columns (one per 16-row MFMA tile).
    int lim[NCT];
    bool valid[NCT];
    int64_t qrow[NCT], qin[NCT];
    const int qbase = a.q_shared ? 0 : q0;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const int r = w * WROWS + ct * 16 + n;
        const int tok = tok0 + r / G;
        valid[ct] = tok < tok_end;
        lim[ct] = valid[ct] ? (a.causal ? p0 + tok : L - 1) : -1;
        qrow[ct] = ((int64_t)(q0 + tok) * a.Hq + g * G + r % G) * D;
        qin[ct] = ((int64_t)(qbase + tok) * a.Hq + g * G + r % G) * D;
    }
    // Smallest key limit over the wave's valid rows (wave-uniform): a tile
    // entirely at or below it needs no mask.
    const int wtok = tok0 + (w * WROWS) / G;
    const int lim_w = wtok < tok_end ? (a.causal ? p0 + wtok : L - 1) : 0x7FFFFFFF;

    // Scores enter the exponent as fma(s, c, -m) with c = |scale| log2(e):
    // for a negative scale the q operand's sign bits are flipped (exact), so
    // the running max of s * c is c times the max of the raw scores.
    // (c is kept away from 0 so that masked -inf scores still give 0.)
    const float c = fmaxf(a.scale_log2 < 0.0f ? -a.scale_log2 : a.scale_log2, 1e-30f);
    const uint32_t qsign = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
    bf16x8 qf[NCT][NDS];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            // Unconditional load (row 0 for a padding column, which the
            // chunk always has), so all of the wave's q loads are in flight
            // together; a load under the condition was waited for alone.
            // (The mask is applied arithmetically: a select lets the
            // compiler move the load back under the condition.)
            const uint4 v = *reinterpret_cast<const uint4 *>(
                a.q + (valid[ct] ? qin[ct] : 0) + ds * 32 + quad * 8);
            const uint32_t mk = 0u - (uint32_t)valid[ct];
            const uint4 x = make_uint4((v.x ^ qsign) & mk, (v.y ^ qsign) & mk,
                                       (v.z ^ qsign) & mk, (v.w ^ qsign) & mk);
            qf[ct][ds] = __builtin_bit_cast(bf16x8, x);
        }

    const int32_t *bt = a.tables + (int64_t)s * a.stride;
    const int64_t hstride = (int64_t)BS * D;         // elements per (block, head) tile
    const int64_t bstride = (int64_t)a.Hkv * hstride;
    const uint16_t *kg = a.kc + g * hstride;
    const uint16_t *vg = a.vc + g * hstride;
    const int nblk = (kend + BS - 1) / BS;           // blocks the workgroup reads

    // Block ids live in a ring of IDS slots (block j at slot j % IDS),
    // two halves of HALF key tiles: the key range's first 2 HALF tiles are
    // staged at the start, and when the loop enters a new half, the half
    // it has left is restaged with the ids HALF tiles further on, used only
    // after many per-tile barriers.  Tables of any length stream through.
    constexpr int HALF = IDS / IPT / 2;
    auto id_at = [&](int jb) {
        const int v = bt[jb < nblk ? jb : (nblk > 0 ? nblk - 1 : 0)];
        if (jb < nblk && (unsigned)v >= (unsigned)a.num_blocks)
            PKV_DBG_NOTE(kDbgBlockId);
        return jb < nblk ? v : -1;
    };
    auto stage_ids = [&](int t, int count) {       // ids of count tiles from tile t
        constexpr int PER = IDS / kThreads;
        int idv[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * kThreads;
            idv[k] = i < count * IPT ? id_at(t * IPT + i) : -1;
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int i = tid + k * kThreads;
            if (i < count * IPT)
                lds_ids[(t * IPT + i) & (IDS - 1)] = idv[k];
        }
    };
    auto restage = [&](int kt) {
        if (kt > t0 && ((kt - t0) & (HALF - 1)) == 0)
            stage_ids(kt + HALF, HALF);
    };

    uint4 kst[Sh::KLD], vst[VK];
    // Global loads of key tile kt into registers.  K: wave w reads part wp
    // of block w / WPB of the tile (WPB = waves per block), one 1 KiB run of
    // the block's (block, head) tile per load; K keeps each token's dims in
    // 16-byte chunks (chunk c of token t at (c * BS + t) * 16 bytes).  V
    // keeps 4 consecutive tokens of one dim together (element (t, d) at
    // ((t / 4) * D + d) * 4 + t % 4, a 4-key group being one 8 D-byte run),
    // and is read in pairs of groups: pair pr = 4 s2 + qd holds the groups of
    // keys 32 s2 + 16 h + 4 qd .. + 3 for h = 0, 1, the two halves of one PV
    // operand.  Wave w reads pairs 2 w and 2 w + 1 (so s2 = w / 2), each lane
    // the same 16-byte unit (2 dims x 4 keys) of both groups of a pair, so
    // that it can store both halves of a dim side by side.  Each load goes
    // through a buffer resource on the wave's block held in scalar registers;
    // a block id outside the pool, or a block past the context, gets an
    // empty resource and reads zeros without touching memory.
    constexpr int WPB = NW * BS / KT;                // waves per block of the tile
    const int wblk = BS * (w / WPB);                 // the wave's first key in the tile
    const int wp = w % WPB;
    static_assert(VK * 64 == 2 * D, "two V group pairs per wave");
    const int vs2 = w / 2;
    int vquad[VK / 2], vu[VK / 2];
#pragma unroll
    for (int j = 0; j < VK / 2; ++j) {
        const int cid = (w * (VK / 2) + j) * 64 + lane;
        vquad[j] = (cid / (D / 2)) % 4;
        vu[j] = cid % (D / 2);
    }
    // (The id is read unconditionally, at an index kept inside the list,
    // and then selected, so that no branch splits the pipelined body.)
    auto tile_rsrc = [&](const uint16_t *base, int j) {
        const int jj = __builtin_amdgcn_readfirstlane(j);
        const int idr = __builtin_amdgcn_readfirstlane(lds_ids[(jj / BS) & (IDS - 1)]);
        const int ids = idr | -(int)(jj >= L);                  // -1 past the context
        const int okm = -(int)((unsigned)ids < (unsigned)a.num_blocks);
        return __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(base + (int64_t)(ids & okm) * bstride), 0,
            (int)(hstride * 2) & okm, kRsrcWord3);
    };
    auto load_k = [&](int kt) {
        const auto rk = tile_rsrc(kg, kt * KT + wblk);
#pragma unroll
        for (int i = 0; i < Sh::KLD; ++i)
            kst[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rk, ((wp * Sh::KLD + i) * 64 + lane) * 16, 0, 0));
    };
    auto load_v = [&](int kt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const auto rv = tile_rsrc(vg, kt * KT + 32 * vs2 + (BS == 16 ? 16 * h : 0));
#pragma unroll
            for (int j = 0; j < VK / 2; ++j)
                vst[2 * j + h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    rv, (BS == 16 ? vquad[j] : 4 * h + vquad[j]) * 8 * D + vu[j] * 16, 0, 0));
        }
    };
    auto store_k = [&](int kt) {
        const int buf = kt & 1;
#pragma unroll
        for (int i = 0; i < Sh::KLD; ++i) {
            const int q = (wp * Sh::KLD + i) * 64 + lane;
            const int kk = wblk + q % BS, cc = q / BS;
            *reinterpret_cast<uint4 *>(&lds_k[buf][kk * KSTR + cc * 8]) = kst[i];
        }
    };
    auto store_v = [&](int kt, auto tail) {
        const int buf = kt & 1;
        if (decltype(tail)::value && kt * KT + KT > L) {   // keys past the end: zeros, not NaN
#pragma unroll
            for (int j = 0; j < VK / 2; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int nv = L - (kt * KT + 32 * vs2 + 16 * h + 4 * vquad[j]);
                    const uint32_t m01 = (nv > 0 ? 0x0000FFFFu : 0u) | (nv > 1 ? 0xFFFF0000u : 0u);
                    const uint32_t m23 = (nv > 2 ? 0x0000FFFFu : 0u) | (nv > 3 ? 0xFFFF0000u : 0u);
                    uint4 &x = vst[2 * j + h];
                    x.x &= m01;
                    x.y &= m23;
                    x.z &= m01;
                    x.w &= m23;
                }
        }
#pragma unroll
        for (int j = 0; j < VK / 2; ++j) {
            uint16_t *v0 = &lds_v[buf][(4 * vs2 + vquad[j]) * VPS + 2 * vu[j] * 8];
            const uint4 a0 = vst[2 * j], b0 = vst[2 * j + 1];
            *reinterpret_cast<uint4 *>(v0) = make_uint4(a0.x, a0.y, b0.x, b0.y);
            *reinterpret_cast<uint4 *>(v0 + 8) = make_uint4(a0.z, a0.w, b0.z, b0.w);
        }
    };

    f32x4 o[NDT][NCT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            o[dt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m[NCT], lsum[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        m[ct] = -INFINITY;
        lsum[ct] = 0.0f;
    }
    bf16x8 phi[NCT][2], plo[NCT][2];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            phi[ct][s2] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
            plo[ct][s2] = phi[ct][s2];
        }
    f32x4 sacc[4][NCT];

    // S^T rows ks0 .. ks0 + 1 (32 keys) of key tile kt from LDS buffer
    // kt & 1, into sacc[ks0], sacc[ks0 + 1].
    auto s_half = [&](int kt, int ks0) {
        const int buf = kt & 1;
#pragma unroll
        for (int ks = ks0; ks < ks0 + 2; ++ks)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                sacc[ks][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
            for (int ks = ks0; ks < ks0 + 2; ++ks) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(
                    &lds_k[buf][(ks * 16 + n) * KSTR + ds * 32 + quad * 8]);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    sacc[ks][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[ct][ds],
                                                                           sacc[ks][ct], 0, 0, 0);
            }
    };
    // O^T += V^T P^T (hi and lo) for the V tile in LDS buffer buf.
    auto pv_tile = [&](int buf) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            auto vload = [&](int dt) {
                return *reinterpret_cast<const bf16x8 *>(
                    &lds_v[buf][(4 * s2 + quad) * VPS + (dt * 16 + n) * 8]);
            };
            bf16x8 vprev = vload(0);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                o[0][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vprev, phi[ct][s2], o[0][ct],
                                                                   0, 0, 0);
#pragma unroll
            for (int dt = 1; dt < NDT; ++dt) {
                const bf16x8 va = vload(dt);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    o[dt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi[ct][s2],
                                                                        o[dt][ct], 0, 0, 0);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    o[dt - 1][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        vprev, plo[ct][s2], o[dt - 1][ct], 0, 0, 0);
                vprev = va;
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                o[NDT - 1][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    vprev, plo[ct][s2], o[NDT - 1][ct], 0, 0, 0);
        }
    };
    bool grew = false;
    float alpha[NCT];
    // Softmax of tile kt's scores in sacc: exponentials in place, running
    // max and sum updated, rescale factor alpha.
    auto softmax1 = [&](int kt, auto mask) {
        if constexpr (decltype(mask)::value) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (kt * KT + ks * 16 + quad * 4 + i > lim[ct])
                            sacc[ks][ct][i] = -INFINITY;
        }
        grew = false;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            float mt = vmax(sacc[0][ct][0], vmax(sacc[0][ct][1], sacc[0][ct][2]));
#pragma unroll
            for (int k = 3; k < 15; k += 2)
                mt = vmax(mt, vmax(sacc[k / 4][ct][k % 4], sacc[(k + 1) / 4][ct][(k + 1) % 4]));
            mt = vmax(mt, sacc[3][ct][3]);
            mt = xmax<16>(mt);
            mt = xmax<32>(mt) * c;
            const bool up = mt > m[ct] + kLazyMax;
            const float mn = up ? mt : m[ct];
            alpha[ct] = up ? __builtin_amdgcn_exp2f(m[ct] - mn) : 1.0f;
            grew |= up;
            m[ct] = mn;
            const float negm = mn == -INFINITY ? 0.0f : -mn;
            float sum = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[ks][ct][i], c, negm));
                    sacc[ks][ct][i] = p;
                    sum += p;
                }
            lsum[ct] = __builtin_fmaf(lsum[ct], alpha[ct], sum);
        }
    };
    // P^T operands of k-step s2 (keys 32 s2 ..), hi = p truncated to bf16,
    // lo = bf16(p - hi), from the exponentials in sacc[2 s2], sacc[2 s2 + 1].
    auto split_pc = [&](int s2, int ct) {
        {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const float p0v = sacc[2 * s2 + hh][ct][i], p1v = sacc[2 * s2 + hh][ct][i + 1];
                    const uint32_t u0 = __builtin_bit_cast(uint32_t, p0v);
                    const uint32_t u1 = __builtin_bit_cast(uint32_t, p1v);
                    const float r0 = p0v - __builtin_bit_cast(float, u0 & 0xFFFF0000u);
                    const float r1 = p1v - __builtin_bit_cast(float, u1 & 0xFFFF0000u);
                    hw[hh * 2 + i / 2] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
                    lw[hh * 2 + i / 2] = __builtin_bit_cast(
                        uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2_t));
                }
            phi[ct][s2] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
            plo[ct][s2] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
        }
    };
    auto split_p = [&](int s2) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            split_pc(s2, ct);
    };
    // A tile no row masks, as one branch-free block (after the rarely
    // taken O rescale for the previous tile's max growth) whose order is
    // fixed by scheduling fences: each slot holds a few MFMAs and a slice
    // of the vector work they do not depend on, and no instruction crosses
    // a slot boundary.  Part A: the previous tile's PV (64 MFMAs, its V
    // operands read from LDS two steps ahead) beside this tile's softmax and
    // the first k-step's P split.  Part B: the next tile's S (32 MFMAs, K
    // operands one step ahead) beside the second k-step's split and the
    // staging.  Such a tile needs no V zeroing past the context end, and its
    // staging runs unconditionally: tiles past the range read through empty
    // buffer resources, into buffers no later tile reads.
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    auto tile_full = [&](int kt) {
        restage(kt);
        if (__builtin_amdgcn_ballot_w64(grew) != 0) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    o[dt][ct] *= alpha[ct];
        }
        const int vb = (kt + 1) & 1;     // V buffer of tile kt - 1
        auto vload = [&](int s2, int dt) {
            return *reinterpret_cast<const bf16x8 *>(
                &lds_v[vb][(4 * s2 + quad) * VPS + (dt * 16 + n) * 8]);
        };
        // Softmax slices.
        float mt[NCT], negm[NCT], sum[NCT];
        auto sm_slice = [&](int i) {
            if (i < NCT) {               // partial max of column tile i
                const int ct = i;
                float x = vmax(sacc[0][ct][0], vmax(sacc[0][ct][1], sacc[0][ct][2]));
#pragma unroll
                for (int k = 3; k < 15; k += 2)
                    x = vmax(x, vmax(sacc[k / 4][ct][k % 4], sacc[(k + 1) / 4][ct][(k + 1) % 4]));
                mt[ct] = vmax(x, sacc[3][ct][3]);
            } else if (i == NCT) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    mt[ct] = xmax<16>(mt[ct]);
            } else if (i == NCT + 1) {
                grew = false;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const float x = xmax<32>(mt[ct]) * c;
                    const bool up = x > m[ct] + kLazyMax;
                    const float mn = up ? x : m[ct];
                    alpha[ct] = up ? __builtin_amdgcn_exp2f(m[ct] - mn) : 1.0f;
                    grew |= up;
                    m[ct] = mn;
                    negm[ct] = mn == -INFINITY ? 0.0f : -mn;
                    sum[ct] = 0.0f;
                }
            } else if (i < NCT + 2 + 8) {  // exponentials: 4 per column tile per slice
                const int e = i - (NCT + 2), ks = e / 2, ct = e % 2;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[ks][ct][j], c,
                                                                           negm[ct]));
                    sacc[ks][ct][j] = pj;
                    sum[ct] += pj;
                }
            } else if (i == NCT + 10) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    lsum[ct] = __builtin_fmaf(lsum[ct], alpha[ct], sum[ct]);
            } else if (i < NCT + 11 + NCT) {
                split_pc(0, i - (NCT + 11));   // the first k-step's P operands
            }
        };
        // Part A: 2 NDT PV steps (hi of dims tile dt, lo of dt - 1) beside
        // the softmax slices.
        bf16x8 vcur = vload(0, 0), vprev = vcur, vnext1 = vload(0, 1);
        int slice = 0;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const int st2 = s2 * NDT + dt + 2;           // step whose operand loads now
                const bf16x8 vnext2 = st2 < 2 * NDT ? vload(st2 / NDT, st2 % NDT) : vcur;
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    o[dt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vcur, phi[ct][s2],
                                                                        o[dt][ct], 0, 0, 0);
                if (dt > 0) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        o[dt - 1][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            vprev, plo[ct][s2], o[dt - 1][ct], 0, 0, 0);
                }
                sm_slice(slice++);
                if (dt == NDT - 1) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct)
                        o[dt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            vcur, plo[ct][s2], o[dt][ct], 0, 0, 0);
                }
                vprev = vcur;
                vcur = vnext1;
                vnext1 = vnext2;
                fence();
            }
        for (; slice < NCT + 11 + NCT; ++slice)   // (head_dim 64: fewer PV steps than slices)
            sm_slice(slice);
        // Part B: the next tile's S in 2 NDS steps beside the split of the
        // second k-step and the staging.
        const int kb = (kt + 1) & 1;
        auto kload = [&](int ks, int ds) {
            return *reinterpret_cast<const bf16x8 *>(
                &lds_k[kb][(ks * 16 + n) * KSTR + ds * 32 + quad * 8]);
        };
        f32x4 snew[4][NCT];
        // K operands loaded one step ahead of their MFMAs.
        bf16x8 kcur[2] = {kload(0, 0), kload(1, 0)};
#pragma unroll
        for (int step = 0; step < 2 * NDS; ++step) {
            const int ks = (step / NDS) * 2, ds = step % NDS;
            const int nstep = step + 1 < 2 * NDS ? step + 1 : step;
            const int nks = (nstep / NDS) * 2, nds = nstep % NDS;
            const bool more = step + 1 < 2 * NDS;
            const bf16x8 knext[2] = {more ? kload(nks, nds) : kcur[0],
                                     more ? kload(nks + 1, nds) : kcur[1]};
#pragma unroll
            for (int kk = ks; kk < ks + 2; ++kk) {
                const bf16x8 ka = kcur[kk - ks];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    snew[kk][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        ka, qf[ct][ds], ds == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : snew[kk][ct],
                        0, 0, 0);
            }
            kcur[0] = knext[0];
            kcur[1] = knext[1];
            if (step < NCT)
                split_pc(1, step);
            if (step == NDS) {
                store_k(kt + 2);
                store_v(kt, std::false_type{});
            }
            if (step == NDS + 1)
                load_k(kt + 3);
            if (step == 2 * NDS - 1)
                load_v(kt + 1);
            fence();
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                sacc[ks][ct] = snew[ks][ct];
        lds_barrier();
    };

    // A tile some row masks (the causal diagonal, or the context end): the
    // same steps in plain order, with the mask, the V zeroing past the
    // context end and range checks on the staging.
    auto tile_masked = [&](int kt) {
        restage(kt);
        if (__builtin_amdgcn_ballot_w64(grew) != 0) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    o[dt][ct] *= alpha[ct];
        }
        pv_tile((kt + 1) & 1);           // buffer of tile kt - 1
        softmax1(kt, std::true_type{});
        split_p(0);
        split_p(1);
        s_half(kt + 1, 0);
        s_half(kt + 1, 2);
        if (kt + 2 < t1)
            store_k(kt + 2);
        store_v(kt, std::true_type{});
        if (kt + 3 < t1)
            load_k(kt + 3);
        if (kt + 1 < t1)
            load_v(kt + 1);
        lds_barrier();
    };

    if (t1 > t0) {
        stage_ids(t0, 2 * HALF);
        __syncthreads();
        load_k(t0);
        store_k(t0);
        if (t0 + 1 < t1) {
            load_k(t0 + 1);
            store_k(t0 + 1);
        }
        // The first tile's PV of "tile t0 - 1" runs with P = 0: its V buffer
        // must hold finite values.
        for (int i = tid; i < Sh::VBUF / 8; i += kThreads)
            *reinterpret_cast<uint4 *>(&lds_v[(t0 + 1) & 1][i * 8]) = make_uint4(0, 0, 0, 0);
        if (t0 + 2 < t1)
            load_k(t0 + 2);
        load_v(t0);
        __syncthreads();
        s_half(t0, 0);
        s_half(t0, 2);
    }

    // Tiles that no row of the workgroup masks (wave 0 holds the lowest
    // limit), then the rest with the mask.
    const int lim0 = __builtin_amdgcn_readfirstlane(
        tok0 < tok_end ? (a.causal ? p0 + tok0 : L - 1) : -1);
    int tf = (lim0 + 1) / KT;
    tf = tf < t0 ? t0 : (tf > t1 ? t1 : tf);
    int kt = t0;
    for (; kt < tf; ++kt)
        tile_full(kt);
    for (; kt < t1; ++kt)
        tile_masked(kt);
    if (t1 > t0) {
        if (__builtin_amdgcn_ballot_w64(grew) != 0) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    o[dt][ct] *= alpha[ct];
        }
        pv_tile((t1 - 1) & 1);
    }

    // Normalise and write: lane holds O^T[dt*16 + 4*quad + i][column n].
    // With key splits the output is split ksp's fp32 state.
    float *const lse_out = a.lse ? a.lse + ksp * a.split_rows : nullptr;
    void *const out = a.ks > 1 ? static_cast<void *>(static_cast<float *>(a.out) +
                                                     ksp * a.split_rows * D)
                               : a.out;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        float l = lsum[ct];
        l = xsum<16>(l);
        l = xsum<32>(l);
        // (A split's state has S * max_query_len rows: rows past that exist
        // only if a chunk exceeds max_query_len, and are not written.)
        if (!valid[ct] || (a.ks > 1 && qrow[ct] / D >= a.split_rows))
            continue;
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        if (lse_out && quad == 0)
            lse_out[qrow[ct] / D] = l > 0.0f ? m[ct] + __log2f(l) : -INFINITY;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int64_t idx = qrow[ct] + dt * 16 + quad * 4;
            const f32x4 r = o[dt][ct] * inv;
            if (a.out_dtype == PKV_F32) {
                *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + idx) = r;
            } else {
                uint2 pk;
                pk.x = (uint32_t)bf16_rne(r[0]) | ((uint32_t)bf16_rne(r[1]) << 16);
                pk.y = (uint32_t)bf16_rne(r[2]) | ((uint32_t)bf16_rne(r[3]) << 16);
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + idx) = pk;
            }
        }
    }
}

using KernelFn = void (*)(PArgs);

template <int D, int BS>
KernelFn pick_sp_g(int G)
{
    switch (G) {
    case 1: return k_prefill<D, BS, 1>;
    case 2: return k_prefill<D, BS, 2>;
    case 4: return k_prefill<D, BS, 4>;
    case 8: return k_prefill<D, BS, 8>;
    default: return nullptr;
    }
}

KernelFn pick_sp(int D, int BS, int G)
{
    if (D == 64)
        return BS == 16 ? pick_sp_g<64, 16>(G) : pick_sp_g<64, 32>(G);
    return BS == 16 ? pick_sp_g<128, 16>(G) : pick_sp_g<128, 32>(G);
}

}  // namespace

int32_t prefill_rows_per_workgroup() { return ROWS; }

int launch_prefill(const PrefillLaunch &p)
{
    if (p.num_seqs == 0 || p.max_query_len == 0)
        return PKV_OK;
    const int G = p.num_q_heads / p.num_kv_heads;
    KernelFn fn = pick_sp(p.head_dim, p.block_size, G);
    if (!fn)
        return fail(PKV_EUNSUPPORTED, "pkv_prefill_chunk: no kernel for head_dim %d, block %d, "
                    "group %d", p.head_dim, p.block_size, G);
    const int tq = ROWS / G;
    const int64_t nqt = ((int64_t)p.max_query_len + tq - 1) / tq;
    const int ks = p.key_splits < 1 ? 1 : p.key_splits;
    if (nqt * ks > 65535)
        return fail(PKV_EINVAL, "pkv_prefill_chunk: max_query_len %d needs %lld q-tiles x %d "
                    "key splits", p.max_query_len, (long long)nqt, ks);
    if (ks > 1 && (p.out_dtype != PKV_F32 || !p.lse || p.split_rows <= 0))
        return fail(PKV_EINVAL, "pkv_prefill_chunk: key splits need fp32 states and lse");
    PArgs a;
    a.q = static_cast<const uint16_t *>(p.q);
    a.qsl = p.query_start;
    a.kc = static_cast<const uint16_t *>(p.k_cache);
    a.vc = static_cast<const uint16_t *>(p.v_cache);
    a.tables = p.block_tables;
    a.lens = p.context_lens;
    a.out = p.out;
    a.stride = p.table_stride;
    a.Hq = p.num_q_heads;
    a.Hkv = p.num_kv_heads;
    a.num_blocks = p.num_blocks;
    a.n_qtiles = (int32_t)nqt;
    a.S = p.num_seqs;
    a.out_dtype = p.out_dtype;
    a.scale_log2 = p.scale * 1.4426950408889634f;
    a.causal = p.causal;
    a.q_shared = p.q_shared;
    a.lse = p.lse;
    a.ks = ks;
    a.split_rows = ks > 1 ? p.split_rows : 0;
    a.syn_rows = p.syn_rows;
    a.syn_nbk = p.syn_nbk;
    a.syn_nb = p.syn_nb;
    hipStream_t st = reinterpret_cast<hipStream_t>(p.stream);
    hipLaunchKernelGGL(fn, dim3(p.num_kv_heads, (unsigned)(nqt * ks), p.num_seqs), dim3(kThreads),
                       0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(PKV_EHIP, "pkv_prefill_chunk: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

#ifdef PKV_DEBUG
uint32_t prefill_debug_take()
{
    uint32_t v = 0, z = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(dbg_word), sizeof v) != hipSuccess ||
        hipMemcpyToSymbol(HIP_SYMBOL(dbg_word), &z, sizeof z) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return v;
}
#endif

}  // namespace pkv
