// Paged decode attention for gfx950 (CDNA4): a work-balanced split pass on
// the matrix cores plus a log-sum-exp merge pass.
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
// Inside a workgroup (one KV head g, one range), 4 waves; for each piece
// (the part of one sequence inside the range) wave w takes blocks w, w+4, ...
// of the piece, each as units of 16 tokens.  Lane l of a wave is
// (quarter g4 = l / 16, column n = l % 16); column n stands for query head
// g*G + n (columns n >= G are idle padding).
//   * Loads.  The cache tile layout makes every 16-byte load of a wave one
//     coalesced run that lands directly in a matrix-core operand: K keeps
//     each token's dims in 16-byte chunks (chunk c of token t at
//     (c * bs + t) * 16 bytes), so load kk gives lane l chunk 4 kk + g4 of
//     token n; V keeps 4 consecutive tokens of one dim together, so a load
//     gives lane l tokens 4 g4 .. 4 g4 + 3 of one or two dims.  Loads go
//     through buffer resources on the (block, head) tile; an id outside the
//     pool gets an empty resource and reads zeros without touching memory.
//     Three register buffers rotate: units e+1 and e+2 are in flight while
//     unit e is computed.
//   * S = K Q^T on MFMA (bf16: v_mfma_f32_16x16x32_bf16, A = the K chunks as
//     loaded, B = the group's q rows, zero for padding columns; fp32:
//     v_mfma_f32_16x16x4_f32).  Lane l gets S for tokens 4 g4 .. 4 g4 + 3 of
//     head n.
//   * Online softmax per head in log2 units: the unit max reduced over the 4
//     quarters (v_permlane16/32_swap), a lazy running max (rescale only when
//     the max grows by more than 2^8), masking by select so NaN poison in
//     unused slots never reaches the result.
//   * O^T += V^T P^T on MFMA: the S layout is already the B-operand layout
//     of P^T, so P never leaves its lane.  bf16: P is split into bf16 high
//     and low parts (two v_mfma_f32_16x16x16_bf16), keeping ~16 significant
//     bits of each weight; fp32: v_mfma_f32_16x16x4_f32 on P as is.
//   * End of a piece: per head the quarters' sums are added, and the 4
//     waves merge through LDS.
//   * Grid (Hkv, W) with the KV head fastest, so workgroups of one KV head
//     land on one XCD and blocks shared between sequences stay in its L2.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_internal.h"

#ifdef PKV_DEBUG
// Device preconditions found violated by this module's kernels (kDbg* bits).
static __device__ uint32_t dbg_word;
#define PKV_DBG_NOTE(bit) atomicOr(&dbg_word, (bit))
#else
#define PKV_DBG_NOTE(bit) ((void)0)
#endif

// Split partials of pkv_decode_noalloc (callers that cannot allocate device
// memory).  Each GPU the library runs on holds its own copy until the
// process ends; in host code the name is only a handle for the symbol
// lookup in decode_noalloc_scratch(), never a device address.
static __device__ __align__(256) unsigned char scratch[PKV_DECODE_NOALLOC_SCRATCH_BYTES];

namespace pkv {
namespace {

constexpr int NW = 4;                 // waves per workgroup
constexpr int kThreads = NW * 64;
constexpr float kLazyMax = 8.0f;      // running-max slack, log2 units
constexpr int kRsrcWord3 = 0x00020000; // raw buffer resource: 32-bit data format, no swizzle
// Cache policy of the K/V tile loads: bit 1 of the buffer load's aux
// operand, the non-temporal hint (nt).  Each tile is read once per call, so
// the streaming hint keeps the tiles from displacing what is reused; the
// Llama-70B-shaped call runs ~10% faster with it than with the default
// policy (sc0 or sc1 alone change nothing).
constexpr int kTilePolicy = 2;
constexpr int kIdChunk = 2 * kThreads; // block-table entries staged in LDS at a time

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

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
    int32_t row_chunks;               // 16-byte chunks per K/V row
    int32_t block_size;
    int32_t head_dim;
    int32_t stride;
    int32_t B, Hq, Hkv, num_blocks;
    int32_t W;                        // workgroups per KV head
    int32_t max_len;                  // context lengths are clamped to this
    int32_t out_dtype;
    float scale_log2;                 // scale * log2(e)
    float *lse;                       // optional [B][Hq]: log2-sum-exp of the scaled scores
    int32_t piece_cost;               // cost of a sequence boundary, in blocks (see cost_at)
};

__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// Workgroup barrier ordering LDS only.  Waves of a workgroup exchange data
// through LDS alone (global stores here are read by later launches), so the
// barrier need not wait for outstanding global stores as __syncthreads()
// does.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int DT, int D, int BS, int G>
struct Shape {
    static constexpr int ES = DT == PKV_F32 ? 4 : 2;   // element bytes
    static constexpr int E = 16 / ES;                  // dims per 16-byte chunk
    static constexpr int LPT = D / E;                  // chunks per K / q row
    static constexpr int NKL = LPT / 4;                // K loads per lane per unit
    static constexpr int NVL = DT == PKV_F32 ? D / 16 : D / 32;   // V loads per lane per unit
    static constexpr int NACC = D / 16;                // O^T accumulator tiles
    static constexpr int NSUB = BS / 16;               // 16-token units per block
    static constexpr int TILE = BS * D * ES;           // bytes of one (block, head) tile
    static constexpr int OSTR = D + 4;                 // LDS row stride of a wave's output
    static_assert(NKL >= 1 && NSUB >= 1 && G <= 16, "shape");
};

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

// Write chunk i (16 bytes) of sequence b's new K (kv = 0) or V (kv = 1) row
// of KV head g into slot nslot of the caches (fused append), in the tile
// layout: K chunk i of token o at (i * bs + o) * 16 bytes, V element (o, d)
// at ((o / 4) * D + d) * 4 + o % 4.
__device__ __forceinline__ void store_new_chunk(const Args &a, int nslot, int g, int kv, int i,
                                                const uint4 &row)
{
    const int bs = a.block_size, D = a.head_dim;
    const int E = D / a.row_chunks, es = 16 / E;
    const int blk = nslot / bs, o = nslot % bs;
    char *tile = static_cast<char *>(kv ? a.vc_w : a.kc_w) +
                 ((int64_t)blk * a.Hkv + g) * ((int64_t)bs * D * es);
    if (kv == 0) {
        *reinterpret_cast<uint4 *>(tile + (i * bs + o) * 16) = row;
        return;
    }
    const uint32_t w[4] = {row.x, row.y, row.z, row.w};
    const int base = (o / 4) * D * 4 + o % 4;
    for (int e = 0; e < E; ++e) {
        const int idx = base + (i * E + e) * 4;
        if (es == 4)
            reinterpret_cast<uint32_t *>(tile)[idx] = w[e];
        else
            reinterpret_cast<uint16_t *>(tile)[idx] = (uint16_t)(w[e / 2] >> (16 * (e & 1)));
    }
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

// A context length clamped to what a table row addresses and to the host's
// bound.
template <int BS>
__device__ __forceinline__ int clamp_raw_len(const Args &a, int L)
{
    const int cap = min(a.stride * BS, a.max_len);
    return L < 0 ? 0 : (L > cap ? cap : L);
}

// Balanced ranges.  Flattened block x of sequence b costs x + pc * b:
// besides its blocks, a workgroup pays a fixed time at every sequence
// boundary in its range (the load pipeline drains and refills, q and block
// ids are staged, the waves merge), measured at 4-6 us on MI355X, the time
// to stream ~144 KiB at one workgroup's share of the bandwidth; pc is that
// in blocks (a sweep of 8 to 256 KiB put the optimum there).  The cost line [0, Ct), Ct = T + pc * B, is cut into W equal
// ranges [floor(Ct w / W), floor(Ct (w+1) / W)), so workgroups whose ranges
// cross more boundaries get fewer blocks.
__device__ __forceinline__ int64_t cost_at(int64_t x, int b, int pc)
{
    return x + (int64_t)pc * b;
}

// Workgroup whose range holds cost c.
__device__ __forceinline__ int owner(int64_t c, int64_t Ct, int W)
{
    return (int)(((c + 1) * W + Ct - 1) / Ct - 1);
}

// Whether the cost range of workgroup w is empty (possible when W exceeds
// Ct); a range between two costs of one sequence is never empty otherwise.
__device__ __forceinline__ bool empty_range(int w, int64_t Ct, int W)
{
    return Ct * w / W == Ct * (w + 1) / W;
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts by 1, 2,
// 4 and 8 (Hillis-Steele within each row of 16), then the totals of the
// rows below added from lanes 15, 31 and 47.
__device__ __forceinline__ int wave_scan(int v, int lane)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(v, 15);
    const int r1 = __builtin_amdgcn_readlane(v, 31);
    const int r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// floor(C * k / W) for 0 <= k <= W < 2^16 and C < 2^31, in 32-bit
// arithmetic: C = q W + r gives q k + floor(r k / W), r k < 2^32.
__device__ __forceinline__ uint32_t cut_at(uint32_t C, uint32_t k, uint32_t W)
{
    const uint32_t q = C / W, r = C % W;
    return q * k + (r * k) / W;
}

// Number of sequences b < B for which pred(b) holds, pred being true on a
// prefix of b: wave ballots, every wave alone (the result is uniform).
template <typename P>
__device__ __forceinline__ int count_prefix(int B, int lane, P pred)
{
    int n = 0;
    for (int base = 0; base < B; base += 64) {
        const int b = base + lane;
        n += __popcll(__ballot(b < B && pred(b)));
    }
    return n;
}

// First flattened block whose cost is >= c (T if none).
__device__ __forceinline__ int block_at_cost(const int32_t *pref, int B, int pc, int64_t c,
                                             int lane)
{
    const int lo = count_prefix(B, lane, [&](int b) { return cost_at(pref[b], b, pc) <= c; }) - 1;
    const int64_t x = pref[lo] + (c - cost_at(pref[lo], lo, pc));
    return (int)(x < pref[lo + 1] ? x : pref[lo + 1]);
}

// One 16-token unit of the split pass: S = K Q^T on MFMA, the online
// softmax update of (o, m, l) in log2 units, O^T += V^T P^T on MFMA.  kr / vr
// hold the unit's K and V chunks as loaded, qr the B operand of the group's
// q rows; pos0 is the position of this lane's first token (4 g4 of the
// unit), `full` says every token of the unit lies inside the context.
template <int DT, int D, int G>
__device__ __forceinline__ void unit_math(const uint4 (&kr)[D / (16 / (DT == PKV_F32 ? 4 : 2)) / 4],
                                          uint4 (&vr)[DT == PKV_F32 ? D / 16 : D / 32],
                                          const uint4 (&qr)[D / (16 / (DT == PKV_F32 ? 4 : 2)) / 4],
                                          f32x4 (&o)[D / 16], float &m, float &l, int pos0,
                                          int L, bool ok, bool full, float scale_log2)
{
    constexpr int NKL = D / (16 / (DT == PKV_F32 ? 4 : 2)) / 4;
    constexpr int NVL = DT == PKV_F32 ? D / 16 : D / 32;
    constexpr int NACC = D / 16;
    // S for tokens 4 g4 .. 4 g4 + 3 of head n.
    f32x4 sacc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < NKL; ++kk) {
        if constexpr (DT == PKV_F32) {
            sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(kr[kk].x), as_f32(qr[kk].x),
                                                        sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(kr[kk].y), as_f32(qr[kk].y),
                                                        sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(kr[kk].z), as_f32(qr[kk].z),
                                                        sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(kr[kk].w), as_f32(qr[kk].w),
                                                        sacc, 0, 0, 0);
        } else {
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, kr[kk]), __builtin_bit_cast(bf16x8, qr[kk]),
                sacc, 0, 0, 0);
        }
    }

    // Scores in log2 units; positions past the context are masked.
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s[i] = sacc[i] * scale_log2;
    if (!full) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s[i] = (ok && pos0 + i < L) ? s[i] : -INFINITY;
    }
    float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mt = xrow<16, true>(mt);
    mt = xrow<32, true>(mt);
    const bool up = mt > m + kLazyMax;
    const float mn = up ? mt : m;
    const float alpha = up ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;
    const bool dead = (mn == -INFINITY);
    float p[4], sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = dead ? 0.0f : __builtin_amdgcn_exp2f(s[i] - mn);
        sum += p[i];
    }
    l = __builtin_fmaf(l, alpha, sum);
    m = mn;
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
        for (int i = 0; i < NACC; ++i)
            o[i] *= alpha;
    }

    // Unused slots past the context end hold arbitrary bits (NaN
    // poison): zero their V so that 0 * NaN never reaches the sum.
    if (!full && ok) {
        const int nv = L - pos0;                     // valid tokens of this quarter
#pragma unroll
        for (int u = 0; u < NVL; ++u) {
            if constexpr (DT == PKV_F32) {
                vr[u].x = nv > 0 ? vr[u].x : 0u;
                vr[u].y = nv > 1 ? vr[u].y : 0u;
                vr[u].z = nv > 2 ? vr[u].z : 0u;
                vr[u].w = nv > 3 ? vr[u].w : 0u;
            } else {
                const uint32_t m01 = (nv > 0 ? 0x0000FFFFu : 0u) | (nv > 1 ? 0xFFFF0000u : 0u);
                const uint32_t m23 = (nv > 2 ? 0x0000FFFFu : 0u) | (nv > 3 ? 0xFFFF0000u : 0u);
                vr[u].x &= m01;
                vr[u].y &= m23;
                vr[u].z &= m01;
                vr[u].w &= m23;
            }
        }
    }

    // O^T += V^T P^T.
    if constexpr (DT == PKV_F32) {
#pragma unroll
        for (int u = 0; u < NVL; ++u) {
            o[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(vr[u].x), p[0], o[u], 0, 0, 0);
            o[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(vr[u].y), p[1], o[u], 0, 0, 0);
            o[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(vr[u].z), p[2], o[u], 0, 0, 0);
            o[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32(vr[u].w), p[3], o[u], 0, 0, 0);
        }
    } else {
        // hi = p truncated to bf16 (its top 16 bits, exact in fp32),
        // lo = bf16(p - hi).
        uint32_t pu[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pu[i] = __builtin_bit_cast(uint32_t, p[i]);
        const uint32_t h01 = __builtin_amdgcn_perm(pu[1], pu[0], 0x07060302u);
        const uint32_t h23 = __builtin_amdgcn_perm(pu[3], pu[2], 0x07060302u);
        const uint32_t l01 = __builtin_bit_cast(uint32_t, __builtin_convertvector(
            f32x2{p[0] - as_f32(pu[0] & 0xFFFF0000u), p[1] - as_f32(pu[1] & 0xFFFF0000u)},
            bf16x2_t));
        const uint32_t l23 = __builtin_bit_cast(uint32_t, __builtin_convertvector(
            f32x2{p[2] - as_f32(pu[2] & 0xFFFF0000u), p[3] - as_f32(pu[3] & 0xFFFF0000u)},
            bf16x2_t));
        const s16x4 phi = __builtin_bit_cast(s16x4, make_uint2(h01, h23));
        const s16x4 plo = __builtin_bit_cast(s16x4, make_uint2(l01, l23));
#pragma unroll
        for (int u = 0; u < NVL; ++u) {
            const s16x4 v0 = __builtin_bit_cast(s16x4, make_uint2(vr[u].x, vr[u].y));
            const s16x4 v1 = __builtin_bit_cast(s16x4, make_uint2(vr[u].z, vr[u].w));
            o[2 * u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, phi, o[2 * u], 0, 0, 0);
            o[2 * u + 1] =
                __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v1, phi, o[2 * u + 1], 0, 0, 0);
            o[2 * u] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, plo, o[2 * u], 0, 0, 0);
            o[2 * u + 1] =
                __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v1, plo, o[2 * u + 1], 0, 0, 0);
        }
    }
}

// fp32 caches at head_dim 128 need more than half the register file for the
// load ring and accumulators: one workgroup per CU (the grid is sized so
// anyway) lets them have it instead of spilling.
template <int DT, int D, int BS, int G>
__global__ __launch_bounds__(kThreads, (DT == PKV_F32 && D == 128) ? 1 : 2) void k_decode(Args a)
{
    using Sh = Shape<DT, D, BS, G>;
    constexpr int LPT = Sh::LPT, NKL = Sh::NKL, NVL = Sh::NVL, NACC = Sh::NACC;
    constexpr int NSUB = Sh::NSUB, TILE = Sh::TILE, OSTR = Sh::OSTR;

    __shared__ int32_t lds_pref[kDecodeMaxSeqs + 1];
    // Each sequence's clamped length and (fused append) slot, read with the
    // lengths at the start: a piece's set-up then needs no global read but
    // its q rows, block ids and new rows, all in flight together.
    __shared__ int32_t lds_len[kDecodeMaxSeqs];
    __shared__ int32_t lds_slot[kDecodeMaxSeqs];
    __shared__ __attribute__((aligned(16))) uint4 lds_q[G * LPT];
    __shared__ __attribute__((aligned(16))) uint4 lds_new[2][LPT];   // fused append: K, V row
    __shared__ int32_t lds_ids[kIdChunk];
    __shared__ int32_t lds_wsum[NW];
    __shared__ float lds_o[NW][G * OSTR];
    __shared__ float lds_m[NW][G];
    __shared__ float lds_l[NW][G];

    const int g = blockIdx.x, wg = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, n = lane & 15;

    // Prefix sums of the per-sequence block counts, and each sequence's
    // clamped length and append slot for the piece set-up (the same in
    // every workgroup); then this workgroup's range [start, end) of the
    // flattened blocks and its first sequence b.  Up to 64 sequences every
    // wave computes them alone, in registers, and writes the whole tables
    // itself, so it reads them back with no barrier (the other waves write
    // the same values).
    int T, b;
    int64_t start, end;
    if (a.B <= 64) {
        // Both loads unconditional (sequence 0 for idle lanes; slots read
        // from the lengths when there is no fused append), so they are in
        // flight together: a load under a condition is waited for alone.
        const int32_t *sp = a.k_new ? a.slots : a.lens;
        const int bi = lane < a.B ? lane : 0;
        const int rl = a.lens[bi], sr = sp[bi];
        const int Lb = lane < a.B ? clamp_raw_len<BS>(a, rl) : 0;
        if (lane < a.B && Lb != rl)
            PKV_DBG_NOTE(kDbgLength);
        const int sl = a.k_new ? sr : -1;
        if (lane < a.B) {
            lds_len[lane] = Lb;
            lds_slot[lane] = sl;
        }
        const int nb = (Lb + BS - 1) / BS;
        const int v = wave_scan(nb, lane);         // pref[lane + 1]
        if (lane < a.B)
            lds_pref[lane + 1] = v;
        if (lane == 0)
            lds_pref[0] = 0;
        // The range, from registers: lane s holds pref[s] (ex) and
        // pref[s + 1] (v) and the cost of its first block (cx).
        const int ex = v - nb;
        const uint32_t cx = (uint32_t)(ex + a.piece_cost * lane);
        T = __builtin_amdgcn_readlane(v, 63);
        const uint32_t Ct = (uint32_t)T + (uint32_t)a.piece_cost * (uint32_t)a.B;
        auto at_cost = [&](uint32_t c) -> int64_t {
            const int lo = __popcll(__ballot(lane < a.B && cx <= c)) - 1;
            const int x = __builtin_amdgcn_readlane(ex, lo) +
                          (int)(c - (uint32_t)__builtin_amdgcn_readlane((int)cx, lo));
            const int p1 = __builtin_amdgcn_readlane(v, lo);
            return x < p1 ? x : p1;
        };
        start = at_cost(cut_at(Ct, wg, a.W));
        end = at_cost(cut_at(Ct, wg + 1, a.W));
        b = __popcll(__ballot(lane < a.B && ex <= start)) - 1;
    } else {
        int carry = 0;
        for (int base = 0; base < a.B; base += kThreads) {
            const int b = base + tid;
            const int32_t *sp = a.k_new ? a.slots : a.lens;
            const int bi = b < a.B ? b : 0;
            const int rl = a.lens[bi], sr = sp[bi];
            const int Lb = b < a.B ? clamp_raw_len<BS>(a, rl) : 0;
            if (b < a.B && Lb != rl)
                PKV_DBG_NOTE(kDbgLength);
            const int sl = a.k_new ? sr : -1;
            if (b < a.B) {
                lds_len[b] = Lb;
                lds_slot[b] = sl;
            }
            int v = (Lb + BS - 1) / BS;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(v, off);
                if (lane >= off)
                    v += t;
            }
            if (lane == 63)
                lds_wsum[w] = v;
            lds_barrier();
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
            lds_barrier();
        }
        if (tid == 0)
            lds_pref[0] = 0;
        lds_barrier();
        T = lds_pref[a.B];
        const int64_t Ct = (int64_t)T + (int64_t)a.piece_cost * a.B;
        start = block_at_cost(lds_pref, a.B, a.piece_cost, Ct * wg / a.W, lane);
        end = block_at_cost(lds_pref, a.B, a.piece_cost, Ct * (wg + 1) / a.W, lane);
        // First sequence with blocks in the range: the last b with
        // pref[b] <= start.
        b = count_prefix(a.B, lane, [&](int s2) { return lds_pref[s2] <= start; }) - 1;
    }
    const int hq0 = g * G;

    if (g == 0 && wg == 0)
        for (int i = tid; i <= a.B; i += kThreads)
            a.ws_pref[i] = lds_pref[i];

    if (start >= end)
        return;
    const int64_t Ct = (int64_t)T + (int64_t)a.piece_cost * a.B;

    const int64_t blk_bytes = (int64_t)a.Hkv * TILE;
    const char *kbase = static_cast<const char *>(a.kc) + (int64_t)g * TILE;
    const char *vbase = static_cast<const char *>(a.vc) + (int64_t)g * TILE;
    // This lane's byte offsets inside a tile: K load kk of unit h, V load u.
    const uint32_t koff = (uint32_t)((g4 * BS + n) * 16);
    const uint32_t voff = DT == PKV_F32 ? (uint32_t)((g4 * D + n) * 16)
                                        : (uint32_t)((g4 * D + 2 * n) * 8);

    int64_t x = start;
    while (x < end) {
        while (lds_pref[b + 1] <= x)
            ++b;
        const int sb = lds_pref[b], se = lds_pref[b + 1];
        const int j0 = (int)(x - sb);
        const int j1 = (int)((end < se ? end : (int64_t)se) - sb);
        const int L = lds_len[b];
        const int nblk = se - sb;
        const int32_t *bt = a.tables + (int64_t)b * a.stride;

        // One round trip brings the group's q rows (G * D elements), the
        // piece's first block ids and, for the fused append, the step's new
        // K/V rows of this KV head and their slot: all loads are issued
        // before any is waited for.  The workgroup holding the sequence's
        // last block keeps the new rows in LDS, so that the attention reads
        // position L-1 from there rather than from the cache; the merge
        // pass writes them to their slot (no workgroup of this pass reads
        // the cache at that slot, and stores here would share the in-order
        // counter with the tile loads or hold the pass's end).
        const int n0 = j1 - j0 < kIdChunk ? j1 - j0 : kIdChunk;
        const bool last_piece = a.k_new && j1 == nblk;
        int32_t nslot = -1;
        {
            static_assert(G * LPT <= kThreads && kIdChunk == 2 * kThreads, "staging shape");
            uint4 qv = make_uint4(0, 0, 0, 0), nv = make_uint4(0, 0, 0, 0);
            int32_t id0 = -1, id1 = -1;
            if (tid < G * LPT)
                qv = static_cast<const uint4 *>(a.q)[((int64_t)b * a.Hq + hq0) * LPT + tid];
            if (tid < n0)
                id0 = bt[j0 + tid];
            if (tid + kThreads < n0)
                id1 = bt[j0 + tid + kThreads];
            if (last_piece) {
                nslot = lds_slot[b];
                if (tid < 2 * LPT)
                    nv = static_cast<const uint4 *>(tid < LPT ? a.k_new : a.v_new)
                        [((int64_t)b * a.Hkv + g) * LPT + tid % LPT];
            }
            if (tid < G * LPT)
                lds_q[tid] = qv;
            if ((tid < n0 && (unsigned)id0 >= (unsigned)a.num_blocks) ||
                (tid + kThreads < n0 && (unsigned)id1 >= (unsigned)a.num_blocks))
                PKV_DBG_NOTE(kDbgBlockId);
            if (tid < n0)
                lds_ids[tid] = id0;
            if (tid + kThreads < n0)
                lds_ids[tid + kThreads] = id1;
            if ((unsigned)nslot < (unsigned)(a.num_blocks * BS) && tid < 2 * LPT)
                lds_new[tid / LPT][tid % LPT] = nv;
        }
        const bool fresh = (unsigned)nslot < (unsigned)(a.num_blocks * BS);
        lds_barrier();

        // This lane's B operand of S = K Q^T: chunk 4 kk + g4 of query head
        // n's row (zero for the padding columns n >= G).
        uint4 qr[NKL];
#pragma unroll
        for (int kk = 0; kk < NKL; ++kk)
            qr[kk] = n < G ? lds_q[n * LPT + 4 * kk + g4] : make_uint4(0, 0, 0, 0);

        f32x4 o[NACC];
#pragma unroll
        for (int i = 0; i < NACC; ++i)
            o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        float m = -INFINITY, l = 0.0f;

        int c0 = j0;                       // first block of the staged id chunk
        auto blk_of = [&](int e) { return c0 + w + (e / NSUB) * NW; };

        // Issue the loads of unit e (16 tokens of one block): NKL K chunks
        // and NVL V chunks per lane, through buffer resources on the block's
        // tile (scalar registers) with this lane's fixed offsets.  Loads past
        // the last unit, or of an id outside the pool, go through an empty
        // resource (zeros, no memory access), so every iteration issues the
        // same loads and the compiler's wait counts stay exact.
        auto issue = [&](int e, int id, uint4 (&kr)[NKL], uint4 (&vr)[NVL]) {
            const bool ok = (unsigned)id < (unsigned)a.num_blocks;
            const int64_t off = (int64_t)(ok ? id : 0) * blk_bytes;
            const int nrec = ok ? TILE : 0;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(kbase + off), 0, nrec, kRsrcWord3);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(vbase + off), 0, nrec, kRsrcWord3);
            const int h = e % NSUB;
#pragma unroll
            for (int kk = 0; kk < NKL; ++kk)
                kr[kk] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(
                               rk, (int)(koff + (uint32_t)((4 * kk * BS + 16 * h) * 16)), 0, kTilePolicy));
#pragma unroll
            for (int u = 0; u < NVL; ++u) {
                const uint32_t c = DT == PKV_F32 ? (uint32_t)((4 * h * D + 16 * u) * 16)
                                                 : (uint32_t)((4 * h * D + 32 * u) * 8);
                vr[u] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(voff + c), 0, kTilePolicy));
            }
        };

        // One unit: S = K Q^T, online softmax update, O^T += V^T P^T.
        auto process = [&](int e, int id, uint4 (&kr)[NKL], uint4 (&vr)[NVL]) {
            const int j = blk_of(e);
            const int ubase = j * BS + 16 * (e % NSUB);     // position of the unit's token 0
            const bool ok = (unsigned)id < (unsigned)a.num_blocks;
            if (fresh && j == nblk - 1 && L - 1 >= ubase && L - 1 < ubase + 16) {
                const int t = L - 1 - ubase;                 // the new row's token in the unit
                if (n == t) {
#pragma unroll
                    for (int kk = 0; kk < NKL; ++kk)
                        kr[kk] = lds_new[0][4 * kk + g4];
                }
                if (g4 == (t >> 2)) {
                    const int ti = t & 3;
#pragma unroll
                    for (int u = 0; u < NVL; ++u) {
                        if constexpr (DT == PKV_F32) {
                            const uint32_t nv = reinterpret_cast<const uint32_t *>(lds_new[1])
                                [16 * u + n];
                            if (ti == 0) vr[u].x = nv;
                            else if (ti == 1) vr[u].y = nv;
                            else if (ti == 2) vr[u].z = nv;
                            else vr[u].w = nv;
                        } else {
                            const uint16_t *nr = reinterpret_cast<const uint16_t *>(lds_new[1]);
                            const uint32_t n0 = nr[32 * u + 2 * n], n1 = nr[32 * u + 2 * n + 1];
                            const int sh = 16 * (ti & 1);
                            const uint32_t keep = ~(0xFFFFu << sh);
                            if (ti < 2) {
                                vr[u].x = (vr[u].x & keep) | (n0 << sh);
                                vr[u].z = (vr[u].z & keep) | (n1 << sh);
                            } else {
                                vr[u].y = (vr[u].y & keep) | (n0 << sh);
                                vr[u].w = (vr[u].w & keep) | (n1 << sh);
                            }
                        }
                    }
                }
            }

            unit_math<DT, D, G>(kr, vr, qr, o, m, l, ubase + 4 * g4, L, ok,
                                ok && (j + 1) * BS <= L, a.scale_log2);
        };

        // Wave w takes blocks j0 + w, j0 + w + NW, ... of the piece, each as
        // NSUB units (e = 0 .. E-1).  Three register buffers rotate: the
        // loads of units e+1 and e+2 are in flight while unit e is computed.
        // The piece's block ids are staged through LDS in chunks, so the
        // loop issues no vector-memory reads besides the K/V tiles: a table
        // read would share the in-order load counter with them and waiting
        // for it would drain the prefetch.
        for (; c0 < j1; c0 += kIdChunk) {
          const int c1 = j1 - c0 < kIdChunk ? j1 : c0 + kIdChunk;
          if (c0 != j0) {                  // the first chunk came with the q rows
              for (int i = tid; i < c1 - c0; i += kThreads) {
                  const int32_t id = bt[c0 + i];
                  if ((unsigned)id >= (unsigned)a.num_blocks)
                      PKV_DBG_NOTE(kDbgBlockId);
                  lds_ids[i] = id;
              }
              lds_barrier();
          }
          if (c0 + w < c1) {
            const int E = ((c1 - c0 - w + NW - 1) / NW) * NSUB;
            auto id_of = [&](int e) {
                const int id = lds_ids[(e < E ? e : E - 1) / NSUB * NW + w];
                return e < E ? id : -1;
            };
            uint4 kA[NKL], vA[NVL], kB[NKL], vB[NVL], kC[NKL], vC[NVL];
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
          lds_barrier();
        }

        // Per head: the sum over the 4 quarters (m is already common to
        // them), then the wave's O^T, m and l to LDS.  Accumulator i holds,
        // in lane (g4, n), rows r = 4 g4 + k of O^T for head n: dim
        // 32 (i / 2) + 2 r + i % 2 (bf16) or 16 i + r (fp32).
        l = xrow<16, false>(l);
        l = xrow<32, false>(l);
        if (n < G) {
#pragma unroll
            for (int i = 0; i < NACC; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int r = 4 * g4 + k;
                    const int d = DT == PKV_F32 ? 16 * i + r : 32 * (i >> 1) + 2 * r + (i & 1);
                    lds_o[w][n * OSTR + d] = o[i][k];
                }
            if (g4 == 0) {
                lds_m[w][n] = m;
                lds_l[w][n] = l;
            }
        }
        lds_barrier();

        // Merge the 4 waves; a sequence held whole by this range is final.
        const bool whole = owner(cost_at(sb, b, a.piece_cost), Ct, a.W) ==
                           owner(cost_at(se - 1, b, a.piece_cost), Ct, a.W);
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
                    O = __builtin_fmaf(lds_o[s2][h * OSTR + d], f, O);
                }
            }
            if (whole) {
                store_out(a.out, a.out_dtype, ((int64_t)b * a.Hq + hq0 + h) * D + d,
                          Ls > 0.0f ? O / Ls : 0.0f);
                if (a.lse && d == 0)
                    a.lse[(int64_t)b * a.Hq + hq0 + h] = Ls > 0.0f ? M + __log2f(Ls) : -INFINITY;
            } else {
                const int64_t pr = ((int64_t)g * (a.W + a.B) + wg + b) * G + h;
                a.ws_o[pr * D + d] = O;
                if (d == 0) {
                    a.ws_ml[pr * 2] = M;
                    a.ws_ml[pr * 2 + 1] = Ls;
                }
            }
        }
        lds_barrier();
        x = sb + j1;
        ++b;
    }
}

// Log-sum-exp merge of the pieces of every (sequence, query head) cut
// between workgroups: M = max_p m_p, L = sum_p l_p 2^(m_p - M),
// out = sum_p o_p 2^(m_p - M) / L, taken in workgroup order over the
// workgroups whose ranges hold blocks of the sequence.  One workgroup per
// (sequence, KV head): a piece's G query heads x D dims are contiguous in
// the workspace, so each thread folds 4 consecutive values (16-byte loads)
// and the grid stays small (the kernel's time follows its workgroup count,
// not its bytes).  Pieces are read 8 (or, past 8 pieces, 16) at a time, all
// loads of a batch in flight together.  Empty sequences get zeros here; sequences held whole by
// one workgroup were written by it.
constexpr int kMergeThreads = 256;

// Folds pieces wf .. wl of (sequence b, KV head g) in workgroup order, NB
// pieces' loads in flight at a time, and writes the normalised output.
template <int D, int NB>
__device__ __forceinline__ void merge_fold(const Args &a, int b, int g, int wf, int wl,
                                           int64_t Ct, bool sparse, int64_t p0, int64_t obase,
                                           int G, int tid)
{
    for (int i4 = tid; i4 < G * D / 4; i4 += kMergeThreads) {
        const int h = (4 * i4) / D, d0 = (4 * i4) % D;
        float M = -INFINITY, Ls = 0.0f, O[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int w0 = wf; w0 <= wl; w0 += NB) {
            float mp[NB], lp[NB];
            f32x4 op[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int w = w0 + k;
                const bool use = w <= wl && !(sparse && empty_range(w, Ct, a.W));
                const int64_t pr = p0 + (int64_t)w * G + h;
                mp[k] = use ? a.ws_ml[pr * 2] : -INFINITY;
                lp[k] = use ? a.ws_ml[pr * 2 + 1] : 0.0f;
                op[k] = use ? *reinterpret_cast<const f32x4 *>(a.ws_o + pr * D + d0)
                            : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            float Mn = M;
#pragma unroll
            for (int k = 0; k < NB; ++k)
                Mn = fmaxf(Mn, mp[k]);
            if (Mn != -INFINITY) {
                const float f0 = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
                Ls *= f0;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    O[e] *= f0;
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const float f = (mp[k] == -INFINITY) ? 0.0f
                                                         : __builtin_amdgcn_exp2f(mp[k] - Mn);
                    Ls = __builtin_fmaf(lp[k], f, Ls);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        O[e] = __builtin_fmaf(op[k][e], f, O[e]);
                }
            }
            M = Mn;
        }
        const int64_t oidx = obase + (int64_t)h * D + d0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            store_out(a.out, a.out_dtype, oidx + e, Ls > 0.0f ? O[e] / Ls : 0.0f);
        if (a.lse && d0 == 0)
            a.lse[(int64_t)b * a.Hq + g * G + h] = Ls > 0.0f ? M + __log2f(Ls) : -INFINITY;
    }
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void k_merge(Args a)
{
    const int b = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
    const int G = a.Hq / a.Hkv;
    const int64_t Ct = (int64_t)a.ws_pref[a.B] + (int64_t)a.piece_cost * a.B;
    const int sb = a.ws_pref[b], se = a.ws_pref[b + 1];
    const int64_t obase = ((int64_t)b * a.Hq + (int64_t)g * G) * D;   // head g*G, dim 0
    // The fused append: sequence b's new K and V rows of KV head g go to
    // their slot here, after the split pass (which read them from k_new /
    // v_new, not from the cache).
    if (a.k_new && tid < 2 * a.row_chunks) {
        const int nslot = a.slots[b];
        if (nslot >= a.num_blocks * a.block_size)         // (negative: padding)
            PKV_DBG_NOTE(kDbgSlot);
        if ((unsigned)nslot < (unsigned)(a.num_blocks * a.block_size)) {
            const int kv = tid / a.row_chunks, i = tid % a.row_chunks;
            const uint4 row = static_cast<const uint4 *>(kv ? a.v_new : a.k_new)
                [((int64_t)b * a.Hkv + g) * a.row_chunks + i];
            store_new_chunk(a, nslot, g, kv, i, row);
        }
    }
    if (se == sb) {
        for (int i = tid; i < G * D; i += kMergeThreads)
            store_out(a.out, a.out_dtype, obase + i, 0.0f);
        if (a.lse && tid < G)
            a.lse[(int64_t)b * a.Hq + g * G + tid] = -INFINITY;
        return;
    }
    const int wf = owner(cost_at(sb, b, a.piece_cost), Ct, a.W);
    const int wl = owner(cost_at(se - 1, b, a.piece_cost), Ct, a.W);
    if (wf == wl)
        return;
    const bool sparse = Ct < a.W;   // only then can a range be empty
    // Piece (w + b) of KV head g holds rows (head h, dim d) at
    // ((g * (W + B) + w + b) * G + h) * D + d.
    const int64_t p0 = ((int64_t)g * (a.W + a.B) + b) * G;
    // Up to 8 pieces (every sequence of a batch of ~one sequence per range)
    // are read in one batch; a sequence cut into more (a small batch spread
    // over all CUs) is read 16 pieces per round trip: one 4096-token
    // sequence, 32 pieces per KV head, 17.2 -> 16.4 us per call.
    if (wl - wf < 8)
        merge_fold<D, 8>(a, b, g, wf, wl, Ct, sparse, p0, obase, G, tid);
    else
        merge_fold<D, 16>(a, b, g, wf, wl, Ct, sparse, p0, obase, G, tid);
}

// Log-sum-exp merge of K attention states of the same rows (each state a
// normalised output and its log2-sum-exp), in state order.  Each thread
// folds 4 consecutive dims of one row (16-byte loads); a 256-thread
// workgroup takes 1024 / D rows.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void k_merge_states(const float *__restrict__ o,
                                                                const float *__restrict__ lse,
                                                                int32_t K, int64_t rows,
                                                                void *out, int32_t out_dtype,
                                                                const int32_t *row_tokens,
                                                                int32_t heads)
{
    constexpr int TPR = D / 4;                       // threads per row
    constexpr int RPW = kMergeThreads / TPR;         // rows per workgroup
    const int64_t r = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
    const int d0 = (threadIdx.x % TPR) * 4;
    if (r >= rows || (row_tokens && r >= (int64_t)row_tokens[0] * heads))
        return;
    // States are read 8 at a time, all loads of a batch in flight together,
    // and folded in state order.
    float M = -INFINITY;
    for (int k0 = 0; k0 < K; k0 += 8) {
        float lk[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            lk[j] = k0 + j < K ? lse[(int64_t)(k0 + j) * rows + r] : -INFINITY;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            M = fmaxf(M, lk[j]);
    }
    float W = 0.0f, O[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (M != -INFINITY) {
        for (int k0 = 0; k0 < K; k0 += 8) {
            float lk[8];
            f32x4 ok[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool use = k0 + j < K;
                const int64_t row = (int64_t)(k0 + j) * rows + r;
                lk[j] = use ? lse[row] : -INFINITY;
                ok[j] = use ? *reinterpret_cast<const f32x4 *>(o + row * D + d0)
                            : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (k0 + j >= K)
                    break;
                const float f = (lk[j] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(lk[j] - M);
                W += f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    O[e] = __builtin_fmaf(ok[j][e], f, O[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        store_out(out, out_dtype, r * D + d0 + e, W > 0.0f ? O[e] / W : 0.0f);
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

int decode_noalloc_scratch(void **ptr)
{
    // The address of the current device's copy of `scratch`, looked up once
    // per device with that device current, then reused.
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void *addr[kMaxDev] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDev) {
        (void)hipGetLastError();
        return fail(PKV_EHIP, "pkv_decode_noalloc: no current device (%s)", hipGetErrorString(e));
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(PKV_EHIP, "pkv_decode_noalloc: scratch lookup on device %d failed: %s",
                        dev, hipGetErrorString(e));
        }
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return PKV_OK;
}

int32_t decode_piece_cost(int32_t block_size, int32_t head_dim, int32_t elem_size)
{
    const int32_t pc = 147456 / (2 * block_size * head_dim * elem_size);
    return pc < 1 ? 1 : pc;
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
        a.head_dim = d.head_dim;
        a.stride = d.table_stride;
        a.B = nb;
        a.Hq = d.num_q_heads;
        a.Hkv = d.num_kv_heads;
        a.num_blocks = d.num_blocks;
        a.W = d.num_splits;
        a.max_len = d.max_context_len;
        a.out_dtype = d.out_dtype;
        a.scale_log2 = d.scale * 1.4426950408889634f;
        a.lse = d.lse ? d.lse + (int64_t)b0 * d.num_q_heads : nullptr;
        a.piece_cost = decode_piece_cost(d.block_size, d.head_dim, esz);
        hipLaunchKernelGGL(fn, dim3(d.num_kv_heads, d.num_splits), dim3(kThreads), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(PKV_EHIP, "pkv_decode: launch failed: %s", hipGetErrorString(e));
        hipLaunchKernelGGL(merge, dim3(nb, d.num_kv_heads), dim3(kMergeThreads), 0, st, a);
        e = hipGetLastError();
        if (e != hipSuccess)
            return fail(PKV_EHIP, "pkv_decode: merge launch failed: %s", hipGetErrorString(e));
    }
    return PKV_OK;
}

int launch_merge_states(const float *o, const float *lse, int32_t k, int64_t rows,
                        int32_t head_dim, void *out, int32_t out_dtype, void *stream,
                        const int32_t *row_tokens, int32_t heads)
{
    if (rows == 0)
        return PKV_OK;
    if (rows > INT32_MAX)
        return fail(PKV_EINVAL, "merge of %lld rows", (long long)rows);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (head_dim == 64)
        hipLaunchKernelGGL(k_merge_states<64>, dim3((unsigned)((rows + 15) / 16)),
                           dim3(kMergeThreads), 0, st, o, lse, k, rows, out, out_dtype,
                           row_tokens, heads);
    else
        hipLaunchKernelGGL(k_merge_states<128>, dim3((unsigned)((rows + 7) / 8)),
                           dim3(kMergeThreads), 0, st, o, lse, k, rows, out, out_dtype,
                           row_tokens, heads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(PKV_EHIP, "state merge launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

#ifdef PKV_DEBUG
uint32_t decode_debug_take()
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
