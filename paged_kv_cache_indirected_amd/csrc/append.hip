// Slot-mapped KV append ("LLM Inference: KV Cache, Batching & Scheduling",
// section "The KV cache": each step appends the new token's K and V).
//
// Row t of k/v ([T][Hkv][D]) is copied bit for bit into slot s =
// slot_mapping[t] of the caches: block s / BS, offset o = s % BS, inside
// the tile of KV head g (tiles are [num_blocks][Hkv], BS x D elements each).
// Tile layout: K keeps each token's dims in 16-byte chunks, chunk c of
// token o at (c * BS + o) * 16 bytes; V keeps groups of 4 tokens together
// per dim, element (o, d) at ((o / 4) * D + d) * 4 + o % 4.
//
// One wave takes 4 consecutive input tokens t0 .. t0+3 (t0 a multiple of 4)
// of one KV head.  When their slots are s0 .. s0+3 with s0 a multiple of 4
// (the rows of a prefill chunk or a prompt land so, apart from the chunk's
// ends), the 4 tokens fill whole 4-token V groups and 64-byte K runs: the
// wave writes the group's V as one contiguous run (16 bytes per lane, each
// lane gathering its dims of the 4 rows) and K as 64-byte runs, so the
// stores fill whole cache lines.  Otherwise every row is copied alone: K as
// 16-byte chunks, V element by element with the lanes of a row on
// consecutive dims.  HBM bound: 2 * T * Hkv * D * elem bytes each way.
#include <hip/hip_runtime.h>

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

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// All index math is 32-bit; the host guarantees T * Hkv * ROWC and
// num_blocks * BS fit.
template <int D, int ES, int BS>
__global__ __launch_bounds__(kThreads) void k_append(const char *__restrict__ k,
                                                     const char *__restrict__ v,
                                                     const int32_t *__restrict__ slots,
                                                     char *__restrict__ kc, char *__restrict__ vc,
                                                     int32_t T, int32_t heads, int32_t n_pairs,
                                                     int32_t cap_slots)
{
    constexpr int ROWC = D * ES / 16;                   // 16-byte chunks per row
    constexpr int E = 16 / ES;                          // elements per chunk
    constexpr int ROWB = D * ES;                        // bytes per row
    constexpr int TILE = BS * D * ES;                   // bytes per (block, head) tile
    static_assert(BS % 4 == 0, "V groups of 4 tokens");
    const int lane = threadIdx.x & 63;
    const int pair = blockIdx.x * kWaves + (threadIdx.x >> 6);   // (group, head), head fastest
    if (pair >= n_pairs)
        return;
    const int grp = pair / heads, g = pair - grp * heads;
    const int t0 = 4 * grp;
    const int nrow = T - t0 < 4 ? T - t0 : 4;
    // Slots of the group's rows (lanes 0 .. 3), then wave-uniform copies.
    const int sl = lane < nrow ? slots[t0 + lane] : -1;
    if (sl >= cap_slots)                                 // (negative: padding)
        PKV_DBG_NOTE(kDbgSlot);
    int s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s[i] = __builtin_amdgcn_readlane(sl, i);
    const bool run = nrow == 4 && s[0] >= 0 && s[0] % 4 == 0 && s[0] + 3 < cap_slots &&
                     s[1] == s[0] + 1 && s[2] == s[0] + 2 && s[3] == s[0] + 3;
    const char *kr = k + ((int64_t)t0 * heads + g) * ROWB;   // row i at kr + i * heads * ROWB
    const char *vr = v + ((int64_t)t0 * heads + g) * ROWB;
    const int rstride = heads * ROWB;
    if (run) {
        const int blk = s[0] / BS, o0 = s[0] % BS;
        const int64_t tile = ((int64_t)blk * heads + g) * TILE;
        // K: unit u = (chunk c = u / 4, token i = u % 4), 16 bytes each; four
        // consecutive lanes write one 64-byte run.
#pragma unroll
        for (int u = lane; u < 4 * ROWC; u += 64) {
            const int c = u >> 2, i = u & 3;
            const u32x4 x = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(kr + i * rstride) + c);
            *reinterpret_cast<u32x4 *>(kc + tile + (c * BS + o0 + i) * 16) = x;
        }
        // V: the group's region (D dims x 4 tokens) is one contiguous run of
        // 4 * ROWB bytes starting at element (o0 / 4) * D * 4; unit u holds
        // 16 / (4 * ES) dims of the 4 tokens.
        char *vdst = vc + tile + (int64_t)(o0 / 4) * D * 4 * ES;
#pragma unroll
        for (int u = lane; u < 4 * ROWC; u += 64) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const uint32_t *>(vr + i * rstride) + u);
            u32x4 x;
            if constexpr (ES == 4) {
                x = u32x4{w[0], w[1], w[2], w[3]};              // dim u, tokens 0..3
            } else {
                // dims 2u, 2u+1: word i holds (dim 2u, dim 2u+1) of token i.
                x = u32x4{(w[0] & 0xFFFFu) | (w[1] << 16), (w[2] & 0xFFFFu) | (w[3] << 16),
                          (w[0] >> 16) | (w[1] & 0xFFFF0000u), (w[2] >> 16) | (w[3] & 0xFFFF0000u)};
            }
            *reinterpret_cast<u32x4 *>(vdst + u * 16) = x;
        }
        return;
    }
    // Row by row: unit u = (row i = u / ROWC, chunk c = u % ROWC); V
    // elements c, c + ROWC, ... of the row, so that the lanes of a row write
    // consecutive dims at each store.
    for (int u = lane; u < 4 * ROWC; u += 64) {
        const int i = u / ROWC, c = u % ROWC;
        if (i >= nrow)
            break;
        const int si = s[0] * (i == 0) + s[1] * (i == 1) + s[2] * (i == 2) + s[3] * (i == 3);
        if (si < 0 || si >= cap_slots)           // padding, or outside the cache: not written
            continue;
        const int blk = si / BS, o = si % BS;
        const int64_t tile = ((int64_t)blk * heads + g) * TILE;
        const u32x4 kk = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(kr + i * rstride) + c);
        *reinterpret_cast<u32x4 *>(kc + tile + (c * BS + o) * 16) = kk;
        const int base = (o / 4) * D * 4 + o % 4;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int d = c + e * ROWC;
            const int idx = base + d * 4;
            if constexpr (ES == 4)
                reinterpret_cast<uint32_t *>(vc + tile)[idx] =
                    __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(vr + i * rstride) + d);
            else
                reinterpret_cast<uint16_t *>(vc + tile)[idx] =
                    __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(vr + i * rstride) + d);
        }
    }
}

template <int D, int ES>
int launch_shape(const AppendLaunch &a, hipStream_t st)
{
    const int32_t n_pairs = (a.num_tokens + 3) / 4 * a.num_kv_heads;
    const unsigned grid = (unsigned)((n_pairs + kWaves - 1) / kWaves);
    const int32_t cap = a.num_blocks * a.block_size;
    auto kp = static_cast<const char *>(a.k);
    auto vp = static_cast<const char *>(a.v);
    auto kc = static_cast<char *>(a.k_cache);
    auto vc = static_cast<char *>(a.v_cache);
    if (a.block_size == 16)
        hipLaunchKernelGGL((k_append<D, ES, 16>), dim3(grid), dim3(kThreads), 0, st, kp, vp,
                           a.slots, kc, vc, a.num_tokens, a.num_kv_heads, n_pairs, cap);
    else
        hipLaunchKernelGGL((k_append<D, ES, 32>), dim3(grid), dim3(kThreads), 0, st, kp, vp,
                           a.slots, kc, vc, a.num_tokens, a.num_kv_heads, n_pairs, cap);
    return PKV_OK;
}

}  // namespace

int launch_append(const AppendLaunch &a)
{
    if (a.num_tokens == 0)
        return PKV_OK;
    const int32_t rowc = a.head_dim * a.elem_size / 16;
    const int64_t total = (int64_t)a.num_tokens * a.num_kv_heads * rowc;
    if (total > INT32_MAX || (int64_t)a.num_blocks * a.block_size > INT32_MAX)
        return fail(PKV_EINVAL, "pkv_append: too many tokens or slots for 32-bit indexing");
    hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
    const int key = a.head_dim * 10 + a.elem_size;
    switch (key) {
    case 642: launch_shape<64, 2>(a, st); break;
    case 1282: launch_shape<128, 2>(a, st); break;
    case 644: launch_shape<64, 4>(a, st); break;
    case 1284: launch_shape<128, 4>(a, st); break;
    default:
        return fail(PKV_EUNSUPPORTED, "pkv_append: head_dim %d with %d-byte elements",
                    a.head_dim, a.elem_size);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(PKV_EHIP, "pkv_append: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

#ifdef PKV_DEBUG
uint32_t append_debug_take()
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
