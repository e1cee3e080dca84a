// Slot-mapped KV append ("LLM Inference: KV Cache, Batching & Scheduling",
// section "The KV cache": each step appends the new token's K and V).
//
// Row t of k/v ([T][Hkv][D]) is copied bit for bit into slot s =
// slot_mapping[t] of the caches: block s / BS, offset o = s % BS, inside
// the tile of KV head g (tiles are [num_blocks][Hkv], BS x D elements each).
// Tile layout: K keeps each token's dims in 16-byte chunks, chunk c of
// token o at (c * BS + o) * 16 bytes; V keeps groups of 4 tokens together
// per dim, element (o, d) at ((o / 4) * D + d) * 4 + o % 4.  Thread c of a
// row moves the row's 16-byte K chunk c (one 16-byte store) and its V
// elements c, c + R, c + 2R, ... (R = 16-byte chunks per row), so that at
// every store the lanes of a row write consecutive dims.  HBM bound:
// 2 * T * Hkv * D * elem bytes each way.
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// All index math is 32-bit; the host guarantees T * Hkv * ROWC and
// num_blocks * BS fit.
template <int D, int ES, int BS>
__global__ __launch_bounds__(kThreads) void k_append(const uint4 *__restrict__ k,
                                                     const char *__restrict__ v,
                                                     const int32_t *__restrict__ slots,
                                                     char *__restrict__ kc, char *__restrict__ vc,
                                                     int32_t total_chunks, int32_t heads,
                                                     int32_t cap_slots)
{
    constexpr int ROWC = D * ES / 16;                   // 16-byte chunks per row
    constexpr int E = 16 / ES;                          // elements per chunk
    constexpr int TILE = BS * D * ES;                   // bytes per (block, head) tile
    const int32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= total_chunks)
        return;
    const int32_t row = i / ROWC;                       // (t, g) row of the input
    const int32_t c = i % ROWC;
    const int32_t t = row / heads;
    const int32_t g = row - t * heads;
    // K: this thread's 16-byte chunk.  V: the row's elements c, c + ROWC,
    // c + 2 ROWC, ... so that the lanes of a row handle consecutive dims at
    // every step (their stores land 8 or 16 bytes apart, in a few runs).
    // The row loads do not depend on the slot: issue them all before it is
    // known, so the copy costs one memory latency, not two in a chain.
    const u32x4 kk = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(k) + i);
    const char *vrow = v + (int64_t)row * D * ES;
    uint32_t vv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if constexpr (ES == 4)
            vv[e] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(vrow) + c + e * ROWC);
        else
            vv[e] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(vrow) + c + e * ROWC);
    }
    const int32_t s = slots[t];
    asm volatile("" ::"v"(kk));            // keep the row loads ahead of the branch
    if (s < 0 || s >= cap_slots)           // padding, or outside the cache: not written
        return;
    const int32_t blk = s / BS, o = s % BS;
    const int64_t tile = ((int64_t)blk * heads + g) * TILE;
    *reinterpret_cast<u32x4 *>(kc + tile + (c * BS + o) * 16) = kk;
    // V element (o, d) of the tile sits at ((o / 4) * D + d) * 4 + o % 4.
    const int base = (o / 4) * D * 4 + o % 4;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int idx = base + (c + e * ROWC) * 4;
        if constexpr (ES == 4)
            reinterpret_cast<uint32_t *>(vc + tile)[idx] = vv[e];
        else
            reinterpret_cast<uint16_t *>(vc + tile)[idx] = (uint16_t)vv[e];
    }
}

template <int D, int ES>
int launch_shape(const AppendLaunch &a, int32_t total, hipStream_t st)
{
    const unsigned grid = (unsigned)((total + kThreads - 1) / kThreads);
    const int32_t cap = a.num_blocks * a.block_size;
    auto kp = static_cast<const uint4 *>(a.k);
    auto vp = static_cast<const char *>(a.v);
    auto kc = static_cast<char *>(a.k_cache);
    auto vc = static_cast<char *>(a.v_cache);
    if (a.block_size == 16)
        hipLaunchKernelGGL((k_append<D, ES, 16>), dim3(grid), dim3(kThreads), 0, st, kp, vp,
                           a.slots, kc, vc, total, a.num_kv_heads, cap);
    else
        hipLaunchKernelGGL((k_append<D, ES, 32>), dim3(grid), dim3(kThreads), 0, st, kp, vp,
                           a.slots, kc, vc, total, a.num_kv_heads, cap);
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
    case 642: launch_shape<64, 2>(a, (int32_t)total, st); break;
    case 1282: launch_shape<128, 2>(a, (int32_t)total, st); break;
    case 644: launch_shape<64, 4>(a, (int32_t)total, st); break;
    case 1284: launch_shape<128, 4>(a, (int32_t)total, st); break;
    default:
        return fail(PKV_EUNSUPPORTED, "pkv_append: head_dim %d with %d-byte elements",
                    a.head_dim, a.elem_size);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(PKV_EHIP, "pkv_append: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

}  // namespace pkv
