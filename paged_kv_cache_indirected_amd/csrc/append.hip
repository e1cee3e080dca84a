// Slot-mapped KV append ("LLM Inference: KV Cache, Batching & Scheduling",
// section "The KV cache": each step appends the new token's K and V).
//
// Row t of k/v ([T][Hkv][D]) is copied bit for bit into slot s =
// slot_mapping[t] of the caches ([num_blocks][Hkv][block_size][D]): block
// s / block_size, offset s % block_size.  One thread moves one 16-byte chunk
// of K and the matching chunk of V; consecutive threads cover consecutive
// chunks of a row, so both the reads and the writes of a row are coalesced
// 16-byte accesses.  HBM bound: 2 * T * Hkv * D * elem bytes each way.
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ROWC: 16-byte chunks per (token, head) row; BS: block size.  All index
// math is 32-bit; the host guarantees T * Hkv * ROWC and num_blocks * BS fit.
template <int ROWC, int BS>
__global__ __launch_bounds__(kThreads) void k_append(const uint4 *__restrict__ k,
                                                     const uint4 *__restrict__ v,
                                                     const int32_t *__restrict__ slots,
                                                     uint4 *__restrict__ kc, uint4 *__restrict__ vc,
                                                     int32_t total_chunks, int32_t heads,
                                                     int32_t cap_slots)
{
    const int32_t c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= total_chunks)
        return;
    const int32_t row = c / ROWC;          // (t, g) row of the input
    const int32_t ch = c % ROWC;
    const int32_t t = row / heads;
    const int32_t g = row - t * heads;
    // The row loads do not depend on the slot: issue all three together so
    // the copy costs one memory latency, not two in a chain.
    const u32x4 kk = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(k) + c);
    const u32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(v) + c);
    const int32_t s = slots[t];
    asm volatile("" ::"v"(kk), "v"(vv));   // keep the row loads ahead of the branch
    if (s < 0 || s >= cap_slots)           // padding, or outside the cache: not written
        return;
    const int32_t blk = s / BS, off = s % BS;
    const int64_t dst = (((int64_t)blk * heads + g) * BS + off) * ROWC + ch;
    reinterpret_cast<u32x4 *>(kc)[dst] = kk;
    reinterpret_cast<u32x4 *>(vc)[dst] = vv;
}

template <int ROWC>
int launch_rowc(const AppendLaunch &a, int32_t total, hipStream_t st)
{
    const unsigned grid = (unsigned)((total + kThreads - 1) / kThreads);
    const int32_t cap = a.num_blocks * a.block_size;
    auto kp = static_cast<const uint4 *>(a.k);
    auto vp = static_cast<const uint4 *>(a.v);
    auto kc = static_cast<uint4 *>(a.k_cache);
    auto vc = static_cast<uint4 *>(a.v_cache);
    if (a.block_size == 16)
        hipLaunchKernelGGL((k_append<ROWC, 16>), dim3(grid), dim3(kThreads), 0, st, kp, vp,
                           a.slots, kc, vc, total, a.num_kv_heads, cap);
    else
        hipLaunchKernelGGL((k_append<ROWC, 32>), dim3(grid), dim3(kThreads), 0, st, kp, vp,
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
    switch (rowc) {
    case 8: launch_rowc<8>(a, (int32_t)total, st); break;
    case 16: launch_rowc<16>(a, (int32_t)total, st); break;
    case 32: launch_rowc<32>(a, (int32_t)total, st); break;
    default: return fail(PKV_EUNSUPPORTED, "pkv_append: row of %d bytes", rowc * 16);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(PKV_EHIP, "pkv_append: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

}  // namespace pkv
