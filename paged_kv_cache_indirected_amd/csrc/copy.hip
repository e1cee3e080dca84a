// Block copy between paged caches: copy-on-write of a shared, partially
// filled block (sequences sharing an identical prefix hold the same pages,
// "LLM Inference Engineering" summary, section 2; a writer needs its own
// page first), and moving a sequence's blocks to and from a second cache
// such as a pinned-host swap area.
//
// Pair i copies block src_ids[i] of (src_k, src_v) to block dst_ids[i] of
// (dst_k, dst_v).  A block is one contiguous run of Hkv * BS * D elements
// in each cache (its Hkv tiles back to back, whatever the order inside a
// tile), so a pair is two plain contiguous copies.  Workgroup x takes pair x / (2 * P), tensor
// (x / P) % 2 and piece x % P of kPiece bytes; each thread moves kUnroll
// 16-byte chunks, issuing every load before any store.  The loads carry the
// non-temporal hint (each source byte is read once): 4096 random pairs of
// 64 KiB blocks copy in ~0.085 ms instead of ~0.113 ms with the default
// policy.  The stores keep the default policy: non-temporal stores slowed
// copies into pinned host memory.  HBM bound: 2 * block bytes read and
// written per pair.
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
constexpr int kUnroll = 4;
constexpr int32_t kPiece = kThreads * kUnroll * 16;   // bytes per workgroup

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void k_copy_blocks(
    const char *__restrict__ sk, const char *__restrict__ sv, int32_t src_nb,
    char *__restrict__ dk, char *__restrict__ dv, int32_t dst_nb,
    const int32_t *__restrict__ src_ids, const int32_t *__restrict__ dst_ids,
    int32_t block_bytes, int32_t pieces)
{
    const int32_t x = blockIdx.x;
    const int32_t pair = x / (2 * pieces);
    const int32_t tensor = (x / pieces) & 1;
    const int32_t piece = x % pieces;
    const int32_t s = src_ids[pair], d = dst_ids[pair];
    if (s < 0 || s >= src_nb || d < 0 || d >= dst_nb) {   // outside a cache: pair skipped
        if (threadIdx.x == 0 && (s >= src_nb || d >= dst_nb))   // (negative: padding)
            PKV_DBG_NOTE(kDbgCopyId);
        return;
    }
    const char *src = (tensor ? sv : sk) + (size_t)s * block_bytes;
    char *dst = (tensor ? dv : dk) + (size_t)d * block_bytes;
    const int32_t base = piece * kPiece + threadIdx.x * 16;
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int32_t o = base + u * kThreads * 16;
        if (o < block_bytes)
            r[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + o));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int32_t o = base + u * kThreads * 16;
        if (o < block_bytes)
            *reinterpret_cast<u32x4 *>(dst + o) = r[u];
    }
}

}  // namespace

int launch_copy_blocks(const CopyLaunch &a)
{
    if (a.n == 0)
        return PKV_OK;
    const int32_t pieces = (int32_t)((a.block_bytes + kPiece - 1) / kPiece);
    const int64_t grid = (int64_t)a.n * 2 * pieces;
    if (grid > INT32_MAX)
        return fail(PKV_EINVAL, "pkv_copy_blocks: %d pairs is too many for one launch", a.n);
    hipLaunchKernelGGL(k_copy_blocks, dim3((unsigned)grid), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(a.stream),
                       static_cast<const char *>(a.src_k), static_cast<const char *>(a.src_v),
                       a.src_num_blocks, static_cast<char *>(a.dst_k),
                       static_cast<char *>(a.dst_v), a.dst_num_blocks, a.src_ids, a.dst_ids,
                       (int32_t)a.block_bytes, pieces);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(PKV_EHIP, "pkv_copy_blocks: launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

#ifdef PKV_DEBUG
uint32_t copy_debug_take()
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
