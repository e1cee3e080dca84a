// Measurement probes for the roofline context of the paged-KV kernels (not
// part of the attention path; only the benchmark loads them).
//
//   pkv_probe_stream_read  read n 16-byte chunks once, contiguously: the
//                          achievable HBM read rate of this part.
//   pkv_probe_tile_read    read whole (block, KV head) tiles of K and V
//                          named by a list of tile indices, with the decode
//                          kernel's access shape (one wave per tile, 16 bytes
//                          per lane per load, 4 KiB contiguous per tile): the
//                          achievable rate of the paged gather itself, with
//                          no arithmetic.
//   pkv_probe_copy         copy n 16-byte chunks: a kernel of known traffic
//                          (n * 16 bytes read, n * 16 written) against which
//                          hardware byte counters are scaled.
// Each reader folds what it loads into an XOR kept in one word per
// workgroup so that no load can be dropped.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_stream_read(const uint4 *__restrict__ src, size_t n,
                                                          uint32_t *__restrict__ sink)
{
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int i = 0; i < kThreads; ++i)
            r ^= red[i];
        sink[blockIdx.x] = r;
    }
}

// tiles[i] = index of a (block, head) tile of tile_bytes in each of k and v.
// Wave w of workgroup x takes tiles x * 4 + w, x * 4 + w + 4 * grid, ...
__global__ __launch_bounds__(kThreads) void k_tile_read(const char *__restrict__ kc,
                                                        const char *__restrict__ vc,
                                                        const int64_t *__restrict__ tiles,
                                                        int64_t ntiles, int tile_bytes,
                                                        uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t acc = 0;
    const int per = tile_bytes / 1024;
    for (int64_t t = (int64_t)blockIdx.x * 4 + w; t < ntiles; t += (int64_t)gridDim.x * 4) {
        const int64_t base = tiles[t] * tile_bytes + lane * 16;
        for (int c = 0; c < per; ++c) {
            const uint4 a = *reinterpret_cast<const uint4 *>(kc + base + c * 1024);
            const uint4 b = *reinterpret_cast<const uint4 *>(vc + base + c * 1024);
            acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
        }
    }
    __shared__ uint32_t red[kThreads];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int i = 0; i < kThreads; ++i)
            r ^= red[i];
        sink[blockIdx.x] = r;
    }
}

__global__ __launch_bounds__(kThreads) void k_copy(const uint4 *__restrict__ src,
                                                   uint4 *__restrict__ dst, size_t n)
{
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

int finish()
{
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace

// sink must hold `grid` words.  Return 0, or -5 on a launch error.
extern "C" int pkv_probe_stream_read(const void *src, size_t n16, void *sink, int grid,
                                     void *stream)
{
    hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const uint4 *>(src), n16,
                       static_cast<uint32_t *>(sink));
    return finish();
}

// tile_bytes: a multiple of 1024 (e.g. 4096 for 16 tokens x 128 bf16).
extern "C" int pkv_probe_tile_read(const void *k_cache, const void *v_cache, const int64_t *tiles,
                                   int64_t ntiles, int tile_bytes, void *sink, int grid,
                                   void *stream)
{
    if (tile_bytes <= 0 || tile_bytes % 1024 != 0)
        return -1;
    hipLaunchKernelGGL(k_tile_read, dim3(grid), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const char *>(k_cache),
                       static_cast<const char *>(v_cache), tiles, ntiles, tile_bytes,
                       static_cast<uint32_t *>(sink));
    return finish();
}

extern "C" int pkv_probe_copy(const void *src, void *dst, size_t n16, int grid, void *stream)
{
    hipLaunchKernelGGL(k_copy, dim3(grid), dim3(kThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), static_cast<const uint4 *>(src),
                       static_cast<uint4 *>(dst), n16);
    return finish();
}
