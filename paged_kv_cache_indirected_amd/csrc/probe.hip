// Measurement probes for the roofline context of the paged-KV kernels (not
// part of the attention path; only the benchmark loads them).
//
//   pkv_probe_stream_read  read n 16-byte chunks once, contiguously: the
//                          achievable HBM read rate of this part.
//   pkv_probe_tile_read    read whole (block, KV head) tiles of K and V
//                          named by a list of tile indices, with the decode
//                          kernel's access shape (each wave a contiguous run
//                          of the list, 16 bytes per lane per load, 4 KiB
//                          contiguous per tile, two tiles in flight): the
//                          achievable rate of the paged gather itself, with
//                          no arithmetic.
//   pkv_probe_copy         copy n 16-byte chunks: a kernel of known traffic
//                          (n * 16 bytes read, n * 16 written) against which
//                          hardware byte counters are scaled.
//   pkv_probe_coissue      matrix-core work beside vector work on one SIMD:
//                          how much of one instruction stream hides under
//                          the other (the prefill's softmax beside its MFMAs).
// Each reader folds what it loads into an XOR kept in one word per
// workgroup so that no load can be dropped.  The readers' loads carry the
// non-temporal hint, as the decode's tile loads do (every byte is read once).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A 16-byte load with the non-temporal hint.
__device__ __forceinline__ uint4 nt_load16(const void *p)
{
    const u32x4 x = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}

__global__ __launch_bounds__(kThreads) void k_stream_read(const uint4 *__restrict__ src, size_t n,
                                                          uint32_t *__restrict__ sink)
{
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * kThreads;
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        const uint4 v = nt_load16(src + i);
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
// Wave v of the grid reads tiles [v * per, (v + 1) * per) of the list, in
// order, as the decode's workgroups read their ranges: 64 tile indices are
// fetched in one load (lane i holds the i-th) and read back with readlane;
// the next 64 are loaded while the current ones are read, so no data load
// waits on an index load; two tiles (both tensors) are in flight at a time,
// 1 KiB per wave load.
__global__ __launch_bounds__(kThreads) void k_tile_read(const char *__restrict__ kc,
                                                        const char *__restrict__ vc,
                                                        const int64_t *__restrict__ tiles,
                                                        int64_t ntiles, int tile_bytes,
                                                        uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
    const int64_t v = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const int64_t per = (ntiles + nwaves - 1) / nwaves;
    const int64_t t0 = v * per;
    const int64_t t1 = t0 + per < ntiles ? t0 + per : ntiles;
    const int runs = tile_bytes / 1024;
    uint32_t acc = 0;
    int64_t next = t0 + lane < t1 ? tiles[t0 + lane] : 0;
    for (int64_t base = t0; base < t1; base += 64) {
        const int nt = (int)(t1 - base < 64 ? t1 - base : 64);
        const int64_t my = next;
        next = base + 64 + lane < t1 ? tiles[base + 64 + lane] : 0;
        const uint32_t lo = (uint32_t)my, hi = (uint32_t)(my >> 32);
        for (int j = 0; j < nt; j += 2) {
            // A pair of tiles, or the last tile alone (the second tile's
            // loads are then skipped).
            const bool pair = j + 1 < nt;
            const int64_t id0 = ((int64_t)__builtin_amdgcn_readlane(hi, j) << 32) |
                                __builtin_amdgcn_readlane(lo, j);
            const int jj = pair ? j + 1 : j;
            const int64_t id1 = ((int64_t)__builtin_amdgcn_readlane(hi, jj) << 32) |
                                __builtin_amdgcn_readlane(lo, jj);
            const char *k0 = kc + id0 * tile_bytes + lane * 16, *v0 = vc + id0 * tile_bytes + lane * 16;
            const char *k1 = kc + id1 * tile_bytes + lane * 16, *v1 = vc + id1 * tile_bytes + lane * 16;
            for (int c = 0; c < runs; c += 4) {
                uint4 r[16];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int cc = c + u < runs ? c + u : runs - 1;
                    r[u] = nt_load16(k0 + cc * 1024);
                    r[4 + u] = nt_load16(v0 + cc * 1024);
                }
                if (pair) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int cc = c + u < runs ? c + u : runs - 1;
                        r[8 + u] = nt_load16(k1 + cc * 1024);
                        r[12 + u] = nt_load16(v1 + cc * 1024);
                    }
                } else {
#pragma unroll
                    for (int u = 8; u < 16; ++u)
                        r[u] = make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < 16; ++u)
                    acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
            }
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

// Waves w and w + 4 of an 8-wave workgroup share a SIMD.  Per iteration an
// MFMA wave issues 8 independent v_mfma_f32_16x16x32_bf16 and an FMA wave 24
// independent fp32 FMAs (96 vector cycles against 128 matrix cycles).
// mode 0: waves 0-3 MFMA, waves 4-7 FMA; 1: the MFMA waves alone; 2: the FMA
// waves alone; 3: waves 0-3 issue both streams, 1 MFMA then 3 FMAs.  Each
// thread writes one word of out, so nothing is dropped.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512, 1) void k_coissue(float *out, int iters, int mode)
{
    const int tid = threadIdx.x;
    const int half = tid >> 8;                       // 0: waves 0-3, 1: waves 4-7
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(tid + i));
        b[i] = (__bf16)(0.002f * (float)i);
    }
    f32x4 c[8];
    float x[8];
    for (int j = 0; j < 8; ++j) {
        c[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        x[j] = 0.5f + 0.01f * (float)(tid + j);
    }
    const float m = 0.999f, ad = 0.001f;
    const bool mfma = half == 0 && mode != 2;
    const bool fma = (half == 1 && mode != 1 && mode != 3) || (half == 0 && mode == 3);
    if (mfma && !fma) {
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
    } else if (fma && !mfma) {
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int r = 0; r < 3; ++r)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    x[j] = __builtin_fmaf(x[j], m, ad);
    } else if (mfma && fma) {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 3; ++r)
                    x[(j + 3 * r) % 8] = __builtin_fmaf(x[(j + 3 * r) % 8], m, ad);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // three vector ops
            }
        }
    }
    float r = 0.0f;
    for (int j = 0; j < 8; ++j)
        r += c[j][0] + c[j][1] + c[j][2] + c[j][3] + x[j];
    out[(size_t)blockIdx.x * 512 + tid] = r;
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

// out must hold grid * 512 floats.  Return 0, -1 on a bad argument, or -5
// on a launch error.
extern "C" int pkv_probe_coissue(void *out, int iters, int mode, int grid, void *stream)
{
    if (!out || iters < 0 || mode < 0 || mode > 3 || grid <= 0)
        return -1;
    hipLaunchKernelGGL(k_coissue, dim3(grid), dim3(512), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<float *>(out), iters, mode);
    return finish();
}
