// Debug builds only (PKV_DEBUG): the checks after every call that enqueued
// device work.  Empty in the release build.
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

#ifdef PKV_DEBUG
#include <algorithm>
#include <iterator>
#include <vector>

namespace pkv {

int debug_finish(int rc, void *stream, const char *who)
{
    if (rc != PKV_OK)
        return rc;
    hipError_t e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(PKV_EHIP, "%s: device error: %s", who, hipGetErrorString(e));
    }
    const uint32_t bits =
        append_debug_take() | copy_debug_take() | decode_debug_take() | prefill_debug_take();
    if (bits == 0)
        return PKV_OK;
    return fail(PKV_EINVAL, "%s: device precondition violated:%s%s%s%s", who,
                bits & kDbgBlockId ? " block id outside the pool;" : "",
                bits & kDbgLength ? " context length outside [0, bound] or below its chunk;" : "",
                bits & kDbgSlot ? " append slot beyond the cache;" : "",
                bits & kDbgCopyId ? " copy block id outside its cache;" : "");
}

namespace {

// n int32 ids from device-readable memory (device or pinned host).
int read_ids(const int32_t *p, int64_t n, void *stream, const char *who,
             std::vector<int32_t> &out)
{
    out.resize((size_t)n);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(out.data(), p, (size_t)n * sizeof(int32_t), hipMemcpyDefault, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(PKV_EHIP, "%s: reading the ids back: %s", who, hipGetErrorString(e));
    }
    return PKV_OK;
}

// First value that occurs twice in a sorted list, or -1.
int32_t first_repeat(const std::vector<int32_t> &v)
{
    const auto it = std::adjacent_find(v.begin(), v.end());
    return it == v.end() ? -1 : *it;
}

}  // namespace

int debug_slots(int rc, const int32_t *slots, int64_t n, int64_t cap, void *stream,
                const char *who)
{
    if (rc != PKV_OK || n <= 0)
        return rc;
    std::vector<int32_t> v;
    if ((rc = read_ids(slots, n, stream, who, v)))
        return rc;
    v.erase(std::remove_if(v.begin(), v.end(), [&](int32_t x) { return x < 0 || x >= cap; }),
            v.end());
    std::sort(v.begin(), v.end());
    const int32_t d = first_repeat(v);
    if (d >= 0)
        return fail(PKV_EINVAL, "%s: device precondition violated: append slot %d mapped twice",
                    who, d);
    return PKV_OK;
}

int debug_copy_ids(int rc, const int32_t *src_ids, const int32_t *dst_ids, int64_t n,
                   int64_t src_nb, int64_t dst_nb, bool in_place, void *stream, const char *who)
{
    if (rc != PKV_OK || n <= 0)
        return rc;
    std::vector<int32_t> s, d;
    if ((rc = read_ids(src_ids, n, stream, who, s)) || (rc = read_ids(dst_ids, n, stream, who, d)))
        return rc;
    // Only the pairs copied count (both ids inside their caches).
    std::vector<int32_t> cs, cd;
    for (int64_t i = 0; i < n; ++i)
        if (s[i] >= 0 && s[i] < src_nb && d[i] >= 0 && d[i] < dst_nb) {
            cs.push_back(s[i]);
            cd.push_back(d[i]);
        }
    std::sort(cs.begin(), cs.end());
    std::sort(cd.begin(), cd.end());
    const int32_t twice = first_repeat(cd);
    if (twice >= 0)
        return fail(PKV_EINVAL,
                    "%s: device precondition violated: destination block %d written twice", who,
                    twice);
    if (in_place) {
        std::vector<int32_t> both;
        std::set_intersection(cs.begin(), cs.end(), cd.begin(), cd.end(),
                              std::back_inserter(both));
        if (!both.empty())
            return fail(PKV_EINVAL,
                        "%s: device precondition violated: block %d is both a source and a "
                        "destination of an in-place copy",
                        who, both[0]);
    }
    return PKV_OK;
}

}  // namespace pkv
#endif
