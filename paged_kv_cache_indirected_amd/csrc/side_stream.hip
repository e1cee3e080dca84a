// The library's side stream per device, for launches that may run beside
// the caller's stream (fork / join through two events).
#include <hip/hip_runtime.h>

#include <functional>
#include <mutex>

#include "pkv_internal.h"

namespace pkv {

int launch_forked(void *stream, const std::function<int(void *)> &on_main,
                  const std::function<int(void *)> &on_side)
{
    // One side stream (non-blocking, default priority) and two events per
    // device, created on first use with that device current.  The mutex
    // keeps one caller's record / wait / launch sequence whole.
    constexpr int kMaxDev = 64;
    struct Side {
        hipStream_t s;
        hipEvent_t fork, join;
    };
    static std::mutex mu;
    static Side side[kMaxDev] = {};
    static bool made[kMaxDev] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDev) {
        (void)hipGetLastError();
        return fail(PKV_EHIP, "side stream: no current device (%s)", hipGetErrorString(e));
    }
    std::lock_guard<std::mutex> lock(mu);
    Side &sd = side[dev];
    if (!made[dev]) {
        const unsigned ef = hipEventDisableTiming;
        Side n = {};
        if ((e = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&n.fork, ef)) != hipSuccess ||
            (e = hipEventCreateWithFlags(&n.join, ef)) != hipSuccess) {
            // Release whatever was made, so a later call starts afresh.
            if (n.fork)
                (void)hipEventDestroy(n.fork);
            if (n.s)
                (void)hipStreamDestroy(n.s);
            (void)hipGetLastError();
            return fail(PKV_EHIP, "side stream on device %d: %s", dev, hipGetErrorString(e));
        }
        sd = n;
        made[dev] = true;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if ((e = hipEventRecord(sd.fork, st)) != hipSuccess ||
        (e = hipStreamWaitEvent(sd.s, sd.fork, 0)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(PKV_EHIP, "side stream fork: %s", hipGetErrorString(e));
    }
    const int rc_main = on_main(stream);
    const int rc_side = on_side(sd.s);
    // Join whatever was launched, also after an error in one branch.
    if ((e = hipEventRecord(sd.join, sd.s)) != hipSuccess ||
        (e = hipStreamWaitEvent(st, sd.join, 0)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(PKV_EHIP, "side stream join: %s", hipGetErrorString(e));
    }
    return rc_main != PKV_OK ? rc_main : rc_side;
}

}  // namespace pkv
