// Return-code text and the per-thread detail message of the last failure.
#include <cstdarg>
#include <cstdio>

#include "pkv_internal.h"

namespace {
thread_local char g_msg[512] = "";
}

namespace pkv {

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_msg[0] = '\0'; }

}  // namespace pkv

extern "C" const char *pkv_strerror(int code)
{
    switch (code) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported shape or dtype";
    case PKV_ENOBLOCKS: return "block pool exhausted";
    case PKV_ESTATE: return "invalid bookkeeping state";
    case PKV_EHIP: return "HIP runtime error";
    default: return "unknown error code";
    }
}

extern "C" const char *pkv_last_error(void) { return g_msg; }

extern "C" int pkv_abi_version(void) { return PKV_ABI_VERSION; }
