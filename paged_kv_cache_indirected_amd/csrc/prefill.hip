// Causal chunked prefill on MFMA (placeholder until the kernel lands).
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace pkv {

int launch_prefill(const PrefillLaunch &)
{
    return fail(PKV_EUNSUPPORTED, "pkv_prefill_chunk: not built in this library");
}

}  // namespace pkv
