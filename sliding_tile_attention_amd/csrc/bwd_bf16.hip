// Sliding-tile attention backward, bf16 (placeholder until the MFMA kernels land).
#include "common.h"

namespace sta {

sta_status launch_bwd_bf16(const void *, const void *, const void *, const void *, const float *, const void *,
                           void *, void *, void *, float *, int, int, int, float, const Geo &, const sta_index &,
                           hipStream_t)
{
    return fail(STA_ERR_UNSUPPORTED, "bf16 backward not built yet");
}

}  // namespace sta
