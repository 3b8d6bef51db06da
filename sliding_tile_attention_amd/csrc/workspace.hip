// Stream-ordered device workspace for kernels that need a temporary buffer
// (the bf16 forward's transposed V tiles, the quantized forward's codes, the
// window-shift producer's tile means).  Each device gets one memory pool of
// its own whose release threshold is unlimited: memory freed on a stream
// goes back to the pool, not to the driver, so a steady-state caller that
// repeats a shape allocates from the driver only on its first call.  The
// pool keeps at most the peak of concurrently live workspaces until the
// process ends.
#include <mutex>

#include "common.h"

namespace sta {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
hipMemPool_t g_pool[kMaxDevices];
}  // namespace

static sta_status pool_for(hipStream_t s, hipMemPool_t &pool)
{
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(s, &dev);
    if (e != hipSuccess) return fail(STA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(STA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_pool[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.handleTypes = hipMemHandleTypeNone;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p = nullptr;
        e = hipMemPoolCreate(&p, &props);
        if (e != hipSuccess) return fail(STA_ERR_HIP, "hipMemPoolCreate: %s", hipGetErrorString(e));
        uint64_t keep = UINT64_MAX;
        e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
        if (e != hipSuccess) {
            (void)hipMemPoolDestroy(p);   // the attribute error is the one reported
            return fail(STA_ERR_HIP, "hipMemPoolSetAttribute: %s", hipGetErrorString(e));
        }
        g_pool[dev] = p;
    }
    pool = g_pool[dev];
    return STA_OK;
}

sta_status workspace_alloc(void **p, size_t bytes, hipStream_t s)
{
    *p = nullptr;
    if (bytes == 0) return STA_OK;
    hipMemPool_t pool;
    sta_status st = pool_for(s, pool);
    if (st != STA_OK) return st;
    hipError_t e = hipMallocFromPoolAsync(p, bytes, pool, s);
    if (e != hipSuccess) {
        *p = nullptr;
        return fail(STA_ERR_HIP, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
    }
    return STA_OK;
}

sta_status workspace_free(void *p, hipStream_t s)
{
    if (!p) return STA_OK;
    hipError_t e = hipFreeAsync(p, s);
    if (e != hipSuccess) return fail(STA_ERR_HIP, "hipFreeAsync: %s", hipGetErrorString(e));
    return STA_OK;
}

}  // namespace sta
