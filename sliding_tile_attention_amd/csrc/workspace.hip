// Stream-ordered device workspace for kernels that need a temporary buffer
// (every attention launch's work plan, with the key-tile order of the
// dK/dV walk; the quantized forward's codes and scales; the window-shift
// producer's tile means).
//
// Each device gets one memory pool of its own whose release threshold is
// unlimited (memory freed on a stream goes back to the pool, not to the
// driver).  On top of it, each stream a call is made on keeps one cached
// buffer, the largest that calls on it have asked for: a later call on the
// same stream takes that buffer again without allocating or freeing
// anything, which is safe because the stream orders the later call's
// kernels after the earlier call's.  Freeing to the pool is avoided on
// purpose: hipFreeAsync returns to the host only once the previous free on
// the device has been reached by the GPU, so a free per call would hold the
// caller's thread one call behind the GPU.  A buffer is replaced (the old
// one freed on its stream) only when a call needs more.  Calls made while
// their stream is being captured into a graph, calls on a stream whose
// buffer is in use (by another thread) take pool memory and free it as
// before.  Every call that used a cached buffer records an event on its
// stream, and the next call that takes the buffer makes its stream wait for
// that event: a no-op on the same stream, and the ordering that makes the
// buffer safe when a new stream reuses a destroyed stream's handle.  At
// most kMaxCached streams per device hold a buffer; a further stream takes
// the slot of the one least recently used and frees its buffer on its own
// stream after that event.  Cached buffers are otherwise kept until the
// process ends.
#include <mutex>

#include "common.h"

namespace sta {

namespace {
constexpr int kMaxDevices = 64;
constexpr int kMaxCached = 16;                 // cached streams per device

struct Cached {
    hipStream_t stream;
    void *ptr;
    size_t bytes;
    bool busy;
    unsigned long long used;  // g_clock at the last call
    hipEvent_t last;          // recorded on the stream after each call that used ptr
};

std::mutex g_mu;
hipMemPool_t g_pool[kMaxDevices];
Cached g_cache[kMaxDevices][kMaxCached];
int g_ncache[kMaxDevices];
unsigned long long g_clock;
}  // namespace

// Device of stream s and its pool (created on first use).  Called with g_mu held.
static sta_status pool_for(hipStream_t s, int &dev, hipMemPool_t &pool)
{
    hipDevice_t d = 0;
    hipError_t e = hipStreamGetDevice(s, &d);
    if (e != hipSuccess) return fail(STA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (d < 0 || d >= kMaxDevices) return fail(STA_ERR_UNSUPPORTED, "device ordinal %d out of range", d);
    dev = d;
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

static sta_status pool_alloc(void **p, size_t bytes, hipMemPool_t pool, hipStream_t s)
{
    hipError_t e = hipMallocFromPoolAsync(p, bytes, pool, s);
    if (e != hipSuccess) {
        *p = nullptr;
        return fail(STA_ERR_HIP, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
    }
    return STA_OK;
}

sta_status workspace_alloc(void **p, size_t bytes, hipStream_t s)
{
    *p = nullptr;
    if (bytes == 0) return STA_OK;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &cap);
    if (e != hipSuccess) return fail(STA_ERR_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    hipMemPool_t pool;
    sta_status st = pool_for(s, dev, pool);
    if (st != STA_OK) return st;
    // under capture the allocation and its free become graph memory nodes
    if (cap != hipStreamCaptureStatusNone) return pool_alloc(p, bytes, pool, s);
    Cached *c = nullptr;
    for (int i = 0; i < g_ncache[dev]; ++i)
        if (g_cache[dev][i].stream == s) c = &g_cache[dev][i];
    if (!c) {
        // a free slot, else the least recently used idle one
        Cached *slot = g_ncache[dev] < kMaxCached ? &g_cache[dev][g_ncache[dev]] : nullptr;
        const bool fresh = slot != nullptr;
        for (int i = 0; !fresh && i < kMaxCached; ++i)
            if (!g_cache[dev][i].busy && (!slot || g_cache[dev][i].used < slot->used)) slot = &g_cache[dev][i];
        if (!slot) return pool_alloc(p, bytes, pool, s);
        hipEvent_t ev = fresh ? nullptr : slot->last;
        if (!ev && (e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess)
            return fail(STA_ERR_HIP, "hipEventCreateWithFlags: %s", hipGetErrorString(e));
        if (!fresh && slot->ptr) {
            // the old stream's buffer, freed on this stream after its last use there
            if ((e = hipStreamWaitEvent(s, ev, 0)) != hipSuccess || (e = hipFreeAsync(slot->ptr, s)) != hipSuccess)
                return fail(STA_ERR_HIP, "workspace eviction: %s", hipGetErrorString(e));
        }
        if (fresh) ++g_ncache[dev];
        *slot = Cached{s, nullptr, 0, false, 0, ev};
        c = slot;
    }
    c->used = ++g_clock;
    if (c->busy) return pool_alloc(p, bytes, pool, s);
    // after the buffer's last use (recorded when that call gave it back)
    if (c->ptr && (e = hipStreamWaitEvent(s, c->last, 0)) != hipSuccess)
        return fail(STA_ERR_HIP, "hipStreamWaitEvent: %s", hipGetErrorString(e));
    if (c->bytes < bytes) {
        if (c->ptr) {
            e = hipFreeAsync(c->ptr, s);        // after the stream's earlier users
            c->ptr = nullptr;
            c->bytes = 0;
            if (e != hipSuccess) return fail(STA_ERR_HIP, "hipFreeAsync: %s", hipGetErrorString(e));
        }
        void *q = nullptr;
        if ((st = pool_alloc(&q, bytes, pool, s)) != STA_OK) return st;
        c->ptr = q;
        c->bytes = bytes;
    }
    c->busy = true;
    *p = c->ptr;
    return STA_OK;
}

sta_status workspace_free(void *p, hipStream_t s)
{
    if (!p) return STA_OK;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        for (int d = 0; d < kMaxDevices; ++d)
            for (int i = 0; i < g_ncache[d]; ++i)
                if (g_cache[d][i].ptr == p && g_cache[d][i].busy) {
                    g_cache[d][i].busy = false;    // kept for the stream's next call
                    const hipError_t e = hipEventRecord(g_cache[d][i].last, s);
                    if (e != hipSuccess) return fail(STA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
                    return STA_OK;
                }
    }
    hipError_t e = hipFreeAsync(p, s);
    if (e != hipSuccess) return fail(STA_ERR_HIP, "hipFreeAsync: %s", hipGetErrorString(e));
    return STA_OK;
}

}  // namespace sta
