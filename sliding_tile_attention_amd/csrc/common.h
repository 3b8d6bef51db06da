// Internal declarations shared by the libsta HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libsta.h"

namespace sta {

// Geometry in the form the kernels use.  tile order: tile id * L + in-tile
// raster index; tile id raster over (nt, nh, nw).
struct Geo {
    int gt, gh, gw;   // token grid
    int tt, th, tw;   // tile extents
    int nt, nh, nw;   // tiles per axis
    int T;            // number of tiles
    int L;            // tokens per tile
    int64_t N;        // tokens
};

// Window start and count on one axis (window rule of the library header).
__host__ __device__ inline void axis_window(int n, int w, int q, int o, int &s, int &c)
{
    c = w < n ? w : n;
    s = q + o - w / 2;
    s = s < 0 ? 0 : s;
    s = s > n - c ? n - c : s;
}

// Truncating border rule: the shifted centre is clamped into the grid and
// the window [centre - w/2, centre - w/2 + w - 1] is cut at the border.
__host__ __device__ inline void axis_window_truncated(int n, int w, int q, int o, int &s, int &c)
{
    int centre = q + o;
    centre = centre < 0 ? 0 : centre;
    centre = centre > n - 1 ? n - 1 : centre;
    int lo = centre - w / 2, hi = lo + w - 1;
    lo = lo < 0 ? 0 : lo;
    hi = hi > n - 1 ? n - 1 : hi;
    s = lo;
    c = hi - lo + 1;
}

// Error reporting: records a thread-local message and returns the status.
sta_status fail(sta_status s, const char *fmt, ...);

// Largest number of windows holding one key tile on an axis (no shifts).
int axis_max_attendees(int n, int w);

// ---- launchers (one per source file) ----
sta_status launch_reorder(const void *src, void *dst, int64_t outer, int64_t row_bytes,
                          const Geo &g, bool inverse, hipStream_t s);

// windows: [H][3] host array; offsets: [T][3], or [H][T][3] when per_head
sta_status launch_build_index(const Geo &g, int H, const int32_t *windows, const int32_t *offsets,
                              bool per_head, bool truncate, const sta_index &idx, hipStream_t s);

sta_status launch_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                          int B, int H, int D, float scale, const Geo &g, const sta_index &idx,
                          hipStream_t s);
sta_status launch_bwd_f32(const float *q, const float *k, const float *v, const float *o,
                          const float *lse, const float *dout, float *dq, float *dk, float *dv,
                          float *delta, int B, int H, int D, float scale, const Geo &g,
                          const sta_index &idx, int parts, hipStream_t s);

sta_status launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int D, float scale, const Geo &g, const sta_index &idx,
                           hipStream_t s);
sta_status launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                           const float *lse, const void *dout, void *dq, void *dk, void *dv,
                           float *delta, int B, int H, int D, float scale, const Geo &g,
                           const sta_index &idx, int parts, hipStream_t s);

// Stream-ordered device workspace (per-device pool that keeps freed memory
// for reuse); the buffer may be used by work queued on `s` until the
// matching workspace_free on the same stream.
sta_status workspace_alloc(void **p, size_t bytes, hipStream_t s);
sta_status workspace_free(void *p, hipStream_t s);

// A 1-D launch of `blocks` workgroups of `threads` must keep the total
// work-item count of the grid dimension below 2^32.
inline bool grid_fits(int64_t blocks, int threads)
{
    return blocks >= 0 && blocks * (int64_t)threads < ((int64_t)1 << 32);
}

inline sta_status check_launch()
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(STA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
    return STA_OK;
}

// Maps a launch-order block index to a work index so that each of the
// chip's 8 XCDs (which take blocks round-robin) receives a contiguous range
// of the work order, keeping neighbouring work in one XCD's L2.
__device__ inline int xcd_remap(int bid, int total)
{
    constexpr int X = 8;
    int per = total / X, rem = total % X;
    int xcd = bid % X, slot = bid / X;
    return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

}  // namespace sta
