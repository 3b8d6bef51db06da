// Block-sparse index builder.
//
// Forward lists: one thread per (head, query tile).  The window is a product
// of three axis ranges (shifted inward, or truncated at the border), so
// walking t, then h, then w inside it emits tile ids in ascending order with
// no sorting.  Shifts are shared by the heads or given per head.
// Transposed lists: one wave per (head, key tile); its lanes test 64 query
// tiles' (possibly shifted) windows at a time and a ballot compacts the hits
// in ascending order.  No atomics, so both list sets are deterministic.
#include "common.h"

namespace sta {

constexpr int kHeadsPerLaunch = 64;

struct Windows {
    int w[kHeadsPerLaunch][3];
};

// Window of query tile q; `offsets` already points at this head's shifts.
__device__ inline void tile_window(const Geo &g, const int *win, const int32_t *offsets, bool truncate, int q,
                                   int s[3], int c[3])
{
    const int qt = q / (g.nh * g.nw), qh = (q / g.nw) % g.nh, qw = q % g.nw;
    const int o0 = offsets ? offsets[3 * q + 0] : 0;
    const int o1 = offsets ? offsets[3 * q + 1] : 0;
    const int o2 = offsets ? offsets[3 * q + 2] : 0;
    if (truncate) {
        axis_window_truncated(g.nt, win[0], qt, o0, s[0], c[0]);
        axis_window_truncated(g.nh, win[1], qh, o1, s[1], c[1]);
        axis_window_truncated(g.nw, win[2], qw, o2, s[2], c[2]);
    } else {
        axis_window(g.nt, win[0], qt, o0, s[0], c[0]);
        axis_window(g.nh, win[1], qh, o1, s[1], c[1]);
        axis_window(g.nw, win[2], qw, o2, s[2], c[2]);
    }
}

__device__ inline const int32_t *head_offsets(const int32_t *offsets, bool per_head, int h, int T)
{
    return offsets && per_head ? offsets + (int64_t)h * T * 3 : offsets;
}

__global__ __launch_bounds__(256) void index_fwd_kernel(Geo g, int h0, int nheads, Windows wins,
                                                        const int32_t *__restrict__ offsets, bool per_head,
                                                        bool truncate, int32_t *__restrict__ kv_idx,
                                                        int32_t *__restrict__ kv_cnt, int max_kv)
{
    const int gid = blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= nheads * g.T) return;
    const int hl = gid / g.T, q = gid % g.T, h = h0 + hl;
    int s[3], c[3];
    tile_window(g, wins.w[hl], head_offsets(offsets, per_head, h, g.T), truncate, q, s, c);
    int32_t *row = kv_idx + ((int64_t)h * g.T + q) * max_kv;
    int n = 0;
    for (int a = s[0]; a < s[0] + c[0]; ++a)
        for (int b = s[1]; b < s[1] + c[1]; ++b)
            for (int d = s[2]; d < s[2] + c[2]; ++d)
                if (n < max_kv) row[n++] = (a * g.nh + b) * g.nw + d;
    kv_cnt[(int64_t)h * g.T + q] = n;
    for (int j = n; j < max_kv; ++j) row[j] = -1;
}

// Heads hl0 .. hl0 + nheads - 1 of the launch's window set (h0 + hl globally).
__global__ __launch_bounds__(256) void index_bwd_kernel(Geo g, int h0, int hl0, int nheads, Windows wins,
                                                        const int32_t *__restrict__ offsets, bool per_head,
                                                        bool truncate, int32_t *__restrict__ q_idx,
                                                        int32_t *__restrict__ q_cnt, int max_q)
{
    const int64_t wid = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (wid >= (int64_t)nheads * g.T) return;       // uniform per wave
    const int hl = hl0 + (int)(wid / g.T), k = (int)(wid % g.T), h = h0 + hl;
    const int32_t *hoff = head_offsets(offsets, per_head, h, g.T);
    const int kt = k / (g.nh * g.nw), kh = (k / g.nw) % g.nh, kw = k % g.nw;
    int32_t *row = q_idx + ((int64_t)h * g.T + k) * max_q;
    int n = 0;                                       // hits so far (uniform)
    for (int q0 = 0; q0 < g.T; q0 += 64) {
        const int q = q0 + lane;
        bool in = false;
        if (q < g.T) {
            int s[3], c[3];
            tile_window(g, wins.w[hl], hoff, truncate, q, s, c);
            in = kt >= s[0] && kt < s[0] + c[0] && kh >= s[1] && kh < s[1] + c[1] && kw >= s[2] && kw < s[2] + c[2];
        }
        const uint64_t hits = __ballot(in);
        const int pos = n + __popcll(hits & ((1ull << lane) - 1ull));   // rank among this pass's hits
        if (in && pos < max_q) row[pos] = q;
        n += __popcll(hits);
    }
    n = n < max_q ? n : max_q;
    if (lane == 0) q_cnt[(int64_t)h * g.T + k] = n;
    for (int j = n + lane; j < max_q; j += 64) row[j] = -1;
}

sta_status launch_build_index(const Geo &g, int H, const int32_t *windows, const int32_t *offsets,
                              bool per_head, bool truncate, const sta_index &idx, hipStream_t s)
{
    for (int h0 = 0; h0 < H; h0 += kHeadsPerLaunch) {
        const int nh = H - h0 < kHeadsPerLaunch ? H - h0 : kHeadsPerLaunch;
        Windows w;
        for (int i = 0; i < kHeadsPerLaunch; ++i)
            for (int d = 0; d < 3; ++d)
                w.w[i][d] = i < nh ? windows[3 * (h0 + i) + d] : 1;
        const int threads = nh * g.T;
        const dim3 grid((threads + 255) / 256);
        hipLaunchKernelGGL(index_fwd_kernel, grid, dim3(256), 0, s, g, h0, nh, w, offsets, per_head, truncate,
                           idx.kv_idx, idx.kv_cnt, idx.max_kv);
        sta_status st = check_launch();
        if (st != STA_OK) return st;
        if (idx.q_idx) {
            // one wave per (head, key tile), 4 per workgroup; heads split so
            // that a launch stays below 2^32 work items
            int per = (int)((((int64_t)1 << 32) - 1) / ((int64_t)g.T * 64));
            per = per < 1 ? 1 : per;
            for (int hs = 0; hs < nh; hs += per) {
                const int n = nh - hs < per ? nh - hs : per;
                const dim3 wgrid((unsigned)(((int64_t)n * g.T + 3) / 4));
                hipLaunchKernelGGL(index_bwd_kernel, wgrid, dim3(256), 0, s, g, h0, hs, n, w, offsets, per_head,
                                   truncate, idx.q_idx, idx.q_cnt, idx.max_q);
                if ((st = check_launch()) != STA_OK) return st;
            }
        }
    }
    return STA_OK;
}

}  // namespace sta
