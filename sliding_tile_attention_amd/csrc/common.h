// Internal declarations shared by the libsta HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libsta.h"

namespace sta {

// Geometry in the form the kernels use.  Tile order: tiles in raster order
// of tile coordinates (nt, nh, nw), each holding its tokens in raster order;
// where the tile does not divide the grid (`ragged`), the last tile of an
// axis is cut by the border and holds only the tokens inside the grid, and
// the next tile starts right after it (compact order, N rows in all).
// Joint text + video sequences: `text` text tokens follow the N video
// tokens of every (b, h) slab (S = N + text rows).  The kernels walk them as
// Tt text pseudo-tiles T .. T+Tt-1 of L rows each (the last one ragged)
// starting at slab row N.
// Raster layout (`raster`, grids the tile divides only): the video rows of
// a slab are in raster token order and a tile's rows are gathered where its
// tokens sit (tile_row); text rows follow them as in tile order.
struct Geo {
    int gt, gh, gw;   // token grid
    int tt, th, tw;   // tile extents
    int nt, nh, nw;   // tiles per axis, ceil(grid / tile)
    int T;            // number of tiles
    int L;            // tokens per whole tile
    int64_t N;        // video tokens
    int ragged;       // some tile is cut by the grid border
    int text;         // text tokens after the video tokens
    int Tt;           // text pseudo-tiles, ceil(text / L)
    int TT;           // T + Tt
    int64_t S;        // rows per (b, h) slab, N + text
    int raster;       // video rows in raster order (whole tiles only)
    // raster layout: walk of 32-row blocks (raster_steps(g, 32)) and the
    // raster distance of row 16 of a tile, as kernel arguments so that the
    // kernels reload them instead of holding registers
    int rs_step, rs_jump, rs_per, rs_16;
    int rs_span;      // rows from a 32-row block's first row to past its last, raster_step(31) + 1
    int rs_pmask;     // th*tw - 1 when th*tw > 32 (a power of two), else 0
    int rs_lt, rs_lp; // log2(tw), log2(th*tw) (powers of two in the bf16 raster layout)
};

// Slab rows [start, start + len) of tile t (a video tile or a text
// pseudo-tile).
struct Span {
    int64_t start;
    int len;
};
__host__ __device__ inline Span tile_span(const Geo &g, int t)
{
    if (t >= g.T) {
        const int j = t - g.T, r = g.text - j * g.L;
        return {g.N + (int64_t)j * g.L, r < g.L ? r : g.L};
    }
    if (!g.ragged) return {(int64_t)t * g.L, g.L};
    const int a = t / (g.nh * g.nw), rem = t - a * (g.nh * g.nw);
    const int b = rem / g.nw, c = rem - b * g.nw;
    const int vt = g.gt - a * g.tt < g.tt ? g.gt - a * g.tt : g.tt;
    const int vh = g.gh - b * g.th < g.th ? g.gh - b * g.th : g.th;
    const int vw = g.gw - c * g.tw < g.tw ? g.gw - c * g.tw : g.tw;
    // tokens of earlier tiles: whole tile planes along t, then earlier rows
    // of tiles in this plane, then earlier tiles in this row
    const int64_t start = (int64_t)a * g.tt * g.gh * g.gw + (int64_t)vt * b * g.th * g.gw +
                          (int64_t)vt * vh * c * g.tw;
    return {start, vt * vh * vw};
}

// Rows of tile t.
__host__ __device__ inline int tile_rows(const Geo &g, int t) { return tile_span(g, t).len; }

// Raster index of the first token of video tile t (whole tiles).
__host__ __device__ inline int64_t raster_base(const Geo &g, int t)
{
    const int a = t / (g.nh * g.nw), b = (t / g.nw) % g.nh, c = t % g.nw;
    return ((int64_t)a * g.tt * g.gh + (int64_t)b * g.th) * g.gw + (int64_t)c * g.tw;
}

// Raster distance of row r of a whole tile from its first token (rows of a
// tile in raster order of its tokens).  For a block of `rows` rows starting
// at a multiple of `rows`, raster_step(k0 + x) = raster_step(k0) +
// raster_step(x) whenever tw divides `rows` and one of th*tw, `rows`
// divides the other: the block is whole rows of one tile plane, or whole
// planes.
__host__ __device__ inline int64_t raster_step(const Geo &g, int r)
{
    const int plane = g.th * g.tw;
    const int i = r / plane, rem = r - i * plane, j = rem / g.tw, l = rem - j * g.tw;
    return ((int64_t)i * g.gh + j) * g.gw + l;
}

// Walk of the raster offsets of consecutive `rows`-row blocks of a whole
// tile (rows a multiple of tw; one of th*tw and rows dividing the other):
// after each block the offset moves by `step`, and after every `per` blocks
// (one tile plane, or the planes a block spans) by `jump` more.  No
// divisions per block.
// (Rows of a slab stay below 2^30, so offsets fit an int.)
struct RasterStep {
    int step, jump, per;
};
__host__ __device__ inline RasterStep raster_steps(const Geo &g, int rows)
{
    const int plane = g.th * g.tw;
    if (rows <= plane) return {(rows / g.tw) * g.gw, (g.gh - g.th) * g.gw, plane / rows};
    return {0, (rows / plane) * g.gh * g.gw, 1};
}

// raster_step when tw and th*tw are powers of two (shifts and masks).
__device__ inline int raster_step_p2(const Geo &g, int r)
{
    const int i = r >> g.rs_lp, j = (r & ((1 << g.rs_lp) - 1)) >> g.rs_lt, l = r & ((1 << g.rs_lt) - 1);
    return (i * g.gh + j) * g.gw + l;
}

// Slab row of row r of tile t whose tile-order span sp is known: raster
// position for a video tile under RASTER, else sp.start + r.
template <bool RASTER>
__device__ inline int64_t slab_row(const Geo &g, int t, const Span &sp, int r)
{
    if constexpr (RASTER)
        if (t < g.T) return raster_base(g, t) + raster_step(g, r);
    return sp.start + r;
}

// Slab row of row r of tile t (a video tile or a text pseudo-tile).
__host__ __device__ inline int64_t tile_row(const Geo &g, int t, int r)
{
    if (!g.raster || t >= g.T) return tile_span(g, t).start + r;
    return raster_base(g, t) + raster_step(g, r);
}

// Tile of entry e of a walk: the cnt tiles of a list (lst, or every video
// tile in order when lst is null), then the text pseudo-tiles.  Token-type-
// aware masking (MOD-DiT README, "Token-Type-Aware Masking"): every query
// attends the text keys, and a text query attends every key.
__host__ __device__ inline int entry_tile(const int32_t *lst, int cnt, int T, int e)
{
    return e < cnt ? (lst ? lst[e] : e) : T + (e - cnt);
}

// Blocks of `step` rows in a walk over the cnt video tiles of a list (lst,
// or every video tile when lst is null) and every text pseudo-tile.
__host__ __device__ inline int walk_blocks(const Geo &g, const int32_t *lst, int cnt, int step)
{
    const int per = (g.L + step - 1) / step;
    int n = cnt * per;
    if (g.ragged) {
        n = 0;
        for (int e = 0; e < cnt; ++e) n += (tile_rows(g, lst ? lst[e] : e) + step - 1) / step;
    }
    if (g.Tt == 0) return n;
    const int last = g.text - (g.Tt - 1) * g.L;
    return n + (g.Tt - 1) * per + (last + step - 1) / step;
}

// Work item of a query- (or key-) stationary kernel: rblocks row blocks of
// every tile of every (b, h); per (b, h) the text pseudo-tiles come first,
// since their walks over every tile are the longest.
__device__ inline void decode_item(int work, int rblocks, const Geo &g, int &bh, int &tile, int &rb)
{
    const int per = g.TT * rblocks;
    bh = work / per;
    const int it = work - bh * per;
    const int t = it / rblocks;
    rb = it - t * rblocks;
    tile = t < g.Tt ? g.T + t : t - g.Tt;
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

__device__ inline int plan_slab(const int *plan, int rank) { return plan[16 + rank]; }

// Video tile at position t of list set h's key-stationary walk: the plan's
// tile order if it has one (plan[9] >= 0), else t itself.
__device__ inline int plan_tile(const int *plan, int h, int T, int t)
{
    const int at = plan[9];
    return at < 0 ? t : plan[at + h * T + t];
}

// Blocks of a query- or key-stationary launch of `total` work items: 8
// times twice the mean share of an XCD, room for cost-balanced ranges of up
// to twice the mean item count (plan_work caps them there).
inline int64_t work_blocks(int64_t total) { return 8 * 2 * ((total + 7) / 8); }

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
// text rows after the grid's tokens of every slab are copied unchanged
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
// quantized forward: INT8 QK^T, FP8 (e4m3) PV, bf16 tensors
sta_status launch_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                          int B, int H, int D, float scale, const Geo &g, const sta_index &idx,
                          hipStream_t s);
sta_status launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                           const float *lse, const void *dout, void *dq, void *dk, void *dv,
                           float *delta, int B, int H, int D, float scale, const Geo &g,
                           const sta_index &idx, int parts, hipStream_t s);

// window-shift producer: windows [H][3] host array; offsets [P][H][T][3]
// with P = B per batch item, else 1; region_max bounds the search region's
// tiles of every query tile
sta_status launch_window_shifts(const void *q, const void *k, int B, int H, int D, sta_dtype dtype, float scale,
                                const Geo &g, const int32_t *windows, const int radius[3], bool truncate,
                                bool per_batch, int region_max, int32_t *offsets, hipStream_t s);

// As launch_window_shifts, with the tile means in a static device scratch
// array of fixed size instead of pool workspace (no allocation);
// STA_ERR_UNSUPPORTED when they do not fit.
sta_status launch_window_shifts_scratch(const void *q, const void *k, int B, int H, int D, sta_dtype dtype,
                                        float scale, const Geo &g, const int32_t *windows, const int radius[3],
                                        bool truncate, bool per_batch, int region_max, int32_t *offsets,
                                        hipStream_t s);

// The work plan (schedule.hip) for a launch of `blocks` blocks
// (work_blocks): launches on stream s write, at the start of ws
// (plan_bytes bytes of device workspace, which also hold their scratch),
// the per-XCD cut points of the work order (int[9]) and, 16 ints on, the
// slab of every rank (int[BH]); *split points there.  plan_slab(split, r)
// is the slab (b*H + h) of rank r.  With walk_cnt (the [IH][T] list
// lengths of a key-stationary walk; plan_bytes then takes the geometry)
// the plan also orders each list set's video tiles by descending length,
// read with plan_tile; grids of more than kMaxOrderedTiles tiles keep tile
// order.
constexpr int kMaxOrderedTiles = 4096;
size_t plan_bytes(int IH, int64_t BH, const Geo *tile_order = nullptr);
sta_status plan_work(const Geo &g, const int32_t *kv_cnt, int IH, int64_t BH, int rblocks, int64_t blocks, void *ws,
                     hipStream_t s, const int **split, const int32_t *walk_cnt = nullptr);

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

}  // namespace sta
