// C-ABI entry points of libsta: argument checks on the host, then dispatch
// to the kernels.  Nothing is launched when a check fails.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace sta {

static thread_local char g_err[512];

sta_status fail(sta_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

int axis_max_attendees(int n, int w)
{
    int best = 0;
    for (int k = 0; k < n; ++k) {
        int cnt = 0;
        for (int q = 0; q < n; ++q) {
            int s, c;
            axis_window(n, w, q, 0, s, c);
            cnt += (k >= s && k < s + c);
        }
        best = cnt > best ? cnt : best;
    }
    return best;
}

// Largest token count / tile count the kernels index with 32-bit ints.
static const int64_t kMaxTokens = (int64_t)1 << 30;
static const int64_t kMaxTiles = (int64_t)1 << 20;
static const int64_t kMaxTileTokens = (int64_t)1 << 16;

// Product of three positive extents, or -1 once it passes `limit` (at most
// 2^30): every partial product stays below 2^61, so nothing overflows.
static int64_t bounded_product(const int v[3], int64_t limit)
{
    int64_t p = 1;
    for (int d = 0; d < 3; ++d) {
        p *= v[d];
        if (p > limit) return -1;
    }
    return p;
}

static sta_status make_geo(const sta_geom *g, Geo &out)
{
    if (!g)
        return fail(STA_ERR_INVALID, "geometry pointer is NULL");
    const int gr[3] = {g->grid.t, g->grid.h, g->grid.w};
    int tl[3] = {g->tile.t, g->tile.h, g->tile.w};
    int n[3];
    bool ragged = false;
    for (int d = 0; d < 3; ++d) {
        if (gr[d] <= 0 || tl[d] <= 0)
            return fail(STA_ERR_INVALID, "grid and tile extents must be positive (axis %d: grid %d tile %d)",
                        d, gr[d], tl[d]);
        // a tile longer than the axis is one tile holding the whole axis,
        // the same tiling as a tile exactly as long as the axis
        tl[d] = tl[d] < gr[d] ? tl[d] : gr[d];
        n[d] = (gr[d] - 1) / tl[d] + 1;
        ragged = ragged || gr[d] % tl[d] != 0;
    }
    const int64_t N = bounded_product(gr, kMaxTokens);
    const int64_t T = bounded_product(n, kMaxTiles);
    const int64_t L = bounded_product(tl, kMaxTileTokens);
    if (N < 0 || T < 0 || L < 0)
        return fail(STA_ERR_UNSUPPORTED,
                    "grid (%d,%d,%d) with tile (%d,%d,%d) too large: at most %lld tokens, %lld tiles, "
                    "%lld tokens per tile", gr[0], gr[1], gr[2], tl[0], tl[1], tl[2], (long long)kMaxTokens,
                    (long long)kMaxTiles, (long long)kMaxTileTokens);
    out.gt = gr[0]; out.gh = gr[1]; out.gw = gr[2];
    out.tt = tl[0]; out.th = tl[1]; out.tw = tl[2];
    out.nt = n[0]; out.nh = n[1]; out.nw = n[2];
    out.T = (int)T;
    out.L = (int)L;
    out.N = N;
    out.ragged = ragged ? 1 : 0;
    out.text = 0;
    out.Tt = 0;
    out.TT = out.T;
    out.S = N;
    out.raster = 0;
    out.rs_step = out.rs_jump = out.rs_16 = out.rs_span = out.rs_pmask = out.rs_lt = out.rs_lp = 0;
    out.rs_per = 1;
    return STA_OK;
}

// Appends the text tokens of the attention options to a geometry.
static sta_status add_text(Geo &g, const sta_attn_opts *opts)
{
    if (!opts || opts->n_text == 0) return STA_OK;
    if (opts->n_text < 0)
        return fail(STA_ERR_INVALID, "n_text must be >= 0 (got %d)", opts->n_text);
    if (g.N + opts->n_text > kMaxTokens)
        return fail(STA_ERR_UNSUPPORTED, "too many tokens: %lld video + %d text",
                    (long long)g.N, opts->n_text);
    g.text = opts->n_text;
    g.Tt = (g.text + g.L - 1) / g.L;
    g.TT = g.T + g.Tt;
    g.S = g.N + g.text;
    return STA_OK;
}

// Sets the row layout of the attention tensors (sta_layout).  Raster order
// needs whole tiles and no text rows; the bf16 kernels also copy 32-row
// blocks of a tile with one per-lane pattern (raster_step) formed with
// shifts, which needs tw | 16, th*tw a power of two (so one of th*tw and 32
// divides the other) and tiles of a multiple of 32 rows.
static sta_status set_layout(Geo &g, int layout, bool bf16)
{
    if (layout != STA_LAYOUT_TILE && layout != STA_LAYOUT_RASTER)
        return fail(STA_ERR_INVALID, "unknown layout %d", layout);
    if (layout == STA_LAYOUT_TILE) return STA_OK;
    if (g.ragged)
        return fail(STA_ERR_UNSUPPORTED, "raster layout needs a grid the tile divides (grid %dx%dx%d, tile %dx%dx%d)",
                    g.gt, g.gh, g.gw, g.tt, g.th, g.tw);
    if (g.text > 0)
        return fail(STA_ERR_UNSUPPORTED, "raster layout takes video rows only (n_text = %d)", g.text);
    const int plane = g.th * g.tw;
    if (bf16 && (16 % g.tw != 0 || (plane & (plane - 1)) != 0 || g.L % 32 != 0))
        return fail(STA_ERR_UNSUPPORTED, "raster layout of bf16 tensors needs tw | 16, th*tw a power of two and "
                    "32 | L (tile %dx%dx%d)", g.tt, g.th, g.tw);
    g.raster = 1;
    const RasterStep rs = raster_steps(g, 32);
    g.rs_step = rs.step;
    g.rs_jump = rs.jump;
    g.rs_per = rs.per;
    g.rs_16 = (int)raster_step(g, 16);
    g.rs_span = (int)raster_step(g, 31) + 1;
    g.rs_pmask = plane > 32 ? plane - 1 : 0;
    g.rs_lt = g.rs_lp = 0;
    while ((1 << g.rs_lt) < g.tw) ++g.rs_lt;
    while ((1 << g.rs_lp) < plane) ++g.rs_lp;
    return STA_OK;
}

static sta_status index_needs(const Geo &g, int H, const sta_dim3 *w, int has_offsets, bool truncate,
                              int32_t &max_kv, int32_t &max_q)
{
    if (H <= 0)
        return fail(STA_ERR_INVALID, "number of heads must be positive (got %d)", H);
    if (!w)
        return fail(STA_ERR_INVALID, "windows pointer is NULL");
    int64_t kv = 0, qq = 0;
    for (int h = 0; h < H; ++h) {
        if (w[h].t < 1 || w[h].h < 1 || w[h].w < 1)
            return fail(STA_ERR_INVALID, "window of head %d must be >= 1 on every axis (%d,%d,%d)",
                        h, w[h].t, w[h].h, w[h].w);
        int64_t c = (int64_t)(w[h].t < g.nt ? w[h].t : g.nt) * (w[h].h < g.nh ? w[h].h : g.nh) *
                    (w[h].w < g.nw ? w[h].w : g.nw);
        kv = c > kv ? c : kv;
        if (!has_offsets) {
            // truncated windows: a key tile lies in the windows of at most
            // min(w, n) query tiles per axis (their centres are within w)
            int64_t a = truncate ? c
                                 : (int64_t)axis_max_attendees(g.nt, w[h].t) * axis_max_attendees(g.nh, w[h].h) *
                                       axis_max_attendees(g.nw, w[h].w);
            qq = a > qq ? a : qq;
        }
    }
    max_kv = (int32_t)kv;
    max_q = has_offsets ? g.T : (int32_t)qq;
    return STA_OK;
}

static sta_status index_options(const sta_index_opts *opts, bool &truncate, bool &per_head)
{
    truncate = per_head = false;
    if (!opts) return STA_OK;
    if (opts->border != STA_BORDER_SHIFT && opts->border != STA_BORDER_TRUNCATE)
        return fail(STA_ERR_INVALID, "unknown border rule %d", opts->border);
    if (opts->per_head_offsets != 0 && opts->per_head_offsets != 1)
        return fail(STA_ERR_INVALID, "per_head_offsets must be 0 or 1 (got %d)", opts->per_head_offsets);
    truncate = opts->border == STA_BORDER_TRUNCATE;
    per_head = opts->per_head_offsets == 1;
    return STA_OK;
}

// An index holds one list set per head (shared by the batch), or one per
// (b, h) for windows shifted per batch item (num_heads == B * H).
static sta_status check_index(const Geo &g, int B, int H, const sta_index *idx, bool need_transposed)
{
    if (!idx)
        return fail(STA_ERR_INVALID, "index pointer is NULL");
    if (idx->num_heads != H && (int64_t)idx->num_heads != (int64_t)B * H)
        return fail(STA_ERR_INVALID, "index has %d list sets, call has %d heads x %d batch items",
                    idx->num_heads, H, B);
    if (idx->num_tiles != g.T)
        return fail(STA_ERR_INVALID, "index has %d tiles, geometry has %d", idx->num_tiles, g.T);
    if (idx->max_kv < 1 || idx->max_kv > g.T || !idx->kv_idx || !idx->kv_cnt)
        return fail(STA_ERR_INVALID, "index forward lists are missing or max_kv=%d is out of range",
                    idx->max_kv);
    if (need_transposed && (idx->max_q < 1 || idx->max_q > g.T || !idx->q_idx || !idx->q_cnt))
        return fail(STA_ERR_INVALID, "backward needs the transposed lists (q_idx, q_cnt, max_q=%d)",
                    idx->max_q);
    return STA_OK;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static sta_status check_attn(const Geo &g, int B, int H, int D, sta_dtype dt, float scale)
{
    if (B <= 0 || H <= 0 || D <= 0)
        return fail(STA_ERR_INVALID, "B, H and D must be positive (B=%d H=%d D=%d)", B, H, D);
    if (dt != STA_BF16 && dt != STA_F32)
        return fail(STA_ERR_INVALID, "unknown dtype %d", (int)dt);
    if (!(scale > 0.0f) || !isfinite(scale))
        return fail(STA_ERR_INVALID, "scale must be positive and finite");
    if (D != 64 && D != 128)
        return fail(STA_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", D);
    if ((int64_t)B * H * g.S * D > ((int64_t)1 << 40))
        return fail(STA_ERR_UNSUPPORTED, "tensor too large");
    if (dt == STA_BF16 && g.L % 16 != 0)
        return fail(STA_ERR_UNSUPPORTED, "bf16 path needs tokens per tile to be a multiple of 16 (L=%d)", g.L);
    return STA_OK;
}

}  // namespace sta

using namespace sta;

// C callers see the ABI enums as plain int-sized enums; the C++ side must
// agree on their size.
static_assert(sizeof(sta_status) == 4 && sizeof(sta_dtype) == 4 && sizeof(sta_border) == 4 &&
                  sizeof(sta_bwd_part) == 4 && sizeof(sta_precision) == 4 && sizeof(sta_layout) == 4,
              "ABI enums are 32-bit");

// Largest candidate count and search region of the window-shift producer.
static const int64_t kMaxShiftCandidates = 4096;
static const int64_t kMaxShiftRegion = 8192;

// Argument checks shared by sta_window_shifts and its allocation-free
// variant: fills the geometry, windows (thread-local [H][3]), radius and the
// largest search region.
static sta_status check_window_shifts(const void *q, const void *k, int32_t B, int32_t H, int32_t D,
                                      sta_dtype dtype, float scale, const sta_geom *g, const sta_dim3 *windows_host,
                                      const sta_dim3 *radius, const sta_shift_opts *opts, int32_t *offsets_dev,
                                      Geo &geo, sta_shift_opts &o, const int32_t *&wins_out, int r[3],
                                      int64_t &region)
{
    sta_status st = make_geo(g, geo);
    if (st != STA_OK) return st;
    o = opts ? *opts : sta_shift_opts{0, 0, 0, 0};
    if (o.border != STA_BORDER_SHIFT && o.border != STA_BORDER_TRUNCATE)
        return fail(STA_ERR_INVALID, "unknown border rule %d", o.border);
    if (o.per_batch != 0 && o.per_batch != 1)
        return fail(STA_ERR_INVALID, "per_batch must be 0 or 1 (got %d)", o.per_batch);
    sta_attn_opts text = {o.n_text, STA_PREC_DEFAULT, STA_LAYOUT_TILE};
    if ((st = add_text(geo, &text)) != STA_OK) return st;
    if ((st = set_layout(geo, o.layout, false)) != STA_OK) return st;
    if (B <= 0 || H <= 0 || D <= 0)
        return fail(STA_ERR_INVALID, "B, H and D must be positive (B=%d H=%d D=%d)", B, H, D);
    if (dtype != STA_BF16 && dtype != STA_F32)
        return fail(STA_ERR_INVALID, "unknown dtype %d", (int)dtype);
    if (!(scale > 0.0f) || !isfinite(scale))
        return fail(STA_ERR_INVALID, "scale must be positive and finite");
    if (!windows_host || !radius)
        return fail(STA_ERR_INVALID, "windows and radius must be non-NULL");
    if (radius->t < 0 || radius->h < 0 || radius->w < 0)
        return fail(STA_ERR_INVALID, "radius must be >= 0 on every axis (%d,%d,%d)", radius->t, radius->h,
                    radius->w);
    if (!q || !k || !offsets_dev)
        return fail(STA_ERR_INVALID, "q, k and offsets must be non-NULL");
    if (!aligned16(q) || !aligned16(k))
        return fail(STA_ERR_INVALID, "q and k must be 16-byte aligned");
    if (D != 64 && D != 128)
        return fail(STA_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", D);
    if ((int64_t)B * H * geo.S * D > ((int64_t)1 << 40))
        return fail(STA_ERR_UNSUPPORTED, "tensor too large");
    const int64_t ncand = (2LL * radius->t + 1) * (2LL * radius->h + 1) * (2LL * radius->w + 1);
    if (ncand > kMaxShiftCandidates)
        return fail(STA_ERR_UNSUPPORTED, "%lld candidate shifts (at most %lld)", (long long)ncand,
                    (long long)kMaxShiftCandidates);
    if (H > 4096)
        return fail(STA_ERR_UNSUPPORTED, "more than 4096 heads");
    static thread_local int32_t wins[3 * 4096];
    const int n[3] = {geo.nt, geo.nh, geo.nw};
    r[0] = radius->t;
    r[1] = radius->h;
    r[2] = radius->w;
    region = 0;
    for (int h = 0; h < H; ++h) {
        const int w[3] = {windows_host[h].t, windows_host[h].h, windows_host[h].w};
        int64_t reg = 1;
        for (int d = 0; d < 3; ++d) {
            if (w[d] < 1)
                return fail(STA_ERR_INVALID, "window of head %d must be >= 1 on every axis (%d,%d,%d)", h, w[0],
                            w[1], w[2]);
            const int64_t span = (int64_t)w[d] + 2LL * r[d];
            reg *= span < n[d] ? span : n[d];
            wins[3 * h + d] = w[d];
        }
        region = reg > region ? reg : region;
    }
    if (region > kMaxShiftRegion)
        return fail(STA_ERR_UNSUPPORTED, "search region of %lld tiles (at most %lld)", (long long)region,
                    (long long)kMaxShiftRegion);
    const int64_t P = o.per_batch ? B : 1;
    if (!grid_fits(2 * P * H * geo.T, 256) || !grid_fits(P * 64 * geo.T, 256))
        return fail(STA_ERR_UNSUPPORTED, "launch too large");
    wins_out = wins;
    return STA_OK;
}

extern "C" {

const char *sta_status_str(sta_status s)
{
    switch (s) {
    case STA_OK: return "STA_OK";
    case STA_ERR_INVALID: return "STA_ERR_INVALID";
    case STA_ERR_UNSUPPORTED: return "STA_ERR_UNSUPPORTED";
    case STA_ERR_HIP: return "STA_ERR_HIP";
    }
    return "STA_ERR_UNKNOWN";
}

const char *sta_last_error(void) { return g_err; }

int32_t sta_version(void) { return 10400; }

sta_status sta_index_dims(const sta_geom *g, int32_t H, const sta_dim3 *windows_host,
                          int32_t has_offsets, int32_t *max_kv, int32_t *max_q)
{
    return sta_index_dims_ex(g, H, windows_host, has_offsets, nullptr, max_kv, max_q);
}

sta_status sta_index_dims_ex(const sta_geom *g, int32_t H, const sta_dim3 *windows_host, int32_t has_offsets,
                             const sta_index_opts *opts, int32_t *max_kv, int32_t *max_q)
{
    Geo geo;
    sta_status st = make_geo(g, geo);
    if (st != STA_OK) return st;
    bool truncate, per_head;
    st = index_options(opts, truncate, per_head);
    if (st != STA_OK) return st;
    int32_t kv, qq;
    st = index_needs(geo, H, windows_host, has_offsets, truncate, kv, qq);
    if (st != STA_OK) return st;
    if (max_kv) *max_kv = kv;
    if (max_q) *max_q = qq;
    return STA_OK;
}

sta_status sta_tile_reorder(const void *src, void *dst, int64_t outer, int64_t row_bytes,
                            const sta_geom *g, int32_t inverse, hipStream_t stream)
{
    return sta_tile_reorder_ex(src, dst, outer, row_bytes, g, inverse, nullptr, stream);
}

sta_status sta_tile_reorder_ex(const void *src, void *dst, int64_t outer, int64_t row_bytes,
                               const sta_geom *g, int32_t inverse, const sta_attn_opts *opts,
                               hipStream_t stream)
{
    Geo geo;
    sta_status st = make_geo(g, geo);
    if (st != STA_OK) return st;
    if ((st = add_text(geo, opts)) != STA_OK) return st;
    if (!src || !dst)
        return fail(STA_ERR_INVALID, "src and dst must be non-NULL");
    if (outer <= 0 || row_bytes <= 0)
        return fail(STA_ERR_INVALID, "outer and row_bytes must be positive");
    if (outer > ((int64_t)1 << 42) || row_bytes > ((int64_t)1 << 42))
        return fail(STA_ERR_UNSUPPORTED, "tensor too large");
    int64_t bytes = outer * geo.S * row_bytes;
    if (bytes / outer / geo.S != row_bytes || bytes > ((int64_t)1 << 42))
        return fail(STA_ERR_UNSUPPORTED, "tensor too large");
    const char *a = (const char *)src, *b = (const char *)dst;
    if (a < b + bytes && b < a + bytes)
        return fail(STA_ERR_INVALID, "src and dst overlap");
    return launch_reorder(src, dst, outer, row_bytes, geo, inverse != 0, stream);
}

sta_status sta_build_index(const sta_geom *g, int32_t H, const sta_dim3 *windows_host,
                           const int32_t *offsets_dev, const sta_index *idx, hipStream_t stream)
{
    return sta_build_index_ex(g, H, windows_host, offsets_dev, nullptr, idx, stream);
}

sta_status sta_build_index_ex(const sta_geom *g, int32_t H, const sta_dim3 *windows_host,
                              const int32_t *offsets_dev, const sta_index_opts *opts, const sta_index *idx,
                              hipStream_t stream)
{
    Geo geo;
    sta_status st = make_geo(g, geo);
    if (st != STA_OK) return st;
    bool truncate, per_head;
    st = index_options(opts, truncate, per_head);
    if (st != STA_OK) return st;
    int32_t kv, qq;
    st = index_needs(geo, H, windows_host, offsets_dev != nullptr, truncate, kv, qq);
    if (st != STA_OK) return st;
    if (!idx)
        return fail(STA_ERR_INVALID, "index pointer is NULL");
    if (idx->num_heads != H || idx->num_tiles != geo.T)
        return fail(STA_ERR_INVALID, "index descriptor is for %d heads x %d tiles, need %d x %d",
                    idx->num_heads, idx->num_tiles, H, geo.T);
    if (!idx->kv_idx || !idx->kv_cnt)
        return fail(STA_ERR_INVALID, "kv_idx and kv_cnt must be allocated");
    if (idx->max_kv < kv)
        return fail(STA_ERR_INVALID, "max_kv=%d is below the %d this geometry needs", idx->max_kv, kv);
    if (idx->q_idx || idx->q_cnt) {
        if (!idx->q_idx || !idx->q_cnt)
            return fail(STA_ERR_INVALID, "q_idx and q_cnt must both be given or both be NULL");
        if (idx->max_q < qq)
            return fail(STA_ERR_INVALID, "max_q=%d is below the %d this geometry needs", idx->max_q, qq);
    }
    int32_t wins[3 * 4096];
    if (H > 4096)
        return fail(STA_ERR_UNSUPPORTED, "more than 4096 heads");
    for (int h = 0; h < H; ++h) {
        wins[3 * h] = windows_host[h].t;
        wins[3 * h + 1] = windows_host[h].h;
        wins[3 * h + 2] = windows_host[h].w;
    }
    return launch_build_index(geo, H, wins, offsets_dev, per_head, truncate, *idx, stream);
}

sta_status sta_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                   int32_t B, int32_t H, int32_t D, sta_dtype dtype, float scale,
                   const sta_geom *g, const sta_index *idx, hipStream_t stream)
{
    return sta_fwd_ex(q, k, v, o, lse, B, H, D, dtype, scale, g, idx, nullptr, stream);
}

sta_status sta_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
                      int32_t B, int32_t H, int32_t D, sta_dtype dtype, float scale,
                      const sta_geom *g, const sta_index *idx, const sta_attn_opts *opts,
                      hipStream_t stream)
{
    Geo geo;
    sta_status st = make_geo(g, geo);
    if (st != STA_OK) return st;
    if ((st = add_text(geo, opts)) != STA_OK) return st;
    const int prec = opts ? opts->precision : STA_PREC_DEFAULT;
    if (prec != STA_PREC_DEFAULT && prec != STA_PREC_FP8)
        return fail(STA_ERR_INVALID, "unknown precision %d", prec);
    if ((st = set_layout(geo, opts ? opts->layout : STA_LAYOUT_TILE, dtype == STA_BF16)) != STA_OK) return st;
    if (prec == STA_PREC_FP8 && dtype != STA_BF16)
        return fail(STA_ERR_UNSUPPORTED, "the FP8 forward takes bf16 tensors");
    if ((st = check_attn(geo, B, H, D, dtype, scale)) != STA_OK) return st;
    if ((st = check_index(geo, B, H, idx, false)) != STA_OK) return st;
    if (!q || !k || !v || !o || !lse)
        return fail(STA_ERR_INVALID, "q, k, v, o and lse must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return fail(STA_ERR_INVALID, "tensor pointers must be 16-byte aligned");
    if (dtype == STA_F32)
        return launch_fwd_f32((const float *)q, (const float *)k, (const float *)v, (float *)o, lse,
                              B, H, D, scale, geo, *idx, stream);
    if (prec == STA_PREC_FP8)
        return launch_fwd_fp8(q, k, v, o, lse, B, H, D, scale, geo, *idx, stream);
    return launch_fwd_bf16(q, k, v, o, lse, B, H, D, scale, geo, *idx, stream);
}

sta_status sta_bwd_parts(const void *q, const void *k, const void *v, const void *o, const float *lse,
                         const void *dout, void *dq, void *dk, void *dv, float *delta_ws,
                         int32_t B, int32_t H, int32_t D, sta_dtype dtype, float scale,
                         const sta_geom *g, const sta_index *idx, int32_t parts, hipStream_t stream)
{
    return sta_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta_ws, B, H, D, dtype, scale, g, idx, parts, nullptr,
                      stream);
}

sta_status sta_bwd_ex(const void *q, const void *k, const void *v, const void *o, const float *lse,
                      const void *dout, void *dq, void *dk, void *dv, float *delta_ws,
                      int32_t B, int32_t H, int32_t D, sta_dtype dtype, float scale,
                      const sta_geom *g, const sta_index *idx, int32_t parts, const sta_attn_opts *opts,
                      hipStream_t stream)
{
    Geo geo;
    sta_status st = make_geo(g, geo);
    if (st != STA_OK) return st;
    if ((st = add_text(geo, opts)) != STA_OK) return st;
    if (opts && opts->precision != STA_PREC_DEFAULT)
        return fail(opts->precision == STA_PREC_FP8 ? STA_ERR_UNSUPPORTED : STA_ERR_INVALID,
                    "the backward runs in the tensors' dtype (precision %d requested)", opts->precision);
    if ((st = set_layout(geo, opts ? opts->layout : STA_LAYOUT_TILE, dtype == STA_BF16)) != STA_OK) return st;
    if ((st = check_attn(geo, B, H, D, dtype, scale)) != STA_OK) return st;
    if (parts < 1 || parts > STA_BWD_ALL)
        return fail(STA_ERR_INVALID, "parts must be a non-empty mask of STA_BWD_DELTA|DKDV|DQ (got %d)", parts);
    if ((st = check_index(geo, B, H, idx, (parts & STA_BWD_DKDV) != 0)) != STA_OK) return st;
    const bool need_do = true, need_o = (parts & STA_BWD_DELTA) != 0;
    const bool need_qkv = (parts & (STA_BWD_DKDV | STA_BWD_DQ)) != 0;
    struct { const void *p; bool need; } ins[] = {{q, need_qkv}, {k, need_qkv}, {v, need_qkv}, {o, need_o},
                                                  {lse, need_qkv}, {dout, need_do}, {delta_ws, true}};
    for (auto &a : ins)
        if (a.need && (!a.p || !aligned16(a.p)))
            return fail(STA_ERR_INVALID, "inputs must be non-NULL and 16-byte aligned");
    struct { void *p; bool need; } outs[] = {{dq, (parts & STA_BWD_DQ) != 0}, {dk, (parts & STA_BWD_DKDV) != 0},
                                             {dv, (parts & STA_BWD_DKDV) != 0}};
    for (auto &a : outs)
        if (a.need && (!a.p || !aligned16(a.p)))
            return fail(STA_ERR_INVALID, "outputs must be non-NULL and 16-byte aligned");
    if (dtype == STA_F32)
        return launch_bwd_f32((const float *)q, (const float *)k, (const float *)v, (const float *)o, lse,
                              (const float *)dout, (float *)dq, (float *)dk, (float *)dv, delta_ws,
                              B, H, D, scale, geo, *idx, parts, stream);
    return launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, delta_ws, B, H, D, scale, geo, *idx, parts, stream);
}

sta_status sta_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dout, void *dq, void *dk, void *dv, float *delta_ws,
                   int32_t B, int32_t H, int32_t D, sta_dtype dtype, float scale,
                   const sta_geom *g, const sta_index *idx, hipStream_t stream)
{
    return sta_bwd_parts(q, k, v, o, lse, dout, dq, dk, dv, delta_ws, B, H, D, dtype, scale, g, idx,
                         STA_BWD_ALL, stream);
}

sta_status sta_window_shifts(const void *q, const void *k, int32_t B, int32_t H, int32_t D, sta_dtype dtype,
                             float scale, const sta_geom *g, const sta_dim3 *windows_host,
                             const sta_dim3 *radius, const sta_shift_opts *opts, int32_t *offsets_dev,
                             hipStream_t stream)
{
    Geo geo;
    sta_shift_opts o;
    const int32_t *wins;
    int r[3];
    int64_t region;
    const sta_status st = check_window_shifts(q, k, B, H, D, dtype, scale, g, windows_host, radius, opts,
                                              offsets_dev, geo, o, wins, r, region);
    if (st != STA_OK) return st;
    return launch_window_shifts(q, k, B, H, D, dtype, scale, geo, wins, r, o.border == STA_BORDER_TRUNCATE,
                                o.per_batch == 1, (int)region, offsets_dev, stream);
}

sta_status sta_window_shifts_noalloc(const void *q, const void *k, int32_t B, int32_t H, int32_t D,
                                     sta_dtype dtype, float scale, const sta_geom *g,
                                     const sta_dim3 *windows_host, const sta_dim3 *radius,
                                     const sta_shift_opts *opts, int32_t *offsets_dev, hipStream_t stream)
{
    Geo geo;
    sta_shift_opts o;
    const int32_t *wins;
    int r[3];
    int64_t region;
    const sta_status st = check_window_shifts(q, k, B, H, D, dtype, scale, g, windows_host, radius, opts,
                                              offsets_dev, geo, o, wins, r, region);
    if (st != STA_OK) return st;
    return launch_window_shifts_scratch(q, k, B, H, D, dtype, scale, geo, wins, r, o.border == STA_BORDER_TRUNCATE,
                                        o.per_batch == 1, (int)region, offsets_dev, stream);
}

}  // extern "C"
