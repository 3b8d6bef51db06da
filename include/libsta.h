/*
 * libsta -- sliding-tile attention (STA) for AMD Instinct MI355X (gfx950).
 *
 * The operator ("Fast Video Generation with Sliding Tile Attention",
 * abstract): in a video diffusion transformer, 3D full attention over the
 * (T,H,W) latent token grid is replaced by attention restricted to a local
 * 3D window that slides with the query.  STA works at tile granularity: the
 * grid is cut into (tt,th,tw) tiles, and every query tile attends to the
 * key/value tiles in a window of tiles around it.  Two extensions:
 *   - per-head window sizes;
 *   - an optional integer shift of each query tile's window, standing in
 *     for the motion-adaptive 3D Deformable Slide Attention (3D-DSA) of
 *     "MegaSlide-DiT: Memory-Centric Adaptation and Deformable Local
 *     Attention for Efficient Video Diffusion" (abstract).
 * Joint text + video sequences (the *_ex attention calls): text tokens
 * follow the video tokens; a pair with a text token on either side is
 * always attended (token-type-aware masking, MOD-DiT README mirror,
 * "Token-Type-Aware Masking").
 *
 * Window rule (the pages give none; this is the reading used throughout):
 * on each axis with n tiles and window size w, the window holds
 * c = min(w, n) tiles starting at clamp(q + o - floor(w/2), 0, n - c),
 * where q is the query tile coordinate and o its shift.  Windows are moved
 * inward at the borders, never cut, so every query tile of a head sees the
 * same number of key tiles.
 *
 * Orders (raster = t slowest, w fastest):
 *   raster token r = (t*H + h)*W + w;
 *   tile id        = (t/tt * nh + h/th) * nw + w/tw,  n* = ceil(grid / tile);
 *   tile order     = tiles in tile-id order, each holding its tokens in
 *                    raster order; where the grid is a multiple of the tile
 *                    this is tile id * L + ((t%tt)*th + h%th)*tw + w%tw,
 *                    L = tt*th*tw tokens per tile.
 * Grids the tile does not divide: the last tile of such an axis is cut by
 * the grid border and holds only the tokens inside the grid (fewer than L);
 * the next tile starts right after it, so tile-order tensors keep N rows.
 * The window rule works on the n* tiles per axis unchanged.  (The pages'
 * grids are all multiples of their tiles; cut tiles are this library's
 * reading of the latent grids that are not, such as (30,45,80) with
 * (6,8,8) tiles.)
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never synchronises or prints.  These calls take temporary
 *     device memory: every bf16 attention call (sta_fwd, sta_bwd and their
 *     variants, the quantized forward included) its work plan (how the
 *     work splits over the chip's XCDs: about 4*B*H + 12*I*(TT + 1) bytes
 *     for an index of I list sets and TT tiles and text pseudo-tiles), the
 *     dK/dV stage of the backward also 8 bytes per row (see sta_bwd), the
 *     quantized forward codes and scales (see sta_fwd_ex), and
 *     sta_window_shifts tile means.
 *     They take it stream-ordered: each stream the library is called on
 *     (up to 16 per device) keeps one cached buffer, as large as the
 *     largest request on it, which later calls on that stream take again
 *     without allocating or freeing (a replaced or evicted buffer is freed
 *     with hipFreeAsync after its last use); calls under graph capture and
 *     calls that find the buffer in use take memory from one pool per
 *     device (hipMallocFromPoolAsync) and free it at their end
 *     (hipFreeAsync).  Pool and buffers are created on first use and kept
 *     until the process ends; a failed allocation returns STA_ERR_HIP
 *     before anything is launched.
 *   - Work is enqueued on the given HIP stream (0 = the null stream) and
 *     is asynchronous: a call returns without waiting for the GPU (a
 *     hipFreeAsync, taken only when a workspace grows or is not cached,
 *     can wait for the device's previous free); device faults surface at
 *     the caller's next sync.
 *   - Arguments are checked on the host before anything is launched: on
 *     any error nothing is written.  STA_ERR_INVALID = malformed arguments;
 *     STA_ERR_UNSUPPORTED = well-formed but not implemented (reason in
 *     sta_last_error()); STA_ERR_HIP = a HIP launch error.
 *   - Attention tensors are [B][H][N][D], D fastest, in TILE order
 *     (sta_tile_reorder converts) unless an _ex call asks for raster order
 *     (sta_layout), 16-byte aligned, not aliasing each other.
 *   - An index holds one list set per head, shared by every batch item, or
 *     one per (b, h) for windows shifted per batch item (see sta_index).
 *   - Thread-safe.  Mutable global state: a thread-local error message,
 *     the per-device workspace pools and the per-stream cached buffers,
 *     guarded by a mutex (a buffer in use by one call is not handed to
 *     another: concurrent calls on one stream from two threads take pool
 *     memory), and sta_window_shifts_noalloc's static
 *     device array with its per-device address table (filled under a
 *     mutex; the array is shared by every call on a GPU, see there).
 */
#ifndef LIBSTA_H
#define LIBSTA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums below are int-sized.  In C++ they take int32_t as their fixed
 * underlying type, so any int32 value a C caller passes for one is a valid
 * value of the type, which the argument checks then refuse as unknown. */
#ifdef __cplusplus
#define STA_ENUM enum : int32_t
#else
#define STA_ENUM enum
#endif

typedef STA_ENUM {
    STA_OK = 0,
    STA_ERR_INVALID = 1,
    STA_ERR_UNSUPPORTED = 2,
    STA_ERR_HIP = 3
} sta_status;

typedef STA_ENUM {
    STA_BF16 = 0,   /* bf16 storage, fp32 accumulation (MFMA path)        */
    STA_F32 = 1     /* fp32 storage and arithmetic (small shapes, checks) */
} sta_dtype;

typedef struct { int32_t t, h, w; } sta_dim3;

/* Token grid and tile extents, all positive.  A tile extent larger than the
 * grid's is taken as the grid's (one tile along that axis).  Limits: at most
 * 2^30 tokens, 2^20 tiles and 2^16 tokens per tile (STA_ERR_UNSUPPORTED). */
typedef struct { sta_dim3 grid; sta_dim3 tile; } sta_geom;

/* Block-sparse index.  All four arrays are caller-owned DEVICE memory:
 *   kv_idx [num_heads][num_tiles][max_kv]  key tiles of each query tile,
 *                                          ascending tile id, padded -1
 *   kv_cnt [num_heads][num_tiles]
 *   q_idx  [num_heads][num_tiles][max_q]   query tiles whose window holds
 *                                          each key tile, ascending, pad -1
 *   q_cnt  [num_heads][num_tiles]
 * Size max_kv / max_q with sta_index_dims.  q_idx/q_cnt are only needed by
 * sta_bwd and may be NULL (with max_q = 0) for forward-only use.
 * Attention calls with B batch items and H heads accept num_heads == H (the
 * lists of head h serve every batch item) or num_heads == B*H (list set
 * b*H + h serves (b, h): windows shifted per batch item).  Build the latter
 * with sta_build_index_ex for B*H "heads" (the H windows repeated B times)
 * and per-head offsets laid out [B][H][num_tiles][3]. */
typedef struct {
    int32_t num_heads, num_tiles, max_kv, max_q;
    int32_t *kv_idx, *kv_cnt;
    int32_t *q_idx, *q_cnt;
} sta_index;

/* Name of a status code (static string). */
const char *sta_status_str(sta_status s);

/* Human-readable reason for the last non-OK status returned on the calling
 * thread (static or thread-local storage; empty string if none). */
const char *sta_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t sta_version(void);

/* Border rule of a query tile's key-tile window, per axis. */
typedef STA_ENUM {
    /* The window keeps its size min(w, n) and its start q + o - floor(w/2)
     * is moved inside [0, n - size]: every query tile of a head sees the
     * same number of key tiles (the default). */
    STA_BORDER_SHIFT = 0,
    /* The shifted centre q + o is clamped into [0, n-1] and the window
     * [centre - floor(w/2), centre - floor(w/2) + w - 1] is cut at the grid
     * border: windows at the border are smaller, never empty. */
    STA_BORDER_TRUNCATE = 1
} sta_border;

/* Options of the index.  A NULL pointer means all fields 0 (the defaults). */
typedef struct {
    int32_t border;            /* an sta_border value */
    int32_t per_head_offsets;  /* 0: offsets are [num_tiles][3], shared by the
                                  heads; 1: [H][num_tiles][3], one set per head */
} sta_index_opts;

/*
 * Host-only helper, launches nothing.  For H heads with window sizes
 * windows_host[H] (tiles, each >= 1) returns
 *   *max_kv: the largest list length of any query tile,
 *            max_h prod_d min(w_hd, n_d);
 *   *max_q : a safe capacity for the transposed lists: the exact maximum
 *            when has_offsets == 0, else num_tiles (shifts can pile many
 *            windows onto one key tile).
 * Either output pointer may be NULL.
 */
sta_status sta_index_dims(const sta_geom *g, int32_t H, const sta_dim3 *windows_host,
                          int32_t has_offsets, int32_t *max_kv, int32_t *max_q);

/* sta_index_dims for an index built with options (opts may be NULL).  With
 * STA_BORDER_TRUNCATE and no offsets, *max_q = max_h prod_d min(w_hd, n_d).
 * STA_ERR_INVALID for an unknown border value. */
sta_status sta_index_dims_ex(const sta_geom *g, int32_t H, const sta_dim3 *windows_host,
                             int32_t has_offsets, const sta_index_opts *opts, int32_t *max_kv,
                             int32_t *max_q);

/*
 * Token permutation between raster order and tile order (the order the
 * attention kernels read), for `outer` independent slabs of N rows of
 * row_bytes bytes each (N = grid.t*grid.h*grid.w):
 *   inverse == 0:  dst[o][tile_pos(r)] = src[o][r]     (raster -> tile)
 *   inverse != 0:  dst[o][r] = src[o][tile_pos(r)]     (tile -> raster)
 * A pure byte copy (exact for any dtype).  [B][H][N][D] bf16 tensors use
 * outer = B*H, row_bytes = 2*D; [B][N][H][D] tensors use outer = B,
 * row_bytes = 2*H*D; LSE [B][H][N] fp32 uses outer = B*H, row_bytes = 4.
 * src and dst must not overlap.  Any alignment is accepted; 16-byte aligned
 * pointers with row_bytes a multiple of 16 take the 16-byte path.
 * Source of the operation: tiles of the token grid are the unit STA
 * attends over ("Fast Video Generation with Sliding Tile Attention").
 */
sta_status sta_tile_reorder(const void *src, void *dst, int64_t outer, int64_t row_bytes,
                            const sta_geom *g, int32_t inverse, hipStream_t stream);

/*
 * Builds the block-sparse index on the device.
 *   windows_host [H]   window size (tiles) of each head, host memory;
 *   offsets_dev        NULL, or DEVICE int32 [num_tiles][3] window shifts
 *                      (dt,dh,dw) in tiles, one per query tile (tile id
 *                      order), shared by all heads;
 *   idx                caller-filled descriptor: num_heads == H,
 *                      num_tiles == number of tiles, max_kv/max_q at least
 *                      what sta_index_dims returns, device arrays
 *                      allocated.  If q_idx is NULL only the forward lists
 *                      are built.
 * Deterministic: list order is ascending tile id, padding -1.
 * Source: STA's tile windows ("Fast Video Generation with Sliding Tile
 * Attention", abstract); shifted windows for 3D-DSA ("MegaSlide-DiT",
 * abstract).
 */
sta_status sta_build_index(const sta_geom *g, int32_t H, const sta_dim3 *windows_host,
                           const int32_t *offsets_dev, const sta_index *idx, hipStream_t stream);

/*
 * sta_build_index with options (opts may be NULL = sta_build_index):
 *   opts->border            STA_BORDER_SHIFT or STA_BORDER_TRUNCATE;
 *   opts->per_head_offsets  1: offsets_dev is DEVICE int32 [H][num_tiles][3],
 *                           one shift triple per head and query tile.
 * Size the lists with sta_index_dims_ex and the same options.  Attention
 * calls read the lists as built; with truncated windows the list lengths
 * differ between query tiles.
 * Source: motion-adaptive local windows of 3D-DSA ("MegaSlide-DiT",
 * abstract); the pages give no rule for them, so both options are
 * readings and the shifts are inputs.
 */
sta_status sta_build_index_ex(const sta_geom *g, int32_t H, const sta_dim3 *windows_host,
                              const int32_t *offsets_dev, const sta_index_opts *opts, const sta_index *idx,
                              hipStream_t stream);

/*
 * Fused forward.  For every (b, h) and query token i (tile order):
 *   s_ij  = scale * <q_i, k_j>   for keys j in the tiles listed for tile(i)
 *   lse_i = ln sum_j exp(s_ij)                                   (fp32)
 *   o_i   = sum_j exp(s_ij - lse_i) v_j                          (dtype)
 * q, k, v, o: [B][H][N][D] in tile order; lse: [B][H][N] fp32 in tile
 * order.  D must be 64 or 128.  bf16 uses MFMA with fp32 accumulation; the
 * probabilities are rounded to bf16 before the PV product.
 * Workspace: only the work plan (Conventions), a few tens of KB, in
 * `stream`'s cached workspace.  A failed allocation returns STA_ERR_HIP
 * before anything is launched.
 * Source: attention restricted to the sliding 3D window ("Fast Video
 * Generation with Sliding Tile Attention", abstract).
 */
sta_status sta_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                   int32_t B, int32_t H, int32_t D, sta_dtype dtype, float scale,
                   const sta_geom *g, const sta_index *idx, hipStream_t stream);

/*
 * Backward of sta_fwd, given the upstream gradient dout and the forward's
 * o and lse:
 *   P_ij  = exp(s_ij - lse_i),  dP_ij = <dout_i, v_j>,
 *   Delta_i = <dout_i, o_i>     (written to delta_ws, fp32 [B][H][N]),
 *   dS_ij = P_ij (dP_ij - Delta_i),
 *   dq_i  = scale * sum_j dS_ij k_j,
 *   dk_j  = scale * sum_i dS_ij q_i,   dv_j = sum_i P_ij dout_i.
 * All tensors [B][H][N][D] in tile order; dq, dk, dv are fully written
 * (no accumulation into existing contents); no atomics, deterministic.
 * Needs the transposed lists (idx->q_idx, idx->q_cnt).  delta_ws is a
 * caller-owned device workspace of B*H*N floats.  bf16: the dK/dV and dQ
 * stages take their work plan from the stream-ordered workspace
 * (Conventions); with dK/dV it also orders each list set's key tiles by the
 * length of their transposed lists (grids of at most 4096 tiles), and the
 * same workspace holds 2*B*H*N more floats, -lse*log2(e) and -Delta of
 * every row, which a pass before the dK/dV kernel writes (Delta is read
 * from delta_ws, so a call of the dK/dV stage alone needs it filled).
 * Source: the pages' system adapts a pre-trained DiT by full-parameter
 * training through the local attention operator ("MegaSlide-DiT",
 * abstract), which needs these gradients.
 */
sta_status sta_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dout, void *dq, void *dk, void *dv, float *delta_ws,
                   int32_t B, int32_t H, int32_t D, sta_dtype dtype, float scale,
                   const sta_geom *g, const sta_index *idx, hipStream_t stream);

/* Stages of the backward, for sta_bwd_parts. */
typedef STA_ENUM {
    STA_BWD_DELTA = 1,   /* delta_ws = rowsum(dout o o)                     */
    STA_BWD_DKDV = 2,    /* dk, dv   (reads delta_ws)                        */
    STA_BWD_DQ = 4,      /* dq       (reads delta_ws)                        */
    STA_BWD_ALL = 7
} sta_bwd_part;

/*
 * sta_bwd restricted to the stages in `parts` (a mask of sta_bwd_part),
 * run in the order DELTA, DKDV, DQ.  sta_bwd == sta_bwd_parts(..., STA_BWD_ALL).
 * Outputs of stages not requested may be NULL and are not touched; a stage
 * that reads delta_ws expects it to hold the DELTA stage's result for the
 * same o and dout.  Lets a caller skip dq (queries that need no gradient) or
 * dk/dv, or time the stages one by one.  Same arguments and errors as sta_bwd.
 */
sta_status sta_bwd_parts(const void *q, const void *k, const void *v, const void *o, const float *lse,
                         const void *dout, void *dq, void *dk, void *dv, float *delta_ws,
                         int32_t B, int32_t H, int32_t D, sta_dtype dtype, float scale,
                         const sta_geom *g, const sta_index *idx, int32_t parts, hipStream_t stream);

/* Arithmetic of the forward (sta_attn_opts.precision). */
typedef STA_ENUM {
    /* The tensors' dtype: bf16 MFMA with fp32 accumulation, or fp32. */
    STA_PREC_DEFAULT = 0,
    /* bf16 tensors, quantized products: per (b, h) K is smoothed by its
     * mean over the rows and V scaled per channel; Q is coded in int8 per
     * row and K per block of 64 keys of a tile (rint(x * 127 / max|x|));
     * S = QK^T runs on int8 MFMA (exact int32 sums); P = 2^(s - m + 4)
     * is rounded to FP8 E4M3 (OCP, nearest even) with m an integer-valued
     * running max (the same as rounding at 16 times the row-max scale), and
     * PV runs on FP8 MFMA with V in E4M3; the row sum uses the rounded P.  lse is that of the unsmoothed scores.  Forward only.
     * Error against exact attention: about 4 % relative L2 on N(0,1)
     * inputs (spread-out softmax rows, the hardest case for P in E4M3). */
    STA_PREC_FP8 = 1
} sta_precision;

/* Row order of the attention tensors (sta_attn_opts.layout). */
typedef STA_ENUM {
    /* Tile order: the rows of a tile are contiguous (sta_tile_reorder makes
     * it from raster order).  Every geometry. */
    STA_LAYOUT_TILE = 0,
    /* Raster order: the video rows of a slab are the tokens in raster order
     * (t slowest, w fastest) and the kernels gather each tile's rows where
     * its tokens sit, so no reorder pass is needed.  Grids the tile divides
     * and n_text = 0 only; with bf16 tensors also tw | 16, th*tw a power of
     * two and 32 | L (else STA_ERR_UNSUPPORTED). */
    STA_LAYOUT_RASTER = 1
} sta_layout;

/* Options of the attention calls.  A NULL pointer means all fields 0. */
typedef struct {
    /* Text tokens appended after the N video tokens of every (b, h) slab
     * (>= 0).  Attention tensors become [B][H][N + n_text][D] (lse and
     * delta_ws [B][H][N + n_text]): rows 0..N-1 are the video tokens in tile
     * order, rows N.. the text tokens in the caller's order.  A text query
     * attends every key, every query attends every text key, and video
     * pairs keep the tile window.  The index is that of the video grid. */
    int32_t n_text;
    /* An sta_precision value (sta_fwd_ex only; sta_bwd_ex needs
     * STA_PREC_DEFAULT and sta_tile_reorder_ex ignores it). */
    int32_t precision;
    /* An sta_layout value: the row order of q, k, v, o, lse, dout, dq, dk,
     * dv and delta_ws (sta_tile_reorder_ex ignores it).  The forward and the
     * backward of one layer must use the same layout. */
    int32_t layout;
} sta_attn_opts;

/*
 * sta_tile_reorder over slabs of N + opts->n_text rows: the first N rows
 * are permuted as by sta_tile_reorder, the text rows after them are copied
 * to the same place.  opts may be NULL (= sta_tile_reorder).  STA_ERR_INVALID
 * for n_text < 0.
 */
sta_status sta_tile_reorder_ex(const void *src, void *dst, int64_t outer, int64_t row_bytes,
                               const sta_geom *g, int32_t inverse, const sta_attn_opts *opts,
                               hipStream_t stream);

/*
 * sta_fwd with options (opts may be NULL = sta_fwd).  With opts->n_text = M
 * > 0, for query row i of a slab of N + M rows the keys j are: for i < N
 * (video) the rows of the tiles listed for tile(i) and the text rows N..;
 * for i >= N (text) every row.  Formulas, dtypes and errors as sta_fwd.
 * With opts->precision = STA_PREC_FP8 (bf16 tensors only) the forward runs
 * the quantized products described at sta_precision; its stream-ordered
 * workspace holds the codes and scales, about B*H*(2*(N+M) + (num_tiles +
 * ceil(M/L))*Lp)*D bytes with Lp = L rounded up to 64.
 * STA_ERR_INVALID for n_text < 0 or an unknown precision;
 * STA_ERR_UNSUPPORTED when N + n_text exceeds 2^30 rows, or for FP8 with
 * fp32 tensors.
 * Source: token-type-aware masking of joint text-video attention (MOD-DiT
 * README, "Token-Type-Aware Masking") over STA's tile windows.
 */
sta_status sta_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
                      int32_t B, int32_t H, int32_t D, sta_dtype dtype, float scale,
                      const sta_geom *g, const sta_index *idx, const sta_attn_opts *opts,
                      hipStream_t stream);

/*
 * sta_bwd_parts with options (opts may be NULL = sta_bwd_parts): the
 * gradients of sta_fwd_ex with the same opts, key set as there.  delta_ws
 * holds B*H*(N + n_text) floats.  Errors as sta_bwd_parts and sta_fwd_ex;
 * STA_ERR_UNSUPPORTED for a precision other than STA_PREC_DEFAULT.
 * Source: as sta_fwd_ex and sta_bwd.
 */
sta_status sta_bwd_ex(const void *q, const void *k, const void *v, const void *o, const float *lse,
                      const void *dout, void *dq, void *dk, void *dv, float *delta_ws,
                      int32_t B, int32_t H, int32_t D, sta_dtype dtype, float scale,
                      const sta_geom *g, const sta_index *idx, int32_t parts, const sta_attn_opts *opts,
                      hipStream_t stream);

/* Options of sta_window_shifts.  A NULL pointer means all fields 0. */
typedef struct {
    /* The sta_border rule of the windows the shifts are chosen for (the
     * index built from them should use the same rule). */
    int32_t border;
    /* 0: one shift set for the batch, chosen on the tile means averaged
     *    over the batch items: offsets_dev is [H][num_tiles][3];
     * 1: one set per batch item: offsets_dev is [B][H][num_tiles][3]. */
    int32_t per_batch;
    /* Text rows after the N video rows of every (b, h) slab of q and k
     * (>= 0; they take no part in the search). */
    int32_t n_text;
    /* An sta_layout value: the row order of q and k. */
    int32_t layout;
} sta_shift_opts;

/*
 * Chooses the window shift of every query tile and head from q and k
 * ([B][H][N + n_text][D], video rows in the order of opts->layout, bf16 or
 * fp32, D 64 or 128, 16-byte aligned) and writes it to offsets_dev (DEVICE int32, the
 * layout of sta_shift_opts.per_batch, (dt, dh, dw) in tiles), ready for
 * sta_build_index_ex with per_head_offsets = 1.
 * Rule (this library's reading: the pages call 3D-DSA's windows motion-
 * adaptive but give no rule):
 *   qbar, kbar = the mean of q and k over the tokens of each tile (a tile
 *     cut by the grid border: over the tokens it holds), per (b, h), then
 *     averaged over the batch items unless per_batch;
 *   z_qk = scale * <qbar_q, kbar_k>;
 *   mass(o) = sum over the key tiles k in the window of q shifted by o of
 *     len_k * exp(z_qk), len_k = tokens of tile k, for every o with
 *     |o_t| <= radius->t, |o_h| <= radius->h, |o_w| <= radius->w, windows of
 *     windows_host[h] under the border rule (as sta_build_index_ex);
 *   the shift of largest mass is written; among equal masses the one with
 *   the smallest |o_t| + |o_h| + |o_w|, then the first in raster order of
 *   (o_t, o_h, o_w).  Masses are fp32 (a choice may differ from exact
 *   arithmetic where two masses agree to fp32 rounding); a query tile whose
 *   masses are all non-finite gets the zero shift.
 * Workspace: 2 * P * H * num_tiles * D * 4 bytes (P = B if per_batch, else
 * 1) from the stream-ordered workspace (Conventions).
 * Errors: STA_ERR_INVALID for NULL or misaligned pointers, B, H, D <= 0, a
 * negative radius, a window < 1, a non-positive or non-finite scale, an
 * unknown border, layout or dtype, per_batch not 0/1, n_text < 0;
 * STA_ERR_UNSUPPORTED for D other than 64 and 128, more than 4096
 * candidate shifts ((2r_t+1)(2r_h+1)(2r_w+1)), a search region (the union
 * of one query tile's candidate windows, at most prod_d min(n_d, w_d +
 * 2 r_d) tiles) above 8192 tiles, or too large a launch.
 * Source: motion-adaptive local windows of 3D-DSA ("MegaSlide-DiT",
 * abstract).
 */
sta_status sta_window_shifts(const void *q, const void *k, int32_t B, int32_t H, int32_t D, sta_dtype dtype,
                             float scale, const sta_geom *g, const sta_dim3 *windows_host,
                             const sta_dim3 *radius, const sta_shift_opts *opts, int32_t *offsets_dev,
                             hipStream_t stream);

/*
 * sta_window_shifts for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, rule, outputs and errors as
 * sta_window_shifts, and the same kernels; the tile means live in a static
 * device array of 16 MiB instead of pool workspace, so the call allocates
 * and frees nothing.  That array (one per GPU, held from the library's
 * first use on that GPU until the process ends) limits a call to
 * 2 * P * H * num_tiles * D * 4 <= 16 MiB (P = B if per_batch, else 1; the
 * 720P shape, 24 heads of 300 tiles at D = 128, fits up to P = 2):
 * STA_ERR_UNSUPPORTED beyond it, before anything is launched.  Every call on
 * a GPU shares that GPU's array, which keeps the last call's contents (each
 * call writes every value it reads, so nothing needs clearing): calls that
 * overlap on one GPU (on different streams, or from different threads
 * without ordering) race on it and give undefined results.  The first call
 * on a GPU looks the array's address up (hipGetSymbolAddress, with that GPU
 * made current for the lookup and the previous device restored).
 */
sta_status sta_window_shifts_noalloc(const void *q, const void *k, int32_t B, int32_t H, int32_t D,
                                     sta_dtype dtype, float scale, const sta_geom *g,
                                     const sta_dim3 *windows_host, const sta_dim3 *radius,
                                     const sta_shift_opts *opts, int32_t *offsets_dev, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBSTA_H */
