// Row tiles in LDS shared by the attention kernels that stage key / value
// (or query / gradient) rows: a row-major tile of D-wide bf16 rows whose
// 16-byte granules are XOR-swizzled by f(r) = 4*(r mod 4) ^ ((r / 4) mod 4),
// which keeps both the 16-byte row reads (16 distinct rows per 16 lanes) and
// the transposing reads (4 rows x 32 bytes per 16 lanes) free of bank
// conflicts; the asynchronous copies that fill such tiles; the LDS ring of
// copy stages; and the counter-walked list of key (or query) tiles.
#pragma once

#include <type_traits>

#include "common.h"
#include "mfma.h"

namespace sta {

template <int GR>
__device__ inline int swz_u(int r) { return ((((r & 3) << 2) ^ ((r >> 2) & 3))) & (GR - 1); }

// Byte offsets (inside a row-major tile of D-wide bf16 rows) of the
// 16-byte granules that copy i of thread tid moves into a swizzled LDS tile:
// wave-wide copy i fills LDS granule slots (i*W + wave)*64 + lane, i.e. row
// r = slot / GR, physical granule p, which receives logical granule
// p ^ f(r).  Loop-invariant: computed once per kernel.
template <int D, int THREADS, int ROWS>
struct RowCopy {
    static constexpr int GR = D / 8;
    static constexpr int W = THREADS / 64;
    static constexpr int COPIES = ROWS * D / (THREADS * 8);
    static constexpr int ROWS_PER_COPY = W * 64 / GR;
    // the swizzle repeats every 16 rows: when a copy spans a multiple of
    // that, copy i is copy 0 shifted by i*ROWS_PER_COPY rows
    static constexpr bool SHIFT = ROWS_PER_COPY % 16 == 0;
    // with 16 granules per row, f(r + 8) = f(r) ^ 2: a copy 8 rows on reads
    // the granule with bit 1 flipped, so the odd copies share one offset
    static constexpr bool SHIFT8 = !SHIFT && GR == 16 && ROWS_PER_COPY == 8;
    static constexpr int NOFF = SHIFT ? 1 : SHIFT8 ? 2 : COPIES;
    static_assert(ROWS * D % (THREADS * 8) == 0, "tile must split evenly");
    int off[NOFF];
    __device__ explicit RowCopy(int tid)
    {
        const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
        for (int i = 0; i < NOFF; ++i) {
            const int slot = (i * W + wave) * 64 + lane;
            const int r = slot / GR, pg = slot % GR;
            off[i] = (r * D + (pg ^ swz_u<GR>(r)) * 8) * 2;
            if constexpr (SHIFT8) off[i] -= i * ROWS_PER_COPY * D * 2;   // the row shift goes to soffset
        }
    }
    // Asynchronous copy of `valid` rows from src into the LDS tile; rows
    // past `valid` (a ragged tile end) read as zero.  Every thread of the
    // workgroup takes part.
    __device__ void copy(const __bf16 *src, int valid, __bf16 *lds, int wave) const
    {
        const auto rs = make_rsrc(src, valid * D * 2);
#pragma unroll
        for (int i = 0; i < COPIES; ++i) {
            if constexpr (SHIFT)
                b2lds16(rs, off[0], lds + (i * W + wave) * 512, i * ROWS_PER_COPY * D * 2);
            else if constexpr (SHIFT8)
                b2lds16(rs, off[i & 1], lds + (i * W + wave) * 512, i * ROWS_PER_COPY * D * 2);
            else
                b2lds16(rs, off[i], lds + (i * W + wave) * 512);
        }
    }
};

// RowCopy for a block of ROWS rows of a whole video tile in raster order:
// row r of the block sits raster_step(r) rows after its first row.  Copy i
// moves the rows of copy 0 shifted by i*ROWS_PER_COPY rows of the tile; with
// at most two copies of 16 rows that is g.rs_16 rows further on (a kernel
// argument), so one register per lane suffices.
template <int D, int THREADS, int ROWS>
struct RowCopyRaster {
    static constexpr int GR = D / 8;
    static constexpr int W = THREADS / 64;
    static constexpr int COPIES = ROWS * D / (THREADS * 8);
    static constexpr int ROWS_PER_COPY = W * 64 / GR;
    static_assert(ROWS_PER_COPY % 16 == 0, "copies must keep the swizzle phase");
    static_assert(COPIES == 1 || (COPIES == 2 && ROWS_PER_COPY == 16), "copy shift is raster_step(16)");
    int off;
    __device__ RowCopyRaster(int tid, const Geo &g)
    {
        const int wave = tid >> 6, lane = tid & 63;
        const int slot = wave * 64 + lane;
        const int r = slot / GR, pg = slot % GR;
        off = (raster_step_p2(g, r) * D + (pg ^ swz_u<GR>(r)) * 8) * 2;
    }
    // Asynchronous copy of a block whose first row is at src; `bytes` bounds
    // the descriptor (every row of a whole tile exists).
    __device__ void copy(const __bf16 *src, int bytes, __bf16 *lds, int wave, const Geo &g) const
    {
        const auto rs = make_rsrc(src, bytes);
#pragma unroll
        for (int i = 0; i < COPIES; ++i) b2lds16(rs, off, lds + (i * W + wave) * 512, i * g.rs_16 * D * 2);
    }
};



// NBUF-slot ring of LDS stages: block b lives in slot b mod NBUF and is
// copied NBUF-1 blocks ahead.  At block blk a wave waits until its copies of
// blk have landed (those of the NBUF-2 later blocks, PER copies each, may
// still be in flight), then a fence-free barrier makes every wave's copies
// visible and tells all waves that the slot of block blk-1 is free.
template <int NBUF, int PER>
__device__ inline void ring_wait(int blk, int nblk)
{
    static_assert(NBUF == 2 || NBUF == 3, "ring depth");
    if constexpr (NBUF == 3) {
        if (blk + 1 < nblk) wait_vmem<PER>();
        else wait_vmem<0>();
    } else {
        wait_vmem<0>();
    }
    barrier_nofence();
}

template <int I, int N, typename F>
__device__ inline void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Position in a walk over the tiles of a key- or query-tile list and then
// the text pseudo-tiles, block by block (no divisions); the next tile id is
// prefetched when a tile is entered.
// With RASTER (video tiles only), `roff` follows the raster row of the
// current 32-row block (no divisions per block: the step of g.rs_step, and
// g.rs_jump more where a tile plane ends).
struct ListWalk {
    int e, r0, next;
    Span sp;                  // rows of the current tile
    int roff;                 // raster layout: first row of the block
};
template <bool RASTER>
__device__ inline void walk_enter(ListWalk &w, int tile, const Geo &g)
{
    w.sp = tile_span(g, tile);
    if constexpr (RASTER) w.roff = (int)raster_base(g, tile);
}
template <bool RASTER>
__device__ inline void walk_init(ListWalk &w, const int32_t *lst, int cnt, const Geo &g)
{
    w.e = 0;
    w.r0 = 0;
    walk_enter<RASTER>(w, entry_tile(lst, cnt, g.T, 0), g);
    w.next = entry_tile(lst, cnt, g.T, 1);
}
template <bool RASTER>
__device__ inline void walk_next(ListWalk &w, const int32_t *lst, int cnt, int step, const Geo &g)
{
    w.r0 += step;
    if constexpr (RASTER) {          // 32-row blocks: the walk of g.rs_*
        w.roff += g.rs_step;
        if ((w.r0 & g.rs_pmask) == 0) w.roff += g.rs_jump;
    }
    if (w.r0 >= w.sp.len) {
        w.r0 = 0;
        ++w.e;
        walk_enter<RASTER>(w, w.next, g);
        w.next = entry_tile(lst, cnt, g.T, w.e + 1);
    }
}

// Element offset of logical (row r, column c) in a swizzled LDS tile.  For
// a column c + 8m whose extra granule bits m are disjoint from those of
// c >> 3, the offset is lds_at(r, c) ^ (8m).
template <int D>
__device__ inline int lds_at(int r, int c)
{
    return r * D + (((c >> 3) ^ swz_u<D / 8>(r)) << 3) + (c & 7);
}

}  // namespace sta
