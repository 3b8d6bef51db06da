// Sliding-tile attention backward, bf16 in / fp32 accumulate, gfx950.
//
// Gradients of the tile-masked softmax attention of the forward pass, for
// full-parameter training through the local attention operator
// ("MegaSlide-DiT: Memory-Centric Adaptation and Deformable Local Attention
// for Efficient Video Diffusion", abstract):
//   P = exp(s - lse),  dP = dO V^T,  Delta = rowsum(dO o O),
//   dS = P o (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// P enters the products rounded to bf16; dK/dV also form dS from that
// rounded P (dQ from the fp32 one).
// Three kernels, no atomics, deterministic:
//   1. bwd_pre: Delta_i = <dO_i, O_i> (fp32), one pass over O and dO.
//   2. dq: query-stationary, walks each query tile's key-tile list (same
//      schedule as the forward) and accumulates dQ in registers.
//   3. dkdv: key-stationary, walks each key tile's TRANSPOSED list (the query
//      tiles whose window holds it) and accumulates dK and dV in registers.
// S and dP are recomputed in both 2 and 3.
// Joint text + video sequences (MOD-DiT README, "Token-Type-Aware
// Masking"): both walks continue past their list into the text
// pseudo-tiles, and a text pseudo-tile walks every video tile first (every
// query attends the text keys; a text query attends every key).
//
// MFMA orientation (see mfma.h for the fragment conventions):
//   dq:   S^T = K Q^T, dP^T = V dO^T      (A = K / V rows from LDS, B = Q / dO
//                                          in VGPRs; lane owns a query row)
//         dQ^T += K^T dS^T                 (A = K^T by LDS transpose reads)
//   dkdv: S = Q K^T, dP = dO V^T          (A = Q / dO rows from LDS, B = K / V
//                                          in VGPRs; lane owns a key row)
//         dV += P^T dO, dK += dS^T Q       (B = dO / Q by LDS transpose reads)
// The key (dQ) or query (dK/dV) blocks of a list are walked with counters
// and copied HBM -> LDS through buffer descriptors whose per-lane offsets
// are loop-invariant; rows past a ragged tile end read as zero.  No mask is
// needed for them: in dQ a zero key row adds dS*0 to dQ (and its P, dS stay
// finite); in dK/dV a zero query row has zero Q and dO, so it adds nothing
// to dK = dS^T Q or dV = P^T dO.
// LDS tiles are row-major with 16-byte granules XOR-swizzled by
// f(r) = 4*(r mod 4) ^ ((r / 4) mod 4), which keeps both the 16-byte row
// reads (16 distinct rows per 16 lanes) and the transpose reads (4 rows x
// 32 bytes per 16 lanes) free of bank conflicts.
#include <type_traits>

#include "common.h"
#include "mfma.h"

namespace sta {

template <int GR>
__device__ inline int swz_u(int r) { return ((((r & 3) << 2) ^ ((r >> 2) & 3))) & (GR - 1); }

// ---------------------------------------------------------------------------
// 1. Delta = rowsum(dO * O).  16 lanes per row (16 bytes each for D=128).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16 *__restrict__ O, const __bf16 *__restrict__ dO,
                                                      float *__restrict__ delta, int64_t rows)
{
    constexpr int LPR = D / 8;                 // lanes per row
    const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LPR;
    const int part = threadIdx.x % LPR;
    float s = 0.f;
    if (row < rows) {
        const bf16x8 a = ld8(O + row * D + part * 8);
        const bf16x8 b = ld8(dO + row * D + part * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) s = fmaf((float)a[i], (float)b[i], s);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, LPR);
    if (row < rows && part == 0) delta[row] = s;
}

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
    static_assert(ROWS * D % (THREADS * 8) == 0, "tile must split evenly");
    int off[SHIFT ? 1 : COPIES];
    __device__ explicit RowCopy(int tid)
    {
        const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
        for (int i = 0; i < (SHIFT ? 1 : COPIES); ++i) {
            const int slot = (i * W + wave) * 64 + lane;
            const int r = slot / GR, pg = slot % GR;
            off[i] = (r * D + (pg ^ swz_u<GR>(r)) * 8) * 2;
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

// ---------------------------------------------------------------------------
// 2. dQ (query-stationary).
// ---------------------------------------------------------------------------
template <int D, int NW, int BN, int NBUF, bool RASTER>
__global__ __launch_bounds__(NW * 64, 2) void dq_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    const __bf16 *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Delta,
    __bf16 *__restrict__ dQ, const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ kv_cnt, int max_kv,
    int IH, Geo g, int rblocks, int total, float scale_log2, float scale)
{
    constexpr int THREADS = NW * 64, M = NW * 32, KS = D / 16, KB = BN / 32, DB = D / 32;
    constexpr int BLK = BN * D, STAGE = 2 * BLK;
    // one array per ring slot: the compiler then sees that LDS reads of one
    // slot never alias the copies in flight into another
    __shared__ __attribute__((aligned(1024))) __bf16 slot0[STAGE], slot1[STAGE], slot2[NBUF > 2 ? STAGE : 1];
    auto stage = [&](auto bc) -> __bf16 * {
        constexpr int b = decltype(bc)::value;
        if constexpr (b == 0) return slot0;
        else if constexpr (b == 1) return slot1;
        else return slot2;
    };

    int bh, qt, rb;
    decode_item(xcd_remap(blockIdx.x, total), rblocks, g, bh, qt, rb);
    const Span qs = tile_span(g, qt);                // query rows of this tile
    const int qlen = qs.len;
    if (rb * M >= qlen) return;                      // row block past a cut tile's end
    const int h = bh % IH;                           // list set: the head's, or (b, h)'s
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, grp = lane >> 5;
    const int64_t base = (int64_t)bh * g.S * D;
    const int row = rb * M + wave * 32 + l32;        // query row (inside the tile) of this lane
    const bool row_ok = row < qlen;
    const int64_t grow = slab_row<RASTER>(g, qt, qs, row_ok ? row : qlen - 1);

    bf16x8 qf[KS], of[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = ld8(Q + base + grow * D + ks * 16 + grp * 8);
        of[ks] = ld8(dO + base + grow * D + ks * 16 + grp * 8);
    }
    const float nlse2 = -LSE[(int64_t)bh * g.S + grow] * 1.4426950408889634f;
    const float dlt = Delta[(int64_t)bh * g.S + grow];
    // Q, dO, LSE, Delta complete before the first copy (later waits leave
    // copies in flight, which would otherwise guard every use of them).
    wait_vmem<0>();

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    // key tiles: the window's list, or every video tile for a text query
    const bool video_q = qt < g.T;
    const int cnt = video_q ? kv_cnt[(int64_t)h * g.T + qt] : g.T;
    const int32_t *lst = video_q ? kv_idx + ((int64_t)h * g.T + qt) * max_kv : nullptr;
    const int nblk = walk_blocks(g, lst, cnt, BN);

    // LDS offsets: a row's swizzle only XORs granule bits, and the granule
    // bits that vary with the step (ks) or column block (db) sit above the
    // lane's own, so every offset is one per-lane base XOR a constant.
    const int kbase = lds_at<D>(sigma32(l32), 8 * grp);            // step ks: ^ 16*ks
    const int vj = (lane & 15) >> 2, vc = lane & 3;
    // (the swizzle of row r depends on r mod 16, so each half has its own base)
    int tbase[2];                                                   // column block db: ^ 32*db
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) tbase[hh] = lds_at<D>(8 * grp + 4 * hh + vj, 16 * ((lane >> 4) & 1) + 4 * vc);

    static_assert(!RASTER || BN == 32, "raster walk of 32-row blocks");
    const RowCopy<D, THREADS, BN> rc(tid);
    const RowCopyRaster<D, THREADS, BN> rcr(tid, g);
    ListWalk cw;                                    // next key block to copy
    walk_init<RASTER>(cw, lst, cnt, g);
    auto gload = [&](auto bc) {
        if constexpr (RASTER) {
            // video tiles only (no text rows in the raster layout); the
            // descriptor spans the block's rows (g.rs_span from its first)
            rcr.copy(K + base + (int64_t)cw.roff * D, g.rs_span * D * 2, stage(bc), wave, g);
            rcr.copy(V + base + (int64_t)cw.roff * D, g.rs_span * D * 2, stage(bc) + BLK, wave, g);
        } else {
            const int valid = cw.sp.len - cw.r0 < BN ? cw.sp.len - cw.r0 : BN;
            const int64_t row0 = cw.sp.start + cw.r0;
            rc.copy(K + base + row0 * D, valid, stage(bc), wave);
            rc.copy(V + base + row0 * D, valid, stage(bc) + BLK, wave);
        }
        walk_next<RASTER>(cw, lst, cnt, BN, g);
    };

    auto step = [&](auto bufc, int blk) {
        constexpr int BUF = decltype(bufc)::value;
        ring_wait<NBUF, 2 * decltype(rc)::COPIES>(blk, nblk);
        if (blk + NBUF - 1 < nblk) gload(std::integral_constant<int, (BUF + NBUF - 1) % NBUF>{});
        const __bf16 *Ks = stage(bufc);
        const __bf16 *Vs = Ks + BLK;

        f32x16 s[KB], dp[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) { s[kb][r] = 0.f; dp[kb][r] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s[kb] = mfma32(ld8(Ks + kb * 32 * D + (kbase ^ (16 * ks))), qf[ks], s[kb]);
                dp[kb] = mfma32(ld8(Vs + kb * 32 * D + (kbase ^ (16 * ks))), of[ks], dp[kb]);
            }
        }
        bf16x8 dsf[KB][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                bf16x8 v;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 8 * hf + i;
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale_log2, nlse2));
                    v[i] = (__bf16)(p * (dp[kb][r] - dlt));
                }
                dsf[kb][hf] = v;
            }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const __bf16 *kp = Ks + (kb * 32 + kk * 16) * D;
                    acc[db] = mfma32(cat8(ld_tr4(kp + (tbase[0] ^ (32 * db))), ld_tr4(kp + (tbase[1] ^ (32 * db)))),
                                     dsf[kb][kk], acc[db]);
                }
    };

    static_for<0, NBUF - 1>([&](auto bc) {
        if ((int)decltype(bc)::value < nblk) gload(bc);
    });
    for (int blk = 0; blk < nblk; blk += NBUF)
        static_for<0, NBUF>([&](auto bc) {
            if (blk + (int)decltype(bc)::value < nblk) step(bc, blk + (int)decltype(bc)::value);
        });

    if (row_ok) {
        __bf16 *op = dQ + base + slab_row<RASTER>(g, qt, qs, row) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 v;
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = (__bf16)(acc[db][4 * j + t] * scale);
                *(bf16x4 *)(op + db * 32 + 8 * j + 4 * grp) = v;
            }
    }
}

// ---------------------------------------------------------------------------
// 3. dK, dV (key-stationary, over the transposed lists).
// ---------------------------------------------------------------------------
template <int D, int NW, int BQ, int NBUF, bool RASTER>
__global__ __launch_bounds__(NW * 64, 2) void dkdv_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    const __bf16 *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Delta,
    __bf16 *__restrict__ dK, __bf16 *__restrict__ dV, const int32_t *__restrict__ q_idx,
    const int32_t *__restrict__ q_cnt, int max_q, int IH, Geo g, int rblocks, int total, float scale_log2,
    float scale)
{
    constexpr int THREADS = NW * 64, M = NW * 32, KS = D / 16, SB = BQ / 32, DB = D / 32;
    constexpr int BLK = BQ * D;
    constexpr int SROWS = BQ > 64 ? BQ : 64;        // LSE / Delta slots (one 64-lane dword copy each)
    constexpr int STAGE = 2 * BLK + 2 * SROWS * 2;  // Q, dO (bf16) + LSE, Delta (fp32 as 2 bf16 slots each)
    static_assert(BQ <= 64 && BQ % 32 == 0, "query block of 32 or 64 rows");
    __shared__ __attribute__((aligned(1024))) __bf16 slot0[STAGE], slot1[STAGE], slot2[NBUF > 2 ? STAGE : 1];
    auto stage = [&](auto bc) -> __bf16 * {
        constexpr int b = decltype(bc)::value;
        if constexpr (b == 0) return slot0;
        else if constexpr (b == 1) return slot1;
        else return slot2;
    };

    int bh, kt, rb;
    decode_item(xcd_remap(blockIdx.x, total), rblocks, g, bh, kt, rb);
    const Span ks_ = tile_span(g, kt);               // key rows of this tile
    const int klen = ks_.len;
    if (rb * M >= klen) return;                      // row block past a cut tile's end
    const int h = bh % IH;                           // list set: the head's, or (b, h)'s
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, grp = lane >> 5;
    const int64_t base = (int64_t)bh * g.S * D;
    const int64_t sbase = (int64_t)bh * g.S;
    const int krow0 = rb * M + wave * 32;            // first key row (inside the tile) of this wave
    const int krow = krow0 + l32;
    const int64_t gk = slab_row<RASTER>(g, kt, ks_, krow < klen ? krow : klen - 1);

    bf16x8 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = ld8(K + base + gk * D + ks * 16 + grp * 8);
        vf[ks] = ld8(V + base + gk * D + ks * 16 + grp * 8);
    }
    wait_vmem<0>();          // K, V complete before the first copy (see dq_kernel)
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dk[db][r] = 0.f; dv[db][r] = 0.f; }

    // query tiles: the transposed list, or every video tile for a text key
    const bool video_k = kt < g.T;
    const int cnt = video_k ? q_cnt[(int64_t)h * g.T + kt] : g.T;
    const int32_t *lst = video_k ? q_idx + ((int64_t)h * g.T + kt) * max_q : nullptr;
    const int nblk = walk_blocks(g, lst, cnt, BQ);

    // LDS offsets: a row's swizzle only XORs granule bits, and the granule
    // bits that vary with the step (ks) or column block (db) sit above the
    // lane's own, so every offset is one per-lane base XOR a constant.
    const int kbase = lds_at<D>(sigma32(l32), 8 * grp);            // step ks: ^ 16*ks
    const int vj = (lane & 15) >> 2, vc = lane & 3;
    // (the swizzle of row r depends on r mod 16, so each half has its own base)
    int tbase[2];                                                   // column block db: ^ 32*db
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) tbase[hh] = lds_at<D>(8 * grp + 4 * hh + vj, 16 * ((lane >> 4) & 1) + 4 * vc);

    static_assert(!RASTER || BQ == 32, "raster walk of 32-row blocks");
    const RowCopy<D, THREADS, BQ> rc(tid);
    const RowCopyRaster<D, THREADS, BQ> rcr(tid, g);
    ListWalk cw;                                    // next query block to copy
    walk_init<RASTER>(cw, lst, cnt, g);
    auto gload = [&](auto bc) {
        int valid;
        int64_t row0;
        int lo = lane * 4;
        if constexpr (RASTER) {
            // video tiles only (no text rows in the raster layout); the
            // descriptors span the block's rows (g.rs_span from its first)
            rcr.copy(Q + base + (int64_t)cw.roff * D, g.rs_span * D * 2, stage(bc), wave, g);
            rcr.copy(dO + base + (int64_t)cw.roff * D, g.rs_span * D * 2, stage(bc) + BLK, wave, g);
            row0 = cw.roff;
            valid = g.rs_span;
            // slot `lane` holds row raster_step(lane); slots past the block
            // read past the descriptor, i.e. zero
            lo = lane < BQ ? raster_step_p2(g, lane) * 4 : 0x7ffffffc;
        } else {
            valid = cw.sp.len - cw.r0 < BQ ? cw.sp.len - cw.r0 : BQ;
            row0 = cw.sp.start + cw.r0;
            rc.copy(Q + base + row0 * D, valid, stage(bc), wave);
            rc.copy(dO + base + row0 * D, valid, stage(bc) + BLK, wave);
        }
        if (wave == 0) {                            // LSE and Delta of the block's rows (zero past the end)
            const auto rl = make_rsrc(LSE + sbase + row0, valid * 4);
            const auto rd = make_rsrc(Delta + sbase + row0, valid * 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (__attribute__((address_space(3))) void *)(stage(bc) + 2 * BLK),
                                                     4, lo, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rd, (__attribute__((address_space(3))) void *)(stage(bc) + 2 * BLK + 2 * SROWS), 4, lo, 0, 0, 0);
        }
        walk_next<RASTER>(cw, lst, cnt, BQ, g);
    };

    auto step = [&](auto bufc, int blk) {
        constexpr int BUF = decltype(bufc)::value;
        if (wave == 0)
            ring_wait<NBUF, 2 * decltype(rc)::COPIES + 2>(blk, nblk);
        else
            ring_wait<NBUF, 2 * decltype(rc)::COPIES>(blk, nblk);
        if (blk + NBUF - 1 < nblk) gload(std::integral_constant<int, (BUF + NBUF - 1) % NBUF>{});
        // keep the per-step offsets (base ^ constant) from being hoisted
        // into registers of their own for the whole loop
        int kb_ = kbase, tb0 = tbase[0], tb1 = tbase[1];
        asm volatile("" : "+v"(kb_), "+v"(tb0), "+v"(tb1));
        const __bf16 *Qs = stage(bufc);
        const __bf16 *Os = Qs + BLK;
        const float *Ls = (const float *)(Qs + 2 * BLK);
        const float *Dl = Ls + SROWS;

#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
            // S, then P (rounded to bf16: the dV operand), then dP and
            // dS = P (dP - Delta) from the same rounded P, so that S and dP
            // are never live together.
            // Registers 8kk..8kk+7 hold query rows sb*32 + 16kk + 8grp + 0..7.
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mfma32(ld8(Qs + sb * 32 * D + (kb_ ^ (16 * ks))), kf[ks], acc);
            bf16x8 pf[2], dsf[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int qr = sb * 32 + 16 * kk + 8 * grp;
                const f32x4 l0 = *(const f32x4 *)(Ls + qr), l1 = *(const f32x4 *)(Ls + qr + 4);
                bf16x8 pv;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float lse = i < 4 ? l0[i] : l1[i - 4];
                    pv[i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(acc[8 * kk + i], scale_log2, -lse * 1.4426950408889634f));
                }
                pf[kk] = pv;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mfma32(ld8(Os + sb * 32 * D + (kb_ ^ (16 * ks))), vf[ks], acc);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int qr = sb * 32 + 16 * kk + 8 * grp;
                const f32x4 d0 = *(const f32x4 *)(Dl + qr), d1 = *(const f32x4 *)(Dl + qr + 4);
                bf16x8 dv8;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float dl = i < 4 ? d0[i] : d1[i - 4];
                    dv8[i] = (__bf16)((float)pf[kk][i] * (acc[8 * kk + i] - dl));
                }
                dsf[kk] = dv8;
            }
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int off = (sb * 32 + kk * 16) * D;
                    const int t0 = tb0 ^ (32 * db), t1 = tb1 ^ (32 * db);
                    dv[db] = mfma32(pf[kk], cat8(ld_tr4(Os + off + t0), ld_tr4(Os + off + t1)), dv[db]);
                    dk[db] = mfma32(dsf[kk], cat8(ld_tr4(Qs + off + t0), ld_tr4(Qs + off + t1)), dk[db]);
                }
        }
    };

    static_for<0, NBUF - 1>([&](auto bc) {
        if ((int)decltype(bc)::value < nblk) gload(bc);
    });
    for (int blk = 0; blk < nblk; blk += NBUF)
        static_for<0, NBUF>([&](auto bc) {
            if (blk + (int)decltype(bc)::value < nblk) step(bc, blk + (int)decltype(bc)::value);
        });

    // lane holds column d = 32*db + l%32 of key rows 8*(r/4) + 4*grp + r%4.
    // Raster: krow0 starts a 32-row block, so row krow0 + x sits
    // raster_step(x) rows after row krow0; lane x of `rstep_x` holds that.
    const int64_t rrow0 = RASTER ? slab_row<RASTER>(g, kt, ks_, krow0) : 0;
    const int rstep_x = RASTER ? raster_step_p2(g, l32) : 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int kr = krow0 + mfma_row(lane, r);
        if (kr < klen) {
            const int64_t orow = RASTER ? rrow0 + __shfl(rstep_x, mfma_row(lane, r)) : ks_.start + kr;
            const int64_t o = base + orow * D + l32;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                dK[o + db * 32] = (__bf16)(dk[db][r] * scale);
                dV[o + db * 32] = (__bf16)dv[db][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------

// Tile shapes (overridable at compile time for tuning sweeps): waves per
// workgroup, keys per block in dQ, query rows per block in dK/dV, LDS ring
// depth.
#ifndef STA_BWD_NW
#define STA_BWD_NW 4
#endif
#ifndef STA_BWD_NBUF
#define STA_BWD_NBUF 2
#endif
#ifndef STA_BWD_BN
#define STA_BWD_BN 32
#endif
#ifndef STA_BWD_BQ
#define STA_BWD_BQ 32
#endif

template <int D>
static sta_status run_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
                          const void *dout, void *dq, void *dk, void *dv, float *delta, int B, int H, float scale,
                          const Geo &g, const sta_index &idx, int parts, hipStream_t s)
{
    constexpr int NW = STA_BWD_NW, BN = STA_BWD_BN, BQ = STA_BWD_BQ, M = NW * 32;
    const int64_t rows = (int64_t)B * H * g.S;
    const int rblocks = (g.L + M - 1) / M;
    const int64_t total = (int64_t)B * H * g.TT * rblocks;
    if (!grid_fits(total, NW * 64) || !grid_fits((rows * (D / 8) + 255) / 256, 256))
        return fail(STA_ERR_UNSUPPORTED, "too many work items");
    const float scale_log2 = scale * 1.4426950408889634f;
    const __bf16 *Q = (const __bf16 *)q, *K = (const __bf16 *)k, *V = (const __bf16 *)v;
    const __bf16 *O = (const __bf16 *)o, *dO = (const __bf16 *)dout;

    sta_status st = STA_OK;
    if (parts & STA_BWD_DELTA) {
        hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((rows * (D / 8) + 255) / 256)), dim3(256), 0, s, O, dO,
                           delta, rows);
        if ((st = check_launch()) != STA_OK) return st;
    }
    if (parts & STA_BWD_DKDV) {
        if (g.raster)
            hipLaunchKernelGGL((dkdv_kernel<D, NW, BQ, STA_BWD_NBUF, true>), dim3((unsigned)total), dim3(NW * 64), 0, s, Q, K,
                               V, dO, lse, (const float *)delta, (__bf16 *)dk, (__bf16 *)dv, idx.q_idx, idx.q_cnt, idx.max_q,
                               idx.num_heads, g, rblocks, (int)total, scale_log2, scale);
        else
            hipLaunchKernelGGL((dkdv_kernel<D, NW, BQ, STA_BWD_NBUF, false>), dim3((unsigned)total), dim3(NW * 64), 0, s, Q, K,
                               V, dO, lse, (const float *)delta, (__bf16 *)dk, (__bf16 *)dv, idx.q_idx, idx.q_cnt, idx.max_q,
                               idx.num_heads, g, rblocks, (int)total, scale_log2, scale);
        if ((st = check_launch()) != STA_OK) return st;
    }
    if (parts & STA_BWD_DQ) {
        if (g.raster)
            hipLaunchKernelGGL((dq_kernel<D, NW, BN, STA_BWD_NBUF, true>), dim3((unsigned)total), dim3(NW * 64), 0, s, Q, K, V,
                               dO, lse, (const float *)delta, (__bf16 *)dq, idx.kv_idx, idx.kv_cnt, idx.max_kv, idx.num_heads,
                               g, rblocks, (int)total, scale_log2, scale);
        else
            hipLaunchKernelGGL((dq_kernel<D, NW, BN, STA_BWD_NBUF, false>), dim3((unsigned)total), dim3(NW * 64), 0, s, Q, K, V,
                               dO, lse, (const float *)delta, (__bf16 *)dq, idx.kv_idx, idx.kv_cnt, idx.max_kv, idx.num_heads,
                               g, rblocks, (int)total, scale_log2, scale);
        if ((st = check_launch()) != STA_OK) return st;
    }
    return st;
}

sta_status launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                           const void *dout, void *dq, void *dk, void *dv, float *delta, int B, int H, int D,
                           float scale, const Geo &g, const sta_index &idx, int parts, hipStream_t s)
{
    if (D == 128) return run_bwd<128>(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, scale, g, idx, parts, s);
    return run_bwd<64>(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, scale, g, idx, parts, s);
}

}  // namespace sta
