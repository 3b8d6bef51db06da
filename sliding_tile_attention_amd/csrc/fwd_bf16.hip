// Fused sliding-tile attention forward, bf16 in / fp32 accumulate, gfx950.
//
// Operator ("Fast Video Generation with Sliding Tile Attention", abstract):
// each query tile attends only to the key/value tiles of its 3D window.  The
// mask is tile-granular, so a workgroup that owns rows of one query tile
// walks that tile's key-tile list and never masks inside a tile.
//
// Joint text + video sequences (MOD-DiT README, "Token-Type-Aware
// Masking"): after its listed tiles a video query tile walks the text
// pseudo-tiles; a text pseudo-tile's queries walk every video tile and then
// the text.  Key rows past a pseudo-tile's ragged end are masked like
// those past any block end.
//
// Work decomposition
//   workgroup = NW waves = M = NW*32*QG consecutive query rows of one query
//   tile of one (b, h); work items are ordered head-major and each of the 8
//   XCDs takes one contiguous range of that order, cut at equal cost
//   (schedule.hip), so that the workgroups sharing an XCD's L2 walk
//   neighbouring windows of the same head.
//   The key loop runs over (listed key tile, BN-key block) pairs.  K and V
//   blocks travel HBM -> LDS directly (global_load_lds, no staging
//   registers) as row tiles (tiles.h) into an NBUF-slot ring: the copy of
//   block j+NBUF-1 runs while block j is computed; one barrier per block.
//
// Per wave (QG groups of 32 query rows; lane l owns row l%32 of each):
//   S^T[BN x 32] = K_blk Q^T    (MFMA: A = K rows from LDS, B = Q in VGPRs)
//   online softmax along the key axis, in base 2 with scale*log2(e) folded
//   into one FMA; the running max is only moved when a block's partial sum
//   of probabilities would reach 2^8, which leaves the result exact and
//   skips almost every rescale of the O accumulator;
//   O^T[D x 32] += V_blk^T P^T  (MFMA: A = V^T by LDS transposing reads of
//                                the V rows, B = P in VGPRs)
// K rows are fed permuted by sigma so that each lane's S^T registers hold 8
// consecutive keys -- the B operand of the PV product without any shuffle.
// The transposing reads (ds_read_b64_tr_b16) fetch V^T fragments straight
// from the row tile, so V needs no transposed copy in HBM.
// With QG = 2 row groups per wave every K or V^T fragment read from LDS
// feeds two MFMAs (one per group), which halves the LDS operand bytes per
// flop; the two groups' Q fragments (64 VGPRs at D = 128) and O accumulators
// (128) then take a wave's whole share of the register file at two waves
// per SIMD, so the softmax runs one group at a time.
#include <type_traits>

#include "common.h"
#include "mfma.h"
#include "tiles.h"

namespace sta {

#ifndef STA_FWD_MINB
#define STA_FWD_MINB 3
#endif
// With two row groups per wave: group 0's PV chain interleaved with group
// 1's exponentials, each group reading the V^T fragments itself.
#ifndef STA_FWD_SPLITPV
#define STA_FWD_SPLITPV 0
#endif

struct NoRasterCopy {
    __device__ NoRasterCopy(int, const Geo &) {}
};

// RASTER: q, k, v, o, lse in raster order (whole tiles; rows of a video
// tile gathered by tile_row, K and V blocks by a per-lane raster pattern).
template <int D, int NW, int BN, int NBUF, bool RASTER, int QG>
__global__ __launch_bounds__(NW * 64, QG == 1 ? STA_FWD_MINB : 2) void fwd_bf16_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    __bf16 *__restrict__ O, float *__restrict__ LSE, const int32_t *__restrict__ kv_idx,
    const int32_t *__restrict__ kv_cnt, int max_kv, int IH, Geo g, int rblocks, const int *__restrict__ split,
    float scale_log2)
{
    constexpr int THREADS = NW * 64, M = NW * 32 * QG, KS = D / 16, KB = BN / 32, DB = D / 32;
    constexpr int BLK = BN * D, STAGE = 2 * BLK;
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
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
    {
        // XCD x = block index mod 8 takes the range [split[x], split[x+1]) of
        // the work order (slabs by descending cost); blocks past it exit
        const int x = blockIdx.x & 7, work = split[x] + (int)(blockIdx.x >> 3);
        if (work >= split[x + 1]) return;
        decode_item(work, rblocks, g, bh, qt, rb);
        bh = plan_slab(split, bh);
    }
    const Span qs = tile_span(g, qt);                // query rows of this tile
    const int qlen = qs.len;
    if (rb * M >= qlen) return;                      // row block past a cut tile's end
    const int h = bh % IH;                           // list set: the head's, or (b, h)'s
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, grp = lane >> 5;
    const int64_t base = (int64_t)bh * g.S * D;

    // Q fragments: B operand of S^T = K Q^T, lane = query row, 8 columns;
    // row group q of the wave holds rows rb*M + (wave*QG + q)*32 + 0..31.
    bf16x8 qf[QG][KS];
#pragma unroll
    for (int q = 0; q < QG; ++q) {
        const int row = rb * M + (wave * QG + q) * 32 + l32;
        const bool row_ok = row < qlen;
        const __bf16 *p = Q + base + slab_row<RASTER>(g, qt, qs, row_ok ? row : qlen - 1) * D + grp * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[q][ks] = row_ok ? ld8(p + ks * 16) : zero8();
    }
    wait_vmem<0>();          // Q complete before the first copy (later waits leave copies in flight)

    f32x16 acc[QG][DB];
#pragma unroll
    for (int q = 0; q < QG; ++q)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[q][db][r] = 0.f;
    float m_i[QG], l_i[QG];
#pragma unroll
    for (int q = 0; q < QG; ++q) m_i[q] = -INFINITY, l_i[q] = 0.f;

    // key tiles: the window's list, or every video tile for a text query
    const bool video_q = qt < g.T;
    const int cnt = video_q ? kv_cnt[(int64_t)h * g.T + qt] : g.T;
    const int32_t *lst = video_q ? kv_idx + ((int64_t)h * g.T + qt) * max_kv : nullptr;
    const int nblk = walk_blocks(g, lst, cnt, BN);

    // LDS offsets: a row's swizzle only XORs granule bits, and the granule
    // bits that vary with the step (ks) or column block (db) sit above the
    // lane's own, so every offset is one per-lane base XOR a constant.
    const int kbase = lds_at<D>(sigma32(l32), 8 * grp);            // S^T operand, step ks: ^ 16*ks
    const int vj = (lane & 15) >> 2, vc = lane & 3;
    // V^T operand by transposing reads (the swizzle of row r depends on
    // r mod 16, so each half has its own base); column block db: ^ 32*db
    int tbase[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) tbase[hh] = lds_at<D>(8 * grp + 4 * hh + vj, 16 * ((lane >> 4) & 1) + 4 * vc);

    static_assert(!RASTER || BN == 32, "raster walk of 32-row blocks");
    const RowCopy<D, THREADS, BN> rc(tid);
    // (the raster copy pattern exists for the raster instantiations only)
    const std::conditional_t<RASTER, RowCopyRaster<D, THREADS, BN>, NoRasterCopy> rcr(tid, g);
    ListWalk cw;                                     // next key block to copy
    walk_init<RASTER>(cw, lst, cnt, g);
    int bvalid[NBUF];                                // valid keys of the block in each slot
    // Asynchronous copy of the next K and V block into ring slot bc: rows
    // past a ragged tile end read as zero (their scores are masked below).
    auto gload = [&](auto bc) {
        constexpr int b = decltype(bc)::value;
        if constexpr (RASTER) {
            // video tiles only (no text rows in the raster layout); the
            // descriptor spans the block's rows (g.rs_span from its first)
            bvalid[b] = BN;
            rcr.copy(K + base + (int64_t)cw.roff * D, g.rs_span * D * 2, stage(bc), wave, g);
            rcr.copy(V + base + (int64_t)cw.roff * D, g.rs_span * D * 2, stage(bc) + BLK, wave, g);
        } else {
            const int valid = cw.sp.len - cw.r0 < BN ? cw.sp.len - cw.r0 : BN;
            const int64_t row0 = cw.sp.start + cw.r0;
            bvalid[b] = valid;
            rc.copy(K + base + row0 * D, valid, stage(bc), wave);
            rc.copy(V + base + row0 * D, valid, stage(bc) + BLK, wave);
        }
        walk_next<RASTER>(cw, lst, cnt, BN, g);
    };

    // One key block from ring slot BUF (a compile-time constant, so every
    // LDS address below is a per-lane register plus an immediate).
    auto step = [&](auto bufc, int blk) {
        constexpr int BUF = decltype(bufc)::value;
        ring_wait<NBUF, 2 * decltype(rc)::COPIES>(blk, nblk);
        if (blk + NBUF - 1 < nblk) gload(std::integral_constant<int, (BUF + NBUF - 1) % NBUF>{});
        const __bf16 *Ks = stage(bufc);
        const __bf16 *Vs = Ks + BLK;
        const int valid = bvalid[BUF];
        int kb0 = kbase, tb0 = tbase[0], tb1 = tbase[1];
        if constexpr (QG > 1) {
            // with two row groups the registers are short: hide the bases
            // from the compiler so that it forms each read's offset (one
            // XOR) at the read instead of keeping one register per offset
            asm volatile("" : "+v"(kb0), "+v"(tb0), "+v"(tb1));
        }

        // S^T chain: the K row fragments read FD ahead into a ring of
        // registers; compiler fences keep that issue order (left to itself
        // the compiler issued each read just before its MFMA, which then
        // waited for it)
        static_assert(KB == 1, "one 32-key block per step");
        constexpr int FD = QG == 1 ? 3 : 2;
        f32x16 s[QG];
#pragma unroll
        for (int q = 0; q < QG; ++q)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[q][r] = 0.f;
        bf16x8 rk[FD];
        __builtin_amdgcn_s_setprio(3);             // MFMA phase: issue ahead of other waves' vector work
#pragma unroll
        for (int j = 0; j < FD; ++j) rk[j] = ld8(Ks + (kb0 ^ (16 * j)));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < QG; ++q) s[q] = mfma32(rk[ks % FD], qf[q][ks], s[q]);
            if (ks + FD < KS) rk[ks % FD] = ld8(Ks + (kb0 ^ (16 * (ks + FD))));
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        if (valid < BN) {
            // key of register r (rows fed permuted by sigma): 16*(r/8) + (r%8)
            // + 8*(lane/32), compared against one per-lane limit (the compiler
            // would otherwise keep 16 per-register key indices live across the
            // loop)
            const int lim = valid - 8 * (lane >> 5);
#pragma unroll
            for (int q = 0; q < QG; ++q)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (16 * (r >> 3) + (r & 7) >= lim) s[q][r] = -INFINITY;
        }

        // Probabilities, rounded to bf16 (the PV operand), and their sum,
        // one row group at a time.  Exponents use the running max m_i; a
        // block whose partial sum stays below 2^8 cannot overflow and is
        // accepted as is.  Otherwise (first block, or scores that jumped) the
        // true max is taken, O and l are rescaled, and the block is
        // recomputed.
        bf16x8 pf[QG][2];
        auto probs = [&](auto qc) {
            constexpr int q = decltype(qc)::value;
            const float mneg = -m_i[q];
            float ls = 0.f;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                bf16x8 v;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    v[i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[q][8 * hf + i], scale_log2, mneg));
                pf[q][hf] = v;
                ls = sum8(v, ls);
            }
            return ls;
        };
        auto settle = [&](auto qc, float ls) {
            constexpr int q = decltype(qc)::value;
            if (__any(!(ls < 256.f))) {
                float mx = -INFINITY;
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[q][r]);
                mx = max_pair32(mx) * scale_log2;
                const float mn = fmaxf(m_i[q], mx);
                const float alpha = __builtin_amdgcn_exp2f(m_i[q] - mn);
                m_i[q] = mn;
                l_i[q] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[q][db][r] *= alpha;
                ls = probs(qc);
            }
            l_i[q] += ls;
        };

        // PV: the V^T fragments (two transposing reads each) FV ahead
        constexpr int FV = QG == 1 ? 3 : 2, NV = 2 * DB;
        auto vfrag = [&](int j) -> bf16x8 {
            const __bf16 *vp = Vs + (j & 1) * 16 * D;
            const int db = j >> 1;
            return cat8(ld_tr4(vp + (tb0 ^ (32 * db))), ld_tr4(vp + (tb1 ^ (32 * db))));
        };
        // one group's PV chain: fences keep the reads FV ahead of the MFMAs
        auto pv_chain = [&](auto qc) {
            constexpr int q = decltype(qc)::value;
            bf16x8 rv[FV];
#pragma unroll
            for (int j = 0; j < FV; ++j) rv[j] = vfrag(j);
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                acc[q][j >> 1] = mfma32(rv[j % FV], pf[q][j & 1], acc[q][j >> 1]);
                if (j + FV < NV) rv[j % FV] = vfrag(j + FV);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        using Q0 = std::integral_constant<int, 0>;
        if constexpr (QG == 2 && STA_FWD_SPLITPV) {
            // Group 0's PV chain runs while group 1's exponentials are formed
            // (scheduling groups interleave one MFMA, the two reads of a later
            // fragment and a few vector instructions), then group 1's chain
            // reads the V^T fragments again: the K fragments still feed both
            // groups, the V^T fragments one each.
            using Q1 = std::integral_constant<int, 1>;
            settle(Q0{}, probs(Q0{}));
            __builtin_amdgcn_s_setprio(3);
            float ls1;
            {
                bf16x8 rv = vfrag(0);
                ls1 = probs(Q1{});
#pragma unroll
                for (int j = 0; j < NV; ++j) {
                    acc[0][j >> 1] = mfma32(rv, pf[0][j & 1], acc[0][j >> 1]);
                    if (j + 1 < NV) rv = vfrag(j + 1);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // the first fragment's reads
#pragma unroll
                for (int i = 0; i < NV; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);    // six vector instructions
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);    // the next fragment's reads
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
            settle(Q1{}, ls1);
            __builtin_amdgcn_s_setprio(3);
            pv_chain(Q1{});
            __builtin_amdgcn_s_setprio(0);
        } else {
            static_for<0, QG>([&](auto qc) { settle(qc, probs(qc)); });
            bf16x8 rv[FV];
            __builtin_amdgcn_s_setprio(3);
#pragma unroll
            for (int j = 0; j < FV; ++j) rv[j] = vfrag(j);
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = 0; q < QG; ++q) acc[q][j >> 1] = mfma32(rv[j % FV], pf[q][j & 1], acc[q][j >> 1]);
                if (j + FV < NV) rv[j % FV] = vfrag(j + FV);
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
        }
    };

    static_for<0, NBUF - 1>([&](auto bc) {
        if ((int)decltype(bc)::value < nblk) gload(bc);
    });
    for (int blk = 0; blk < nblk; blk += NBUF)
        static_for<0, NBUF>([&](auto bc) {
            if (blk + (int)decltype(bc)::value < nblk) step(bc, blk + (int)decltype(bc)::value);
        });

    // Epilogue: lanes l and l^32 hold the two halves of a row's sum.  The
    // lane's row is formed anew from its lane id (mbcnt), so that no address
    // or index has to stay live through the key loop.
    const int elane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int egrp = elane >> 5;
#pragma unroll
    for (int q = 0; q < QG; ++q) {
        const float lt = sum_pair32(l_i[q]);
        const float inv = 1.f / lt;
        const int erow = rb * M + (wave * QG + q) * 32 + (elane & 31);
        if (erow < qlen) {
            const int64_t orow = slab_row<RASTER>(g, qt, qs, erow);
            __bf16 *op = O + base + orow * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bf16x4 v;
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = (__bf16)(acc[q][db][4 * j + t] * inv);
                    *(bf16x4 *)(op + db * 32 + 8 * j + 4 * egrp) = v;
                }
            if (egrp == 0) LSE[(int64_t)bh * g.S + orow] = (m_i[q] + __log2f(lt)) * 0.69314718055994531f;
        }
    }
}

// Tile shape: waves per workgroup, keys per LDS block, ring slots, row
// groups per wave.  The operand rings of the step walk one 32-key block per
// step, so the key block stays 32 rows wide (the step asserts it); the wave
// count and the LDS ring depth may be set at compile time for tuning sweeps.
// STA_FWD_QG = 2 builds the tile-order D = 128 forward with two row groups
// per wave in workgroups of STA_FWD_NW2 waves (two waves per SIMD): half the
// LDS operand bytes per flop, but slower at the 720p workload than one group
// at three waves per SIMD, so one group is the default.  D = 64 and the
// raster layout (whose copy pattern needs 16-row copy strides, i.e. four
// waves) always run one group per wave.
#ifndef STA_FWD_NW
#define STA_FWD_NW 4
#endif
#ifndef STA_FWD_BN
#define STA_FWD_BN 32
#endif
#ifndef STA_FWD_NBUF
#define STA_FWD_NBUF 2
#endif
#ifndef STA_FWD_QG
#define STA_FWD_QG 1
#endif
#ifndef STA_FWD_NW2
#define STA_FWD_NW2 2
#endif

// The work plan, then the attention kernel.
template <int D, int NW, int QG, bool RASTER>
static sta_status run_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                          float scale, const Geo &g, const sta_index &idx, hipStream_t s)
{
    constexpr int BN = STA_FWD_BN, NBUF = STA_FWD_NBUF, M = NW * 32 * QG;
    const int rblocks = (g.L + M - 1) / M;
    const int64_t total = (int64_t)B * H * g.TT * rblocks;
    const int64_t blocks = work_blocks(total);
    if (!grid_fits(blocks, NW * 64)) return fail(STA_ERR_UNSUPPORTED, "too many work items");
    void *ws = nullptr;
    sta_status st = workspace_alloc(&ws, plan_bytes(idx.num_heads, (int64_t)B * H), s);
    if (st != STA_OK) return st;
    const int *split = nullptr;
    if ((st = plan_work(g, idx.kv_cnt, idx.num_heads, (int64_t)B * H, rblocks, blocks, ws, s, &split)) != STA_OK) {
        (void)workspace_free(ws, s);          // the launch error is the one reported
        return st;
    }
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, BN, NBUF, RASTER, QG>), dim3((unsigned)blocks), dim3(NW * 64), 0, s,
                       (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (__bf16 *)o, lse, idx.kv_idx,
                       idx.kv_cnt, idx.max_kv, idx.num_heads, g, rblocks, split, scale_log2);
    st = check_launch();
    const sta_status fs = workspace_free(ws, s);
    return st != STA_OK ? st : fs;
}

sta_status launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                           int D, float scale, const Geo &g, const sta_index &idx, hipStream_t s)
{
    constexpr int NW = STA_FWD_NW;
    if (D == 128) {
        if (g.raster) return run_fwd<128, NW, 1, true>(q, k, v, o, lse, B, H, scale, g, idx, s);
        if constexpr (STA_FWD_QG > 1)
            return run_fwd<128, STA_FWD_NW2, STA_FWD_QG, false>(q, k, v, o, lse, B, H, scale, g, idx, s);
        return run_fwd<128, NW, 1, false>(q, k, v, o, lse, B, H, scale, g, idx, s);
    }
    if (g.raster) return run_fwd<64, NW, 1, true>(q, k, v, o, lse, B, H, scale, g, idx, s);
    return run_fwd<64, NW, 1, false>(q, k, v, o, lse, B, H, scale, g, idx, s);
}

}  // namespace sta
