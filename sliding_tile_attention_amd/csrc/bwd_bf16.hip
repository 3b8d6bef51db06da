// Sliding-tile attention backward, bf16 in / fp32 accumulate, gfx950.
//
// Gradients of the tile-masked softmax attention of the forward pass, for
// full-parameter training through the local attention operator
// ("MegaSlide-DiT: Memory-Centric Adaptation and Deformable Local Attention
// for Efficient Video Diffusion", abstract):
//   P = exp(s - lse),  dP = dO V^T,  Delta = rowsum(dO o O),
//   dS = P o (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// P enters the dV product rounded to bf16; both kernels form dS from the
// fp32 P.
// Three kernels, no atomics, deterministic:
//   1. bwd_pre: Delta_i = <dO_i, O_i> (fp32), one pass over O and dO; and
//      for dK/dV, lse_log2: -lse_i log2(e) and -Delta_i of every row, so
//      that their loop forms each exponent with one multiply-add and starts
//      the dP product from -Delta.
// Both dP products accumulate onto -Delta (the MFMA chain's initial value),
// so dS = P * (that sum) needs no subtraction.
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
#include "tiles.h"

namespace sta {

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


// -lse * log2(e) of every row (the base-2 exponent offset of dK/dV's P) and
// -Delta (the initial value of its dP product).
__global__ __launch_bounds__(256) void lse_log2_kernel(const float *__restrict__ lse, const float *__restrict__ delta,
                                                       float *__restrict__ nlse2, float *__restrict__ ndelta,
                                                       int64_t rows)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < rows) {
        nlse2[i] = -lse[i] * 1.4426950408889634f;
        ndelta[i] = -delta[i];
    }
}

// ---------------------------------------------------------------------------
// 2. dQ (query-stationary).
// ---------------------------------------------------------------------------
template <int D, int NW, int BN, int NBUF, bool RASTER>
__global__ __launch_bounds__(NW * 64, 2) void dq_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    const __bf16 *__restrict__ dO, const float *__restrict__ LSE, const float *__restrict__ Delta,
    __bf16 *__restrict__ dQ, const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ kv_cnt, int max_kv,
    int IH, Geo g, int rblocks, const int *__restrict__ split, float scale_log2, float scale)
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
    // -Delta of the lane's row in every register: the dP^T chain's start
    f32x16 ndl;
    {
        const float nd = -Delta[(int64_t)bh * g.S + grow];
#pragma unroll
        for (int r = 0; r < 16; ++r) ndl[r] = nd;
    }
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

        static_assert(KB == 1, "one 32-key block per step");
        // S^T and dP^T chains interleaved: pairs (K, V row fragments) read
        // QD pairs ahead into a ring of registers; compiler fences keep
        // that issue order (left to itself the compiler issued each pair of
        // reads just before its MFMAs, which then waited for them).
        constexpr int QD = 2;
        f32x16 s0, dp0 = ndl;
#pragma unroll
        for (int r = 0; r < 16; ++r) s0[r] = 0.f;
        bf16x8 rk[QD], rv[QD];
#pragma unroll
        for (int j = 0; j < QD; ++j) {
            rk[j] = ld8(Ks + (kbase ^ (16 * j)));
            rv[j] = ld8(Vs + (kbase ^ (16 * j)));
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            s0 = mfma32(rk[ks % QD], qf[ks], s0);
            dp0 = mfma32(rv[ks % QD], of[ks], dp0);
            if (ks + QD < KS) {
                rk[ks % QD] = ld8(Ks + (kbase ^ (16 * (ks + QD))));
                rv[ks % QD] = ld8(Vs + (kbase ^ (16 * (ks + QD))));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 dsf[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            bf16x8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * hf + i;
                const float p = __builtin_amdgcn_exp2f(fmaf(s0[r], scale_log2, nlse2));
                v[i] = (__bf16)(p * dp0[r]);
            }
            dsf[hf] = v;
        }
        // dQ^T += K^T dS^T: the K^T fragments (two transposing reads each)
        // QT ahead
        constexpr int QT = 3, NT = 2 * DB;
        auto tfrag = [&](int j) -> bf16x8 {
            const int db = j >> 1, kk = j & 1;
            const __bf16 *kp = Ks + kk * 16 * D;
            return cat8(ld_tr4(kp + (tbase[0] ^ (32 * db))), ld_tr4(kp + (tbase[1] ^ (32 * db))));
        };
        bf16x8 tr[QT];
#pragma unroll
        for (int j = 0; j < QT; ++j) tr[j] = tfrag(j);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            acc[j >> 1] = mfma32(tr[j % QT], dsf[j & 1], acc[j >> 1]);
            if (j + QT < NT) tr[j % QT] = tfrag(j + QT);
        }
        __builtin_amdgcn_sched_barrier(0);
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
    const __bf16 *__restrict__ dO, const float *__restrict__ NLSE2, const float *__restrict__ NDelta,
    __bf16 *__restrict__ dK, __bf16 *__restrict__ dV, const int32_t *__restrict__ q_idx,
    const int32_t *__restrict__ q_cnt, int max_q, int IH, Geo g, int rblocks, const int *__restrict__ split, float scale_log2,
    float scale)
{
    constexpr int THREADS = NW * 64, M = NW * 32, KS = D / 16, SB = BQ / 32, DB = D / 32;
    constexpr int BLK = BQ * D;
    constexpr int SROWS = BQ > 64 ? BQ : 64;        // -lse log2(e) / -Delta slots (one 64-lane dword copy each)
    constexpr int STAGE = 2 * BLK + 2 * SROWS * 2;  // Q, dO (bf16) + -lse log2(e), -Delta (fp32 as 2 bf16 slots each)
    static_assert(BQ <= 64 && BQ % 32 == 0, "query block of 32 or 64 rows");
    __shared__ __attribute__((aligned(1024))) __bf16 slot0[STAGE], slot1[STAGE], slot2[NBUF > 2 ? STAGE : 1];
    auto stage = [&](auto bc) -> __bf16 * {
        constexpr int b = decltype(bc)::value;
        if constexpr (b == 0) return slot0;
        else if constexpr (b == 1) return slot1;
        else return slot2;
    };

    int bh, kt, rb;
    {
        // XCD x = block index mod 8 takes the range [split[x], split[x+1]) of
        // the work order (slabs by descending cost); blocks past it exit
        const int x = blockIdx.x & 7, work = split[x] + (int)(blockIdx.x >> 3);
        if (work >= split[x + 1]) return;
        decode_item(work, rblocks, g, bh, kt, rb);
        bh = plan_slab(split, bh);
        if (kt < g.T) kt = plan_tile(split, bh % IH, g.T, kt);    // longest transposed lists first
    }
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
        if (wave == 0) {                            // -lse log2(e) and -Delta of the block's rows (zero past the end)
            const auto rl = make_rsrc(NLSE2 + sbase + row0, valid * 4);
            const auto rd = make_rsrc(NDelta + sbase + row0, valid * 4);
            if constexpr (NBUF > 2) {
                // LDS addresses from the low 32 bits of the generic ones: the
                // address-space cast's null check fails to compile here
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rl, (__attribute__((address_space(3))) void *)(uint32_t)(uintptr_t)(stage(bc) + 2 * BLK), 4, lo, 0,
                    0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rd, (__attribute__((address_space(3))) void *)(uint32_t)(uintptr_t)(stage(bc) + 2 * BLK + 2 * SROWS),
                    4, lo, 0, 0, 0);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rl, (__attribute__((address_space(3))) void *)(stage(bc) + 2 * BLK), 4, lo, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rd, (__attribute__((address_space(3))) void *)(stage(bc) + 2 * BLK + 2 * SROWS), 4, lo, 0, 0, 0);
            }
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
            // Registers 8kk..8kk+7 hold query rows sb*32 + 16kk + 8grp + 0..7.
            // The S and dP chains as one run of 2*KS MFMAs whose A operands
            // (Q, then dO row fragments) are read PD fragments ahead into a
            // ring of registers; compiler fences keep that issue order (left
            // to itself the compiler issued each read just before its MFMA,
            // which then waited for it).  S and dP are live together (255
            // VGPRs, no spills).
            constexpr int PD = 3;
            f32x16 acc, dpa;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {           // the dP chain starts from -Delta
                const int qr = sb * 32 + 16 * kk + 8 * grp;
                const f32x4 d0 = *(const f32x4 *)(Dl + qr), d1 = *(const f32x4 *)(Dl + qr + 4);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dpa[8 * kk + i] = d0[i];
                    dpa[8 * kk + 4 + i] = d1[i];
                }
            }
            auto frag = [&](int j) -> bf16x8 {
                return j < KS ? ld8(Qs + sb * 32 * D + (kb_ ^ (16 * j))) : ld8(Os + sb * 32 * D + (kb_ ^ (16 * (j - KS))));
            };
            bf16x8 ring[PD];
            __builtin_amdgcn_s_setprio(3);         // MFMA phase: issue ahead of the other wave's vector work
#pragma unroll
            for (int j = 0; j < PD; ++j) ring[j] = frag(j);
#pragma unroll
            for (int j = 0; j < 2 * KS; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                if (j < KS) acc = mfma32(ring[j % PD], kf[j], acc);
                else dpa = mfma32(ring[j % PD], vf[j - KS], dpa);
                if (j + PD < 2 * KS) ring[j % PD] = frag(j + PD);
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
            // P (fp32 in place of S; bf16 for the dV product), dS = P (dP - Delta)
            bf16x8 pf[2], dsf[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int qr = sb * 32 + 16 * kk + 8 * grp;
                const f32x4 l0 = *(const f32x4 *)(Ls + qr), l1 = *(const f32x4 *)(Ls + qr + 4);
                bf16x8 pv, dv8;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float nl2 = i < 4 ? l0[i] : l1[i - 4];
                    const float p = __builtin_amdgcn_exp2f(fmaf(acc[8 * kk + i], scale_log2, nl2));
                    pv[i] = (__bf16)p;
                    dv8[i] = (__bf16)(p * dpa[8 * kk + i]);
                }
                pf[kk] = pv;
                dsf[kk] = dv8;
            }
            // dV += P^T dO, dK += dS^T Q: their B fragments (two transposing
            // reads each) PT MFMAs ahead
            constexpr int PT = 2, NT = 4 * DB;
            auto tfrag = [&](int j) -> bf16x8 {
                const int db = j >> 2, kk = (j >> 1) & 1;
                const int off = (sb * 32 + kk * 16) * D;
                const int t0 = tb0 ^ (32 * db), t1 = tb1 ^ (32 * db);
                const __bf16 *src = (j & 1) ? Qs : Os;
                return cat8(ld_tr4(src + off + t0), ld_tr4(src + off + t1));
            };
            bf16x8 tr[PT];
            __builtin_amdgcn_s_setprio(3);
#pragma unroll
            for (int j = 0; j < PT; ++j) tr[j] = tfrag(j);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                const int db = j >> 2, kk = (j >> 1) & 1;
                if (j & 1) dk[db] = mfma32(dsf[kk], tr[j % PT], dk[db]);
                else dv[db] = mfma32(pf[kk], tr[j % PT], dv[db]);
                if (j + PT < NT) tr[j % PT] = tfrag(j + PT);
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

// Tile shapes: waves per workgroup, LDS ring depth, keys per block in dQ,
// query rows per block in dK/dV.  The dQ operand rings walk one 32-key block
// per step, so its key block stays 32 rows wide (the dQ step asserts it); the
// others may be set at compile time for tuning sweeps.
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
    const int64_t blocks = work_blocks(total);
    if (!grid_fits(blocks, NW * 64) || !grid_fits((rows * (D / 8) + 255) / 256, 256))
        return fail(STA_ERR_UNSUPPORTED, "too many work items");
    const float scale_log2 = scale * 1.4426950408889634f;
    const __bf16 *Q = (const __bf16 *)q, *K = (const __bf16 *)k, *V = (const __bf16 *)v;
    const __bf16 *O = (const __bf16 *)o, *dO = (const __bf16 *)dout;

    sta_status st = STA_OK;
    // the per-XCD work split (both walks have the same cost per slab: the
    // listed tile pairs, counted from either list)
    void *ws = nullptr;
    const int *split = nullptr;
    // (with dK/dV, the key tiles in order of their transposed-list lengths,
    // and after the plan, at 256-byte boundaries, -lse log2(e) and -Delta of
    // every row)
    float *nlse2 = nullptr, *ndelta = nullptr;
    if (parts & (STA_BWD_DKDV | STA_BWD_DQ)) {
        const bool kv = parts & STA_BWD_DKDV;
        const size_t plan = (plan_bytes(idx.num_heads, (int64_t)B * H, kv ? &g : nullptr) + 255) & ~(size_t)255;
        const size_t row_bytes = ((size_t)rows * 4 + 255) & ~(size_t)255;
        if ((st = workspace_alloc(&ws, plan + (kv ? 2 * row_bytes : 0), s)) != STA_OK) return st;
        if (kv) {
            nlse2 = (float *)((char *)ws + plan);
            ndelta = (float *)((char *)ws + plan + row_bytes);
        }
        if ((st = plan_work(g, idx.kv_cnt, idx.num_heads, (int64_t)B * H, rblocks, blocks, ws, s, &split,
                            kv ? idx.q_cnt : nullptr)) != STA_OK) {
            (void)workspace_free(ws, s);      // the launch error is the one reported
            return st;
        }
    }
    auto done = [&](sta_status r) {
        const sta_status fs = workspace_free(ws, s);
        return r != STA_OK ? r : fs;
    };
    if (parts & STA_BWD_DELTA) {
        hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((rows * (D / 8) + 255) / 256)), dim3(256), 0, s, O, dO,
                           delta, rows);
        if ((st = check_launch()) != STA_OK) return done(st);
    }
    if (parts & STA_BWD_DKDV) {
        hipLaunchKernelGGL(lse_log2_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, lse,
                           (const float *)delta, nlse2, ndelta, rows);
        if ((st = check_launch()) != STA_OK) return done(st);
        if (g.raster)
            hipLaunchKernelGGL((dkdv_kernel<D, NW, BQ, STA_BWD_NBUF, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, s, Q, K,
                               V, dO, (const float *)nlse2, (const float *)ndelta, (__bf16 *)dk, (__bf16 *)dv, idx.q_idx, idx.q_cnt, idx.max_q,
                               idx.num_heads, g, rblocks, split, scale_log2, scale);
        else
            hipLaunchKernelGGL((dkdv_kernel<D, NW, BQ, STA_BWD_NBUF, false>), dim3((unsigned)blocks), dim3(NW * 64), 0, s, Q, K,
                               V, dO, (const float *)nlse2, (const float *)ndelta, (__bf16 *)dk, (__bf16 *)dv, idx.q_idx, idx.q_cnt, idx.max_q,
                               idx.num_heads, g, rblocks, split, scale_log2, scale);
        if ((st = check_launch()) != STA_OK) return done(st);
    }
    if (parts & STA_BWD_DQ) {
        if (g.raster)
            hipLaunchKernelGGL((dq_kernel<D, NW, BN, STA_BWD_NBUF, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, s, Q, K, V,
                               dO, lse, (const float *)delta, (__bf16 *)dq, idx.kv_idx, idx.kv_cnt, idx.max_kv, idx.num_heads,
                               g, rblocks, split, scale_log2, scale);
        else
            hipLaunchKernelGGL((dq_kernel<D, NW, BN, STA_BWD_NBUF, false>), dim3((unsigned)blocks), dim3(NW * 64), 0, s, Q, K, V,
                               dO, lse, (const float *)delta, (__bf16 *)dq, idx.kv_idx, idx.kv_cnt, idx.max_kv, idx.num_heads,
                               g, rblocks, split, scale_log2, scale);
        if ((st = check_launch()) != STA_OK) return done(st);
    }
    return done(st);
}

sta_status launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                           const void *dout, void *dq, void *dk, void *dv, float *delta, int B, int H, int D,
                           float scale, const Geo &g, const sta_index &idx, int parts, hipStream_t s)
{
    if (D == 128) return run_bwd<128>(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, scale, g, idx, parts, s);
    return run_bwd<64>(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, scale, g, idx, parts, s);
}

}  // namespace sta
