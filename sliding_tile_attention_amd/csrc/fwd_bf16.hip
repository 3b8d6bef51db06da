// Fused sliding-tile attention forward, bf16 in / fp32 accumulate, gfx950.
//
// Operator ("Fast Video Generation with Sliding Tile Attention", abstract):
// each query tile attends only to the key/value tiles of its 3D window.  The
// mask is tile-granular, so a workgroup that owns rows of one query tile
// walks that tile's key-tile list and never masks inside a tile.
//
// Two launches:
//   1. vt_kernel: V^T of every tile (and text pseudo-tile), [b,h,tile][D][Lp]
//      with the key axis padded with zeros to Lp (a multiple of the key
//      block), into a stream-ordered workspace.  Every V tile is read by ~45 query tiles'
//      workgroups, so transposing it once lets the PV product fetch its
//      operand with full-width LDS reads instead of transposing reads,
//      which move half the bytes per LDS instruction -- the LDS port, not
//      the matrix cores, is what bounds this kernel.
//   2. fwd_bf16_kernel, below.
//
// Joint text + video sequences (MOD-DiT README, "Token-Type-Aware
// Masking"): after its listed tiles a video query tile walks the text
// pseudo-tiles; a text pseudo-tile's queries walk every video tile and then
// the text.  Key rows past a pseudo-tile's ragged end are masked like
// those past any block end.
//
// Work decomposition
//   workgroup = NW waves = M = NW*QB*32 consecutive query rows of one query
//   tile of one (b, h); work items are ordered head-major and each of the 8
//   XCDs takes one contiguous range of that order, cut at equal cost
//   (schedule.hip), so that the workgroups sharing an XCD's L2 walk
//   neighbouring windows of the same head.
//   The key loop runs over (listed key tile, BN-key block) pairs.  K and V^T
//   blocks travel HBM -> LDS directly (global_load_lds, no staging
//   registers) into a double buffer: the copy of block j+1 runs while block j
//   is computed; one barrier per block.
//
// Per wave and 32-row query block (lane l owns query row l%32):
//   S^T[BN x 32] = K_blk Q^T    (MFMA: A = K rows from LDS, B = Q in VGPRs)
//   online softmax along the key axis, in base 2 with scale*log2(e) folded
//   into one FMA; the running max is only moved when a block max exceeds it
//   by more than 8 (2^8 headroom), which leaves the result exact and skips
//   almost every rescale of the O accumulator;
//   O^T[D x 32] += V^T_blk P^T  (MFMA: A = V^T rows from LDS, B = P in VGPRs)
// K rows are fed permuted by sigma so that each lane's S^T registers hold 8
// consecutive keys -- the B operand of the PV product without any shuffle.
//
// LDS layout: the K block is row-major [BN][D], the V^T block [D][BN]; the
// 16-byte granules of each row are XOR-swizzled (granule c of row r stored
// at c ^ f(r)) so that 16 lanes reading 16 consecutive rows at one logical
// granule touch 16 distinct 16-byte bank groups -- conflict free, no padding.
#include <type_traits>

#include "common.h"
#include "mfma.h"

namespace sta {

template <int D, int NW, int QB, int BN>
struct FwdCfg {
    static constexpr int THREADS = NW * 64;
    static constexpr int M = NW * QB * 32;     // query rows per workgroup
    static constexpr int KS = D / 16;           // reduction steps of QK^T
    static constexpr int KB = BN / 32;          // 32-key sub-blocks
    static constexpr int DB = D / 32;           // 32-wide column blocks of O^T
    static constexpr int GR = D / 8;            // 16-byte granules per K row
    static constexpr int GV = BN / 8;           // 16-byte granules per V^T row
    static constexpr int BLK = BN * D;          // bf16 elements of one K (or V^T) block
    static constexpr int STAGE = 2 * BLK;       // K + V^T
    static constexpr int WAVE_ELEMS = 512;      // one wave-wide 16-byte copy = 1 KB
    static constexpr int GRANULES = BLK / 8;    // 16-byte granules of one block
    static constexpr int COPIES = (GRANULES + THREADS - 1) / THREADS;   // copies per thread per block
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
    static_assert(GRANULES % 64 == 0, "a block is a whole number of wave-wide copies");
};

// Swizzle of a row of G 16-byte granules: rows r = 0..15 read at one logical
// granule land in 16 distinct 16-byte slots of a 256-byte bank line.
template <int G>
__device__ inline int swz_row(int r)
{
    if constexpr (G >= 16) return r & 15;
    else return (r / (16 / G)) & (G - 1);
}

#ifndef STA_FWD_MINB
#define STA_FWD_MINB 3
#endif

// Key padding of the V^T workspace (a multiple of every key block size).
constexpr int kVtPad = 64;

template <int D>
__global__ __launch_bounds__(256) void vt_kernel(const __bf16 *__restrict__ V, __bf16 *__restrict__ VT, Geo g,
                                                 int Lp, int chunks)
{
    // one workgroup per 64-key chunk of one (b, h, tile)
    __shared__ uint32_t tile[64][D / 2 + 1];   // 64 keys x D values as bf16 pairs; odd stride: no conflicts
    const int c = (int)(blockIdx.x % (unsigned)chunks);
    const int64_t bt = blockIdx.x / (unsigned)chunks;
    const int64_t bh = bt / g.TT;
    const int t = (int)(bt - bh * g.TT);
    const Span sp = tile_span(g, t);
    const int L = sp.len;
    const int k0 = c * 64;
    const __bf16 *src = V + bh * g.S * D;
    constexpr int RG = D / 8;                 // 16-byte granules per V row
    for (int i = threadIdx.x; i < 64 * RG; i += 256) {
        const int r = i / RG, gc = i % RG;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (k0 + r < L) v = __builtin_nontemporal_load((const u32x4 *)(src + tile_row(g, t, k0 + r) * D + gc * 8));
#pragma unroll
        for (int t = 0; t < 4; ++t) tile[r][gc * 4 + t] = v[t];
    }
    __syncthreads();
    // unit u: column pair p (rows 2p, 2p+1 of V^T), key group kg (8 keys)
    __bf16 *dst = VT + bt * D * Lp + k0;
    for (int u = threadIdx.x; u < (D / 2) * 8; u += 256) {
        const int p = u / 8, kg = u % 8;
        uint32_t w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = tile[kg * 8 + j][p];
        u32x4 lo, hi;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            lo[t] = (w[2 * t] & 0xffffu) | (w[2 * t + 1] << 16);
            hi[t] = (w[2 * t] >> 16) | (w[2 * t + 1] & 0xffff0000u);
        }
        __builtin_nontemporal_store(lo, (u32x4 *)(dst + (int64_t)(2 * p) * Lp + kg * 8));
        __builtin_nontemporal_store(hi, (u32x4 *)(dst + (int64_t)(2 * p + 1) * Lp + kg * 8));
    }
}

// RASTER: q, k, o, lse in raster order (whole tiles; rows of a video tile
// gathered by tile_row, K blocks by a per-lane raster pattern).
template <int D, int NW, int QB, int BN, bool RASTER>
__global__ __launch_bounds__(NW * 64, STA_FWD_MINB) void fwd_bf16_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ VT,
    __bf16 *__restrict__ O, float *__restrict__ LSE, const int32_t *__restrict__ kv_idx,
    const int32_t *__restrict__ kv_cnt, int max_kv, int IH, Geo g, int Lp, int rblocks, const int *__restrict__ split,
    float scale_log2)
{
    using C = FwdCfg<D, NW, QB, BN>;
    __shared__ __attribute__((aligned(1024))) __bf16 smem[2 * C::STAGE];

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
    if (rb * C::M >= qlen) return;                   // row block past a cut tile's end
    const int h = bh % IH;                           // list set: the head's, or (b, h)'s
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, grp = lane >> 5;
    const int64_t base = (int64_t)bh * g.S * D;
    const int64_t vt_base = (int64_t)bh * g.TT * D * Lp;
    const int wrow0 = rb * C::M + wave * QB * 32;   // first row of this wave inside the tile

    // Q fragments: B operand of S^T = K Q^T, lane = query row, 8 columns.
    bf16x8 qf[QB][C::KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = wrow0 + qb * 32 + l32;
        const __bf16 *p = Q + base + slab_row<RASTER>(g, qt, qs, row) * D + grp * 8;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qf[qb][ks] = row < qlen ? ld8(p + ks * 16) : zero8();
    }

    f32x16 acc[QB][C::DB];
    float m_i[QB], l_i[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_i[qb] = -INFINITY;
        l_i[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qb][db][r] = 0.f;
    }

    // key tiles: the window's list, or every video tile for a text query
    const bool video_q = qt < g.T;
    const int cnt = video_q ? kv_cnt[(int64_t)h * g.T + qt] : g.T;
    const int32_t *lst = video_q ? kv_idx + ((int64_t)h * g.T + qt) * max_kv : nullptr;
    const int nblk = walk_blocks(g, lst, cnt, BN);

    // ---- per-lane offsets (bf16 elements), fixed for the whole kernel ----
    // Copies: wave-wide copy i of a block fills granule slots
    // (i*NW + wave)*64 + lane, i.e. row r = slot / (granules per row) and
    // physical granule p, which must receive logical granule p ^ f(r).
    int gk[C::COPIES], gv[C::COPIES];     // byte offsets inside a K block / V^T tile
    int gkr[RASTER ? C::COPIES : 1];      // raster: K row r of a video block sits raster_step(r) rows on
#pragma unroll
    for (int i = 0; i < C::COPIES; ++i) {
        const int slot = (i * NW + wave) * 64 + lane;
        const int r = slot / C::GR, pg = slot % C::GR;
        gk[i] = (r * D + (pg ^ swz_row<C::GR>(r)) * 8) * 2;
        if constexpr (RASTER) gkr[i] = (raster_step_p2(g, r) * D + (pg ^ swz_row<C::GR>(r)) * 8) * 2;
        const int rv = slot / C::GV, pv = slot % C::GV;
        gv[i] = (rv * Lp + (pv ^ swz_row<C::GV>(rv)) * 8) * 2;
    }
    // A copy slot past the block (workgroups whose thread count does not
    // divide the block) is skipped; the test is uniform per wave.
    auto copy_live = [&](int i) { return C::GRANULES % C::THREADS == 0 || (i * NW + wave) * 64 < C::GRANULES; };
    // S^T operand: lane feeds K row sigma(l%32) of each 32-key sub-block;
    // the swizzle of that row does not depend on the sub-block.
    const int arow = sigma32(l32);
    int kofs[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kofs[ks] = arow * D + ((2 * ks + grp) ^ swz_row<C::GR>(arow)) * 8;
    // PV operand: lane feeds V^T row d = db*32 + l%32, keys kb*32 + kk*16 +
    // 8*grp .. +7, i.e. logical granule 4kb + 2kk + grp of that row; the
    // swizzle depends only on l%32.
    int vofs[C::KB][2];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            vofs[kb][kk] = l32 * BN + (((4 * kb + 2 * kk + grp) ^ swz_row<C::GV>(l32)) << 3);

    // The key-block stream is walked with counters (no divisions): the
    // copy stream is one block ahead of the compute stream; the next tile
    // id of the list is prefetched when a tile is entered.
    int c_e = 0, c_k0 = 0;                               // next block to copy
    int c_tile = entry_tile(lst, cnt, g.T, 0);
    Span c_sp = tile_span(g, c_tile);
    int n_tile = entry_tile(lst, cnt, g.T, 1);
    int bvalid[2];                                       // valid keys of the block in each buffer
    static_assert(!RASTER || BN == 32, "raster walk of 32-row blocks");
    int c_roff = RASTER ? (int)raster_base(g, c_tile) : 0;   // raster row of the block (video tiles only)
    // Issue the asynchronous copy of the next block into LDS buffer `buf`
    // through buffer descriptors over that block: K rows past a ragged
    // tile end read as zero (their scores are masked), V^T keys past it are
    // the workspace's zero padding.
    auto gload = [&](int buf) {
        const int valid = c_sp.len - c_k0 < BN ? c_sp.len - c_k0 : BN;
        bvalid[buf] = valid;
        const auto rv = make_rsrc(VT + vt_base + (int64_t)c_tile * D * Lp + c_k0, (D * Lp - c_k0) * 2);
        __bf16 *Ks = smem + buf * C::STAGE;
        __bf16 *Vs = Ks + C::BLK;
        if (RASTER) {
            // whole video tile (no text rows in the raster layout): every row
            // of the block exists; the descriptor spans the block's rows
            // (g.rs_span from its first)
            const auto rk = make_rsrc(K + base + (int64_t)c_roff * D, g.rs_span * D * 2);
#pragma unroll
            for (int i = 0; i < C::COPIES; ++i) {
                if (!copy_live(i)) continue;
                const int lds_off = (i * NW + wave) * C::WAVE_ELEMS;
                b2lds16(rk, gkr[RASTER ? i : 0], Ks + lds_off);
                b2lds16(rv, gv[i], Vs + lds_off);
            }
        } else {
            const auto rk = make_rsrc(K + base + (c_sp.start + c_k0) * D, valid * D * 2);
#pragma unroll
            for (int i = 0; i < C::COPIES; ++i) {
                if (!copy_live(i)) continue;
                const int lds_off = (i * NW + wave) * C::WAVE_ELEMS;
                b2lds16(rk, gk[i], Ks + lds_off);
                b2lds16(rv, gv[i], Vs + lds_off);
            }
        }
        c_k0 += BN;
        if constexpr (RASTER) {          // the walk of g.rs_*: no divisions per block
            c_roff += g.rs_step;
            if ((c_k0 & g.rs_pmask) == 0) c_roff += g.rs_jump;
        }
        if (c_k0 >= c_sp.len) {
            c_k0 = 0;
            ++c_e;
            c_tile = n_tile;
            c_sp = tile_span(g, c_tile);
            n_tile = entry_tile(lst, cnt, g.T, c_e + 1);
            if constexpr (RASTER) c_roff = (int)raster_base(g, c_tile);
        }
    };

    // One key block from LDS buffer BUF (a compile-time constant, so every
    // LDS address below is a per-lane register plus an immediate).
    auto step = [&](auto bufc, int blk) {
        constexpr int BUF = decltype(bufc)::value;
        __builtin_amdgcn_s_waitcnt(0);     // this wave's copies of block blk have landed
        __syncthreads();                   // ... and everyone's; the other buffer is free
        const int valid = bvalid[BUF];
        if (blk + 1 < nblk) gload(1 - BUF);
        const __bf16 *Ks = smem + BUF * C::STAGE;
        const __bf16 *Vs = Ks + C::BLK;

        f32x16 s[QB][C::KB];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const bf16x8 a = ld8(Ks + kb * 32 * D + kofs[ks]);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32(a, qf[qb][ks], s[qb][kb]);
            }
        }

        // Probabilities, rounded to bf16 (the PV operand), and their sum.
        // Exponents use the running max m_i; a block whose partial sum stays
        // below 2^8 cannot overflow and is accepted as is.  Otherwise (first
        // block, or scores that jumped) the true max is taken, O and l are
        // rescaled, and the block is recomputed.
        bf16x8 pf[QB][C::KB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if (valid < BN) {
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kb * 32 + mfma_row_sigma(lane, r) >= valid) s[qb][kb][r] = -INFINITY;
            }
            auto probs = [&]() {
                const float mneg = -m_i[qb];
                float ls = 0.f;
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        bf16x8 v;
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            v[i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[qb][kb][8 * hf + i], scale_log2, mneg));
                        pf[qb][kb][hf] = v;
                        ls = sum8(v, ls);
                    }
                return ls;
            };
            float ls = probs();
            if (__any(!(ls < 256.f))) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
                mx = max_pair32(mx) * scale_log2;
                const float mn = fmaxf(m_i[qb], mx);
                const float alpha = __builtin_amdgcn_exp2f(m_i[qb] - mn);
                m_i[qb] = mn;
                l_i[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
                ls = probs();
            }
            l_i[qb] += ls;
        }

#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 a = ld8(Vs + db * 32 * BN + vofs[kb][kk]);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32(a, pf[qb][kb][kk], acc[qb][db]);
                }
    };

    if (nblk > 0) gload(0);
    for (int blk = 0; blk < nblk; blk += 2) {
        step(std::integral_constant<int, 0>{}, blk);
        if (blk + 1 < nblk) step(std::integral_constant<int, 1>{}, blk + 1);
    }

    // Epilogue: lanes l and l^32 hold the two halves of row l%32's sum.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = sum_pair32(l_i[qb]);
        const float inv = 1.f / lt;
        const int row = wrow0 + qb * 32 + l32;
        if (row < qlen) {
            const int64_t orow = slab_row<RASTER>(g, qt, qs, row);
            __bf16 *op = O + base + orow * D;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bf16x4 v;
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = (__bf16)(acc[qb][db][4 * j + t] * inv);
                    *(bf16x4 *)(op + db * 32 + 8 * j + 4 * grp) = v;
                }
            if (grp == 0)
                LSE[(int64_t)bh * g.S + orow] = (m_i[qb] + __log2f(lt)) * 0.69314718055994531f;
        }
    }
}

// V^T workspace + transpose, then the attention kernel.
template <int D, int NW, int QB, int BN>
static sta_status run_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                          float scale, const Geo &g, const sta_index &idx, hipStream_t s)
{
    using C = FwdCfg<D, NW, QB, BN>;
    static_assert(kVtPad % BN == 0, "V^T padding must be a multiple of the key block");
    const int rblocks = (g.L + C::M - 1) / C::M;
    const int64_t total = (int64_t)B * H * g.TT * rblocks;
    const int64_t blocks = work_blocks(total);
    const int chunks = (g.L + kVtPad - 1) / kVtPad;
    const int Lp = chunks * kVtPad;
    const int64_t vt_blocks = (int64_t)B * H * g.TT * chunks;
    if (!grid_fits(blocks, C::THREADS) || !grid_fits(vt_blocks, 256))
        return fail(STA_ERR_UNSUPPORTED, "too many work items");
    // workspace: the per-XCD work split, then the V^T tiles
    const size_t plan = (plan_bytes(idx.num_heads, (int64_t)B * H) + 255) & ~(size_t)255;
    const size_t vt_bytes = (size_t)B * H * g.TT * D * Lp * sizeof(__bf16);
    void *ws = nullptr;
    sta_status st = workspace_alloc(&ws, plan + vt_bytes, s);
    if (st != STA_OK) return st;
    void *vt = (char *)ws + plan;
    const int *split = nullptr;
    if ((st = plan_work(g, idx.kv_cnt, idx.num_heads, (int64_t)B * H, rblocks, blocks, ws, s, &split)) != STA_OK) {
        (void)workspace_free(ws, s);          // the launch error is the one reported
        return st;
    }
    hipLaunchKernelGGL(vt_kernel<D>, dim3((unsigned)vt_blocks), dim3(256), 0, s, (const __bf16 *)v, (__bf16 *)vt,
                       g, Lp, chunks);
    const float scale_log2 = scale * 1.4426950408889634f;
    if (g.raster)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, QB, BN, true>), dim3((unsigned)blocks), dim3(C::THREADS), 0, s,
                           (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)vt, (__bf16 *)o, lse, idx.kv_idx,
                           idx.kv_cnt, idx.max_kv, idx.num_heads, g, Lp, rblocks, split, scale_log2);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, QB, BN, false>), dim3((unsigned)blocks), dim3(C::THREADS), 0, s,
                           (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)vt, (__bf16 *)o, lse, idx.kv_idx,
                           idx.kv_cnt, idx.max_kv, idx.num_heads, g, Lp, rblocks, split, scale_log2);
    st = check_launch();
    const sta_status fs = workspace_free(ws, s);
    return st != STA_OK ? st : fs;
}

// Tile shape: waves per workgroup, 32-row query blocks per wave, keys per
// LDS block.  Overridable at compile time for tuning sweeps.
#ifndef STA_FWD_NW
#define STA_FWD_NW 4
#endif
#ifndef STA_FWD_QB
#define STA_FWD_QB 1
#endif
#ifndef STA_FWD_BN
#define STA_FWD_BN 32
#endif

sta_status launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                           int D, float scale, const Geo &g, const sta_index &idx, hipStream_t s)
{
    if (D == 128) return run_fwd<128, STA_FWD_NW, STA_FWD_QB, STA_FWD_BN>(q, k, v, o, lse, B, H, scale, g, idx, s);
    return run_fwd<64, STA_FWD_NW, STA_FWD_QB, STA_FWD_BN>(q, k, v, o, lse, B, H, scale, g, idx, s);
}

}  // namespace sta
