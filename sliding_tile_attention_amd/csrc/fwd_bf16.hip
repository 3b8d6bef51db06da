// Fused sliding-tile attention forward, bf16 in / fp32 accumulate, gfx950.
//
// Operator ("Fast Video Generation with Sliding Tile Attention", abstract):
// each query tile attends only to the key/value tiles of its 3D window.  The
// mask is tile-granular, so a workgroup that owns rows of one query tile
// walks that tile's key-tile list and never masks inside a tile.
//
// Work decomposition
//   workgroup = NW waves = M = NW*QB*32 consecutive query rows of one query
//   tile of one (b, h); work items are ordered head-major and spread over the
//   8 XCDs in contiguous ranges (xcd_remap) so that the workgroups sharing an
//   XCD's L2 walk neighbouring windows of the same head.
//   The key loop runs over (listed key tile, BN-key block) pairs.  K and V of
//   the next block are fetched into registers while the current block is
//   computed from LDS (double buffer, one barrier per block).
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
// V is stored transposed in LDS (D rows of BN keys), so the A operand of the
// PV product is one 16-byte LDS read.  Rows of both LDS tiles are padded by
// 16 bytes, which makes the 16-byte fragment reads bank-conflict free.
#include "common.h"
#include "mfma.h"

namespace sta {

template <int D, int NW, int QB, int BN>
struct FwdCfg {
    static constexpr int THREADS = NW * 64;
    static constexpr int M = NW * QB * 32;    // query rows per workgroup
    static constexpr int KS = D / 16;          // reduction steps of QK^T
    static constexpr int KB = BN / 32;         // 32-key sub-blocks
    static constexpr int DB = D / 32;          // 32-wide column blocks of O^T
    static constexpr int KP = D + 8;           // LDS row pitch of K (bf16)
    static constexpr int VP = BN + 8;          // LDS row pitch of V^T (bf16)
    static constexpr int KE = BN * KP;
    static constexpr int VE = D * VP;
    static constexpr int STAGE = KE + VE;      // one buffer, bf16 elements
    static constexpr int KCH = BN * D / 8;     // 16-byte chunks of a K block
    static constexpr int VCH = (BN / 4) * (D / 8);  // 4-key x 8-column chunks of V
    static constexpr int KPT = (KCH + THREADS - 1) / THREADS;
    static constexpr int VPT = (VCH + THREADS - 1) / THREADS;
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
};

template <int D, int NW, int QB, int BN>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(
    const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
    __bf16 *__restrict__ O, float *__restrict__ LSE, const int32_t *__restrict__ kv_idx,
    const int32_t *__restrict__ kv_cnt, int max_kv, int H, Geo g, int rblocks, int total,
    float scale_log2)
{
    using C = FwdCfg<D, NW, QB, BN>;
    __shared__ __attribute__((aligned(16))) __bf16 smem[2 * C::STAGE];

    const int work = xcd_remap(blockIdx.x, total);
    const int rb = work % rblocks;
    const int qt = (work / rblocks) % g.T;
    const int bh = work / (rblocks * g.T);
    const int h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, grp = lane >> 5;
    const int L = g.L;
    const int64_t base = (int64_t)bh * g.N * D;
    const int wrow0 = rb * C::M + wave * QB * 32;   // first row of this wave inside the tile

    // Q fragments: B operand of S^T = K Q^T, lane = query row, 8 columns.
    bf16x8 qf[QB][C::KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = wrow0 + qb * 32 + l32;
        const __bf16 *p = Q + base + ((int64_t)qt * L + row) * D + grp * 8;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qf[qb][ks] = row < L ? ld8(p + ks * 16) : zero8();
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

    const int cnt = kv_cnt[(int64_t)h * g.T + qt];
    const int32_t *lst = kv_idx + ((int64_t)h * g.T + qt) * max_kv;
    const int nkb = (L + BN - 1) / BN;
    const int nblk = cnt * nkb;

    u32x4 kreg[C::KPT];
    u32x4 vreg[C::VPT][4];

    auto gload = [&](int blk) {
        const int e = blk / nkb;
        const int k0 = (blk - e * nkb) * BN;
        const int valid = L - k0 < BN ? L - k0 : BN;
        const int64_t kbase = base + ((int64_t)lst[e] * L + k0) * D;
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int c = tid + i * C::THREADS;
            const int row = c / (D / 8), col = c % (D / 8);
            const bool ok = c < C::KCH && row < valid;
            kreg[i] = ok ? *(const u32x4 *)(K + kbase + (int64_t)row * D + col * 8) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < C::VPT; ++i) {
            const int c = tid + i * C::THREADS;
            const int kg = c % (BN / 4), dg = c / (BN / 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = kg * 4 + r;
                const bool ok = c < C::VCH && key < valid;
                vreg[i][r] = ok ? *(const u32x4 *)(V + kbase + (int64_t)key * D + dg * 8) : (u32x4){0u, 0u, 0u, 0u};
            }
        }
    };
    auto swrite = [&](int buf) {
        __bf16 *Ks = smem + buf * C::STAGE;
        __bf16 *Vs = Ks + C::KE;
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int c = tid + i * C::THREADS;
            if (c < C::KCH) *(u32x4 *)(Ks + (c / (D / 8)) * C::KP + (c % (D / 8)) * 8) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < C::VPT; ++i) {
            const int c = tid + i * C::THREADS;
            if (c < C::VCH) {
                const int kg = c % (BN / 4), dg = c / (BN / 4);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    *(u32x2 *)(Vs + (dg * 8 + j) * C::VP + kg * 4) =
                        column4(vreg[i][0], vreg[i][1], vreg[i][2], vreg[i][3], j);
            }
        }
    };

    if (nblk > 0) {
        gload(0);
        swrite(0);
    }
    __syncthreads();

    const int arow = sigma32(l32);   // K row this lane feeds to the S^T MFMA
    for (int blk = 0; blk < nblk; ++blk) {
        if (blk + 1 < nblk) gload(blk + 1);
        const __bf16 *Ks = smem + (blk & 1) * C::STAGE;
        const __bf16 *Vs = Ks + C::KE;
        const int k0 = (blk % nkb) * BN;
        const int valid = L - k0 < BN ? L - k0 : BN;

        f32x16 s[QB][C::KB];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const bf16x8 a = ld8(Ks + (kb * 32 + arow) * C::KP + ks * 16 + grp * 8);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32(a, qf[qb][ks], s[qb][kb]);
            }
        }

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
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
            mx = fmaxf(mx, xor32(mx)) * scale_log2;
            if (__any(mx > m_i[qb] + 8.f)) {
                const float mn = fmaxf(m_i[qb], mx);
                const float alpha = __builtin_amdgcn_exp2f(m_i[qb] - mn);
                m_i[qb] = mn;
                l_i[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
            }
            const float mneg = -m_i[qb];
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r], scale_log2, mneg));
                    s[qb][kb][r] = p;
                    ls += p;
                }
                pf[qb][kb][0] = cvt8(s[qb][kb], 0);
                pf[qb][kb][1] = cvt8(s[qb][kb], 8);
            }
            l_i[qb] += ls;
        }

#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 a = ld8(Vs + (db * 32 + l32) * C::VP + kb * 32 + kk * 16 + grp * 8);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma32(a, pf[qb][kb][kk], acc[qb][db]);
                }

        if (blk + 1 < nblk) swrite((blk + 1) & 1);
        __syncthreads();
    }

    // Epilogue: lanes l and l^32 hold the two halves of row l%32's sum.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = l_i[qb] + xor32(l_i[qb]);
        const float inv = 1.f / lt;
        const int row = wrow0 + qb * 32 + l32;
        if (row < L) {
            __bf16 *op = O + base + ((int64_t)qt * L + row) * D;
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
                LSE[(int64_t)bh * g.N + (int64_t)qt * L + row] = (m_i[qb] + __log2f(lt)) * 0.69314718055994531f;
        }
    }
}

template <int D, int NW, int QB, int BN>
static sta_status run_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                          float scale, const Geo &g, const sta_index &idx, hipStream_t s)
{
    using C = FwdCfg<D, NW, QB, BN>;
    const int rblocks = (g.L + C::M - 1) / C::M;
    const int64_t total = (int64_t)B * H * g.T * rblocks;
    if (total >= ((int64_t)1 << 31))
        return fail(STA_ERR_UNSUPPORTED, "too many work items");
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, QB, BN>), dim3((unsigned)total), dim3(C::THREADS), 0, s,
                       (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (__bf16 *)o, lse, idx.kv_idx,
                       idx.kv_cnt, idx.max_kv, H, g, rblocks, (int)total, scale_log2);
    return check_launch();
}

sta_status launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                           int D, float scale, const Geo &g, const sta_index &idx, hipStream_t s)
{
    if (D == 128) return run_fwd<128, 4, 1, 64>(q, k, v, o, lse, B, H, scale, g, idx, s);
    return run_fwd<64, 4, 1, 64>(q, k, v, o, lse, B, H, scale, g, idx, s);
}

}  // namespace sta
