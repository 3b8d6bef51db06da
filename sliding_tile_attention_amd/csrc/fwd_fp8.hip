// Quantized sliding-tile attention forward, gfx950: INT8 QK^T and FP8 (e4m3)
// PV on the matrix cores, bf16 in / bf16 out, fp32 softmax.
//
// Quantized attention kernels appear on the pages only as a dependency of
// one of them (MOD-DiT README, "Project Structure": the SageAttention
// submodule); this scheme is the library's own:
//   1. per (b, h): K smoothed by its mean over the rows (every score of a
//      query moves by the same amount: the softmax is unchanged; the LSE
//      gets scale * <q, mean> back), V scaled per channel to e4m3's range;
//   2. Q int8 codes per row, K int8 codes per 64-key block of a tile;
//   3. S^T = K Q^T on v_mfma_i32_32x32x32_i8 (exact int32 sums), scaled by
//      the row and block scales into base-2 logits;
//   4. P = 2^(s - m + 4) rounded to e4m3, O^T += V^T P^T on
//      v_mfma_scale_f32_32x32x64_f8f6f4, the row sum taken from the rounded
//      P.  The running max m only takes integer values, so every rescale is
//      an exact power of two and P's e4m3 rounding commutes with it (normal
//      range): the result is that of rounding 2^(s - ceil(max s) + 4), which
//      keeps probabilities down to 2^-10 of the row's largest in e4m3's
//      normal range.
// Both products run at twice the bf16 rate per cycle, and both operands
// are one byte per element, so a 64-key block costs the LDS traffic and
// matrix-core time of a 32-key bf16 block.
//
// Launches: statistics (two passes, fixed reduction order: deterministic),
// Q/K codes, V^T codes (per tile [D][Lp], each 64-key group permuted so
// that the 32 bytes a lane half feeds the PV product are contiguous), then
// the attention kernel.  The work decomposition, list walk, copies and
// swizzles are those of the bf16 forward.
#include <cfloat>
#include <type_traits>

#include "common.h"
#include "mfma.h"

namespace sta {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kKeyBlock = 64;       // keys per LDS block and per K scale
constexpr int kStatChunks = 64;     // row chunks per (b, h) in the statistics pass
constexpr float kE4M3Max = 448.f;

// Swizzle of a row of G 16-byte granules (see the bf16 forward).
template <int G>
__device__ inline int swz8(int r)
{
    if constexpr (G >= 16) return r & 15;
    else return (r / (16 / G)) & (G - 1);
}

// 1a. Partial column sums of K in fp64 (a bf16 value is added exactly while
// the sum stays below 2^45 times its magnitude, so the mean, rounded once to
// fp32, is that of the exact mean unless the two straddle an fp32 rounding
// boundary) and column maxima of |V| over one chunk of the rows of one
// (b, h): part[bh][chunk][0 = sum K, 1 = max |V|][D].
template <int D>
__global__ __launch_bounds__(256) void qstat_kernel(const __bf16 *__restrict__ K, const __bf16 *__restrict__ V,
                                                    double *__restrict__ part, int64_t S)
{
    constexpr int TPR = D / 8;          // threads per row, 8 columns (16 bytes) each
    constexpr int RG = 256 / TPR;       // row groups
    __shared__ double red[2][RG][D];
    const int chunk = (int)(blockIdx.x % kStatChunks);
    const int64_t bh = blockIdx.x / kStatChunks;
    const int cg = threadIdx.x % TPR, rg = threadIdx.x / TPR;
    const int64_t r0 = S * chunk / kStatChunks, r1 = S * (chunk + 1) / kStatChunks;
    const __bf16 *kb = K + bh * S * D + 8 * cg, *vb = V + bh * S * D + 8 * cg;
    double sum[8];
    float mx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        sum[j] = 0.0;
        mx[j] = 0.f;
    }
    for (int64_t r = r0 + rg; r < r1; r += RG) {
        const bf16x8 k8 = ld8(kb + r * D);
        const bf16x8 v8 = ld8(vb + r * D);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            sum[j] += (double)(float)k8[j];
            mx[j] = fmaxf(mx[j], fabsf((float)v8[j]));
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        red[0][rg][8 * cg + j] = sum[j];
        red[1][rg][8 * cg + j] = mx[j];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 2 * D; i += 256) {
        const int w = i / D, d = i % D;
        double a = red[w][0][d];
        for (int j = 1; j < RG; ++j) a = w ? fmax(a, red[w][j][d]) : a + red[w][j][d];
        part[((bh * kStatChunks + chunk) * 2 + w) * D + d] = a;
    }
}

// 1b. Per (b, h, d): the smoothing mean of K (the fp64 sum over the rows
// divided by their count, rounded once to fp32) and V's channel scale.
template <int D>
__global__ __launch_bounds__(256) void qstat_final_kernel(const double *__restrict__ part, float *__restrict__ kmean,
                                                          float *__restrict__ vscale, float *__restrict__ vinv,
                                                          int64_t S, int BH)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= BH * D) return;
    const int64_t bh = i / D;
    const int d = i % D;
    double s = 0.0;
    float m = 0.f;
    for (int c = 0; c < kStatChunks; ++c) {
        s += part[((bh * kStatChunks + c) * 2 + 0) * D + d];
        m = fmaxf(m, (float)part[((bh * kStatChunks + c) * 2 + 1) * D + d]);
    }
    kmean[i] = (float)(s / (double)S);
    vscale[i] = m / kE4M3Max;
    vinv[i] = m > 0.f ? kE4M3Max / m : 0.f;
}

// rint(x * inv) as a byte (|x * inv| <= 127 by construction).
__device__ inline unsigned i8code(float x, float inv) { return (unsigned)(int)rintf(x * inv) & 0xffu; }

// 2. Q and K codes: one workgroup per 64-row block of one tile (or text
// pseudo-tile) of one (b, h); 4 threads per row.  Q: per-row scale folded
// with scale * log2(e) (sq) and the LSE correction scale * <q, mean K>
// (corr); K - mean: one scale per block (sk[bh][tile][block]).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int D>
__global__ __launch_bounds__(256) void quant_qk_kernel(const __bf16 *__restrict__ Q, const __bf16 *__restrict__ K,
                                                       const float *__restrict__ kmean, uint8_t *__restrict__ Q8,
                                                       uint8_t *__restrict__ K8, float *__restrict__ sq,
                                                       float *__restrict__ corr, float *__restrict__ sk, Geo g,
                                                       int nkb, float c_log2, float scale)
{
    // TPR threads per row, 8 consecutive values (16 bytes) each, so that the
    // lanes of a wave read whole rows with consecutive 16-byte loads; the
    // 64 rows of the block are taken PASSES at a time.
    constexpr int TPR = D / 8, RPP = 256 / TPR, PASSES = kKeyBlock / RPP;
    static_assert(kKeyBlock % RPP == 0, "block of whole passes");
    __shared__ float wmax[4];
    const int blk = (int)(blockIdx.x % nkb);
    const int64_t bt = blockIdx.x / nkb;
    const int64_t bh = bt / g.TT;
    const int t = (int)(bt - bh * g.TT);
    const Span sp = tile_span(g, t);
    const int rows = sp.len - blk * kKeyBlock < kKeyBlock ? sp.len - blk * kKeyBlock : kKeyBlock;
    if (rows <= 0) return;                           // block past a cut tile's end (uniform)
    const int part = threadIdx.x % TPR;
    const float *mk = kmean + bh * D + part * 8;
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = mk[j];
    float k[PASSES][8];
    float ka = 0.f;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int r = ps * RPP + threadIdx.x / TPR;
        const bool live = r < rows;
        // codes, scales: tile order (the attention kernel's); inputs: the layout's rows
        const int64_t row = bh * g.S + sp.start + (int64_t)blk * kKeyBlock + (live ? r : 0);
        const int64_t src = bh * g.S + tile_row(g, t, blk * kKeyBlock + (live ? r : 0));
        bf16x8 a = zero8(), b = zero8();
        if (live) {
            a = ld8(Q + src * D + part * 8);
            b = ld8(K + src * D + part * 8);
        }
        float q[8];
        float qa = 0.f, dq = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            q[j] = (float)a[j];
            k[ps][j] = live ? (float)b[j] - m[j] : 0.f;
            qa = fmaxf(qa, fabsf(q[j]));
            ka = fmaxf(ka, fabsf(k[ps][j]));
            dq = fmaf(q[j], m[j], dq);
        }
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) {
            qa = fmaxf(qa, __shfl_xor(qa, o, 64));
            dq += __shfl_xor(dq, o, 64);
        }
        const float qinv = qa > 0.f ? 127.f / qa : 0.f;
        if (live) {
            u32x2 wq;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                wq[j] = i8code(q[4 * j], qinv) | i8code(q[4 * j + 1], qinv) << 8 | i8code(q[4 * j + 2], qinv) << 16 |
                        i8code(q[4 * j + 3], qinv) << 24;
            *(u32x2 *)(Q8 + row * D + part * 8) = wq;
            if (part == 0) {
                sq[row] = qa / 127.f * c_log2;
                corr[row] = scale * dq;
            }
        }
    }
    // the block's K scale: max |k - mean| over its rows
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) ka = fmaxf(ka, __shfl_xor(ka, o, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = ka;
    __syncthreads();
    ka = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float kinv = ka > 0.f ? 127.f / ka : 0.f;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int r = ps * RPP + threadIdx.x / TPR;
        if (r < rows) {
            const int64_t row = bh * g.S + sp.start + (int64_t)blk * kKeyBlock + r;
            u32x2 wk;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                wk[j] = i8code(k[ps][4 * j], kinv) | i8code(k[ps][4 * j + 1], kinv) << 8 |
                        i8code(k[ps][4 * j + 2], kinv) << 16 | i8code(k[ps][4 * j + 3], kinv) << 24;
            *(u32x2 *)(K8 + row * D + part * 8) = wk;
        }
    }
    if (threadIdx.x == 0) sk[bh * ((int64_t)g.TT * nkb) + (int64_t)t * nkb + blk] = ka / 127.f;
}

// Position of key k of a 64-key group in the permuted V^T row: lane half g
// of the PV operand reads bytes 32g .. 32g+31, byte b holding key
// 32(b/16) + 16((b%16)/8) + 8g + b%8 -- the key order of the P bytes that
// lane half builds from its S^T registers.
__device__ inline int vt_key_of(int pos)
{
    const int gg = pos >> 5, b = pos & 31;
    return 32 * (b >> 4) + 16 * ((b >> 3) & 1) + 8 * gg + (b & 7);
}

// 3. V^T codes: one workgroup per 64-key chunk of one (b, h, tile):
// e4m3(v * 448 / max|v_d|) transposed to [D][Lp] (keys past the tile's end
// zero), each 64-key group in the permuted order above.
template <int D>
__global__ __launch_bounds__(256) void quant_vt_kernel(const __bf16 *__restrict__ V, const float *__restrict__ vinv,
                                                       uint8_t *__restrict__ VT8, Geo g, int Lp, int chunks)
{
    __shared__ float tv[kKeyBlock][D + 1];
    const int c = (int)(blockIdx.x % chunks);
    const int64_t bt = blockIdx.x / chunks;
    const int64_t bh = bt / g.TT;
    const int t = (int)(bt - bh * g.TT);
    const Span sp = tile_span(g, t);
    const int k0 = c * kKeyBlock;
    const __bf16 *src = V + bh * g.S * D;
    const float *vi = vinv + bh * D;
    for (int i = threadIdx.x; i < kKeyBlock * D / 8; i += 256) {
        const int r = i / (D / 8), gc = i % (D / 8);
        bf16x8 v = zero8();
        if (k0 + r < sp.len) v = ld8(src + tile_row(g, t, k0 + r) * D + gc * 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) tv[r][gc * 8 + j] = (float)v[j] * vi[gc * 8 + j];
    }
    __syncthreads();
    uint8_t *dst = VT8 + bt * D * Lp + k0;
    for (int u = threadIdx.x; u < D * 4; u += 256) {
        const int d = u >> 2, qq = u & 3;
        u32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p0 = 16 * qq + 4 * j;
            int x = __builtin_amdgcn_cvt_pk_fp8_f32(tv[vt_key_of(p0)][d], tv[vt_key_of(p0 + 1)][d], 0, false);
            x = __builtin_amdgcn_cvt_pk_fp8_f32(tv[vt_key_of(p0 + 2)][d], tv[vt_key_of(p0 + 3)][d], x, true);
            w[j] = (unsigned)x;
        }
        *(u32x4 *)(dst + (int64_t)d * Lp + 16 * qq) = w;
    }
}

template <int D, int NW>
struct F8Cfg {
    static constexpr int THREADS = NW * 64;
    static constexpr int M = NW * 32;              // query rows per workgroup
    static constexpr int BN = kKeyBlock;           // keys per block
    static constexpr int KS = D / 32;              // int8 steps of QK^T (32 d each)
    static constexpr int DB = D / 32;              // 32-row blocks of O^T
    static constexpr int GK = D / 16;              // 16-byte granules per K row
    static constexpr int GV = BN / 16;             // 16-byte granules per V^T row
    static constexpr int KBYTES = BN * D;
    static constexpr int STAGE = 2 * KBYTES;       // K block + V^T block
    static constexpr int COPIES = KBYTES / 16 / THREADS;
    static_assert(KBYTES % (16 * THREADS) == 0, "a block is a whole number of copies per thread");
};

#ifndef STA_F8_MINB
#define STA_F8_MINB 3
#endif

// 4. Attention.  Workgroup = NW waves = NW*32 query rows of one tile; lane
// l of a wave owns query row l%32 (lanes l and l+32 hold the two halves of
// each key block).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, STA_F8_MINB) void fwd_fp8_kernel(
    const uint8_t *__restrict__ Q8, const uint8_t *__restrict__ K8, const uint8_t *__restrict__ VT8,
    const float *__restrict__ sq, const float *__restrict__ corr, const float *__restrict__ sk,
    const float *__restrict__ vscale, __bf16 *__restrict__ O, float *__restrict__ LSE,
    const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ kv_cnt, int max_kv, int IH, Geo g, int Lp,
    int nkb, int rblocks, const int *__restrict__ split)
{
    using C = F8Cfg<D, NW>;
    constexpr int BN = C::BN;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::STAGE];

    int bh, qt, rb;
    {
        // XCD x = block index mod 8 takes the range [split[x], split[x+1]) of
        // the work order (slabs by descending cost); blocks past it exit
        const int x = blockIdx.x & 7, work = split[x] + (int)(blockIdx.x >> 3);
        if (work >= split[x + 1]) return;
        decode_item(work, rblocks, g, bh, qt, rb);
        bh = plan_slab(split, bh);
    }
    const Span qs = tile_span(g, qt);
    const int qlen = qs.len;
    if (rb * C::M >= qlen) return;                   // row block past a cut tile's end
    const int h = bh % IH;                           // list set: the head's, or (b, h)'s
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, grp = lane >> 5;
    const int64_t base = (int64_t)bh * g.S * D;      // bytes of the codes, elements of O
    const int64_t vt_base = (int64_t)bh * g.TT * D * Lp;
    const int row = rb * C::M + wave * 32 + l32;
    const bool row_ok = row < qlen;
    const int64_t grow = qs.start + (row_ok ? row : qlen - 1);

    // Q codes: B operand of S^T = K Q^T, 16 bytes per step
    i32x4 qf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qf[ks] = *(const i32x4 *)(Q8 + base + grow * D + ks * 32 + grp * 16);
    const float fq = sq[(int64_t)bh * g.S + grow];
    const float cq = corr[(int64_t)bh * g.S + grow];
    wait_vmem<0>();                                  // register loads complete before the first copy

    f32x16 acc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float m_i = -INFINITY, l_i = 0.f;

    const bool video_q = qt < g.T;
    const int cnt = video_q ? kv_cnt[(int64_t)h * g.T + qt] : g.T;
    const int32_t *lst = video_q ? kv_idx + ((int64_t)h * g.T + qt) * max_kv : nullptr;
    const int nblk = walk_blocks(g, lst, cnt, BN);

    // per-lane copy offsets (bytes): wave-wide copy i fills granule slots
    // (i*NW + wave)*64 + lane of the block
    int gk[C::COPIES], gv[C::COPIES];
#pragma unroll
    for (int i = 0; i < C::COPIES; ++i) {
        const int slot = (i * NW + wave) * 64 + lane;
        const int r = slot / C::GK, pg = slot % C::GK;
        gk[i] = r * D + (pg ^ swz8<C::GK>(r)) * 16;
        const int rv = slot / C::GV, pv = slot % C::GV;
        gv[i] = rv * Lp + (pv ^ swz8<C::GV>(rv)) * 16;
    }
    // S^T operand: lane feeds K row sigma(l%32) of each 32-key sub-block, the
    // 16 bytes of d-slots 32ks + 16grp .. +15 (those its Q fragment holds)
    const int arow = sigma32(l32);
    int kofs[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) kofs[ks] = arow * D + (((2 * ks + grp) ^ swz8<C::GK>(arow)) << 4);
    // PV operand: lane feeds V^T row d = 32db + l%32, bytes 32grp .. 32grp+31
    const int vo0 = l32 * BN + (((2 * grp) ^ swz8<C::GV>(l32)) << 4);
    const int vo1 = l32 * BN + (((2 * grp + 1) ^ swz8<C::GV>(l32)) << 4);

    int c_e = 0, c_k0 = 0;                           // next block to copy
    int c_tile = entry_tile(lst, cnt, g.T, 0);
    Span c_sp = tile_span(g, c_tile);
    int n_tile = entry_tile(lst, cnt, g.T, 1);
    int bvalid[2];                                   // valid keys of the block in each buffer
    float bscale[2];                                 // its K scale
    const float *skb = sk + (int64_t)bh * g.TT * nkb;
    auto gload = [&](int buf) {
        const int valid = c_sp.len - c_k0 < BN ? c_sp.len - c_k0 : BN;
        bvalid[buf] = valid;
        bscale[buf] = skb[c_tile * nkb + c_k0 / BN];
        const auto rk = make_rsrc(K8 + base + (c_sp.start + c_k0) * D, valid * D);
        const auto rv = make_rsrc(VT8 + vt_base + (int64_t)c_tile * D * Lp + c_k0, D * Lp - c_k0);
        uint8_t *Ks = smem + buf * C::STAGE;
        uint8_t *Vs = Ks + C::KBYTES;
#pragma unroll
        for (int i = 0; i < C::COPIES; ++i) {
            b2lds16(rk, gk[i], Ks + (i * NW + wave) * 1024);
            b2lds16(rv, gv[i], Vs + (i * NW + wave) * 1024);
        }
        c_k0 += BN;
        if (c_k0 >= c_sp.len) {
            c_k0 = 0;
            ++c_e;
            c_tile = n_tile;
            c_sp = tile_span(g, c_tile);
            n_tile = entry_tile(lst, cnt, g.T, c_e + 1);
        }
    };

    auto step = [&](auto bufc, int blk) {
        constexpr int BUF = decltype(bufc)::value;
        __builtin_amdgcn_s_waitcnt(0);               // this wave's copies of block blk have landed
        __syncthreads();                             // ... and everyone's; the other buffer is free
        const int valid = bvalid[BUF];
        // Logit factor of the block.  Masked keys get s = -inf below, and f is
        // zero for an all-zero Q row or a K block equal to the smoothing mean
        // (-inf * 0 would be NaN); raising f to the smallest normal float
        // keeps them at -inf and changes nothing else: such a row or block
        // has all-zero codes, so its unmasked s are 0 either way.
        const float f = fmaxf(fq * bscale[BUF], FLT_MIN);
        if (blk + 1 < nblk) gload(1 - BUF);
        const uint8_t *Ks = smem + BUF * C::STAGE;
        const uint8_t *Vs = Ks + C::KBYTES;

        // s[kb][r]: the exact int32 dot product of register r of sub-block
        // kb, as a float; the logit is s * f
        float s[2][16];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            i32x16 a;
#pragma unroll
            for (int r = 0; r < 16; ++r) a[r] = 0;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
                a = __builtin_amdgcn_mfma_i32_32x32x32_i8(*(const i32x4 *)(Ks + kb * 32 * D + kofs[ks]), qf[ks], a, 0,
                                                          0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = (float)a[r];
        }
        if (valid < BN) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kb * 32 + mfma_row_sigma(lane, r) >= valid) s[kb][r] = -INFINITY;
        }
        // P = 2^(s*f - m + 4) in e4m3 (exponent by one fused multiply-add),
        // byte 16kb + r of the operand = register r of sub-block kb; the row
        // sum is taken from the rounded values, two at a time (e4m3 -> bf16
        // is exact, then a dot product with ones).
        // The integer running max m is kept while every P of the lane stays
        // below 2^8 (e4m3 reaches 448); otherwise the block max, rounded up,
        // becomes the new max and O, l are rescaled by an exact power of two.
        i32x8 pw;
        auto probs = [&]() {
            const float nmo = 4.f - m_i;
            const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * j], f, nmo));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * j + 1], f, nmo));
                    const float p2 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * j + 2], f, nmo));
                    const float p3 = __builtin_amdgcn_exp2f(fmaf(s[kb][4 * j + 3], f, nmo));
                    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
                    pw[4 * kb + j] = w;
                    ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false), one2,
                                                         ls, false);
                    ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true), one2,
                                                         ls, false);
                }
            return ls;
        };
        float ls = probs();
        if (__any(!(ls < 256.f))) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            const float mn = ceilf(fmaxf(m_i, max_pair32(mx) * f));
            const float alpha = __builtin_amdgcn_exp2f(m_i - mn);
            m_i = mn;
            l_i *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            ls = probs();
        }
        l_i += ls;

#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const i32x4 a0 = *(const i32x4 *)(Vs + db * 32 * BN + vo0);
            const i32x4 a1 = *(const i32x4 *)(Vs + db * 32 * BN + vo1);
            const i32x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pw, acc[db], 0, 0, 0, 127, 0, 127);
        }
    };

    if (nblk > 0) gload(0);
    for (int blk = 0; blk < nblk; blk += 2) {
        step(std::integral_constant<int, 0>{}, blk);
        if (blk + 1 < nblk) step(std::integral_constant<int, 1>{}, blk + 1);
    }

    // Epilogue: O = acc * (V channel scale) / l; lanes l and l^32 hold the
    // two halves of row l%32's sum.
    const float lt = sum_pair32(l_i);
    const float inv = 1.f / lt;
    if (row_ok) {
        const int64_t orow = tile_row(g, qt, row);   // the layout's row of the output
        __bf16 *op = O + base + orow * D;
        const float *svp = vscale + (int64_t)bh * D;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 sv = *(const f32x4 *)(svp + db * 32 + 8 * j + 4 * grp);
                bf16x4 v;
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = (__bf16)(acc[db][4 * j + t] * sv[t] * inv);
                *(bf16x4 *)(op + db * 32 + 8 * j + 4 * grp) = v;
            }
        if (grp == 0)
            LSE[(int64_t)bh * g.S + orow] = (m_i - 4.f + __log2f(lt)) * 0.69314718055994531f + cq;
    }
}

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

template <int D, int NW>
static sta_status run_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                              float scale, const Geo &g, const sta_index &idx, hipStream_t s)
{
    using C = F8Cfg<D, NW>;
    const int nkb = (g.L + kKeyBlock - 1) / kKeyBlock;
    const int Lp = nkb * kKeyBlock;
    const int64_t BH = (int64_t)B * H;
    const int rblocks = (g.L + C::M - 1) / C::M;
    const int64_t total = BH * g.TT * rblocks;
    const int64_t blocks = work_blocks(total);
    const int64_t qk_blocks = BH * g.TT * nkb;
    if (!grid_fits(blocks, C::THREADS) || !grid_fits(qk_blocks, 256) || !grid_fits(BH * kStatChunks, 256))
        return fail(STA_ERR_UNSUPPORTED, "too many work items");
    // workspace: codes, scales and statistics
    const size_t n_codes = (size_t)BH * g.S * D, n_vt = (size_t)BH * g.TT * D * Lp;
    const size_t n_rows = (size_t)BH * g.S, n_sk = (size_t)BH * g.TT * nkb, n_ch = (size_t)BH * D;
    const size_t n_part = (size_t)BH * kStatChunks * 2 * D;
    const size_t off_q8 = 0, off_k8 = off_q8 + align256(n_codes), off_vt = off_k8 + align256(n_codes);
    const size_t off_sq = off_vt + align256(n_vt), off_corr = off_sq + align256(n_rows * 4);
    const size_t off_sk = off_corr + align256(n_rows * 4), off_km = off_sk + align256(n_sk * 4);
    const size_t off_vs = off_km + align256(n_ch * 4), off_vi = off_vs + align256(n_ch * 4);
    const size_t off_part = off_vi + align256(n_ch * 4), off_plan = off_part + align256(n_part * 8);
    const size_t bytes = off_plan + align256(plan_bytes(idx.num_heads, (int64_t)B * H));
    void *ws = nullptr;
    sta_status st = workspace_alloc(&ws, bytes, s);
    if (st != STA_OK) return st;
    char *w = (char *)ws;
    uint8_t *q8 = (uint8_t *)(w + off_q8), *k8 = (uint8_t *)(w + off_k8), *vt8 = (uint8_t *)(w + off_vt);
    float *sq = (float *)(w + off_sq), *corr = (float *)(w + off_corr), *sk = (float *)(w + off_sk);
    float *km = (float *)(w + off_km), *vs = (float *)(w + off_vs), *vi = (float *)(w + off_vi);
    double *part = (double *)(w + off_part);
    const int *split = nullptr;
    if ((st = plan_work(g, idx.kv_cnt, idx.num_heads, BH, rblocks, blocks, w + off_plan, s, &split)) != STA_OK) {
        (void)workspace_free(ws, s);          // the launch error is the one reported
        return st;
    }
    const __bf16 *Q = (const __bf16 *)q, *K = (const __bf16 *)k, *V = (const __bf16 *)v;
    const float c_log2 = scale * 1.4426950408889634f;

    hipLaunchKernelGGL(qstat_kernel<D>, dim3((unsigned)(BH * kStatChunks)), dim3(256), 0, s, K, V, part, g.S);
    hipLaunchKernelGGL(qstat_final_kernel<D>, dim3((unsigned)((BH * D + 255) / 256)), dim3(256), 0, s, part, km, vs,
                       vi, g.S, (int)BH);
    hipLaunchKernelGGL(quant_qk_kernel<D>, dim3((unsigned)qk_blocks), dim3(256), 0, s, Q, K, km, q8, k8, sq, corr, sk,
                       g, nkb, c_log2, scale);
    hipLaunchKernelGGL(quant_vt_kernel<D>, dim3((unsigned)qk_blocks), dim3(256), 0, s, V, vi, vt8, g, Lp, nkb);
    hipLaunchKernelGGL((fwd_fp8_kernel<D, NW>), dim3((unsigned)blocks), dim3(C::THREADS), 0, s, q8, k8, vt8, sq, corr,
                       sk, vs, (__bf16 *)o, lse, idx.kv_idx, idx.kv_cnt, idx.max_kv, idx.num_heads, g, Lp, nkb, rblocks,
                       split);
    st = check_launch();
    const sta_status fs = workspace_free(ws, s);
    return st != STA_OK ? st : fs;
}

#ifndef STA_F8_NW
#define STA_F8_NW 4
#endif

sta_status launch_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int D,
                          float scale, const Geo &g, const sta_index &idx, hipStream_t s)
{
    if (D == 128) return run_fwd_fp8<128, STA_F8_NW>(q, k, v, o, lse, B, H, scale, g, idx, s);
    return run_fwd_fp8<64, STA_F8_NW>(q, k, v, o, lse, B, H, scale, g, idx, s);
}

}  // namespace sta
