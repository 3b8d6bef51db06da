// fp32 attention path: one thread per query row (forward, dQ) or key row
// (dK/dV), walking the block-sparse lists.  Plain VALU code meant for small
// shapes and for fp32 callers; the bf16 MFMA kernels carry the performance.
#include "common.h"

namespace sta {

// Tile holding video row i of a slab (compact tile order: whole tile planes
// along t, tile rows along h inside a plane, tiles along w inside a row,
// the last of each cut by the grid border; or raster order).
__device__ inline int tile_of_row(const Geo &g, int64_t i)
{
    if (g.raster) {                    // raster order, whole tiles
        const int64_t plane = (int64_t)g.gh * g.gw;
        const int t = (int)(i / plane), h = (int)((i / g.gw) % g.gh), w = (int)(i % g.gw);
        return ((t / g.tt) * g.nh + h / g.th) * g.nw + w / g.tw;
    }
    if (!g.ragged) return (int)(i / g.L);
    const int64_t plane = (int64_t)g.tt * g.gh * g.gw;
    int a = (int)(i / plane);
    a = a < g.nt - 1 ? a : g.nt - 1;
    int64_t r = i - a * plane;
    const int vt = g.gt - a * g.tt < g.tt ? g.gt - a * g.tt : g.tt;
    const int64_t trow = (int64_t)vt * g.th * g.gw;
    int b = (int)(r / trow);
    b = b < g.nh - 1 ? b : g.nh - 1;
    r -= b * trow;
    const int vh = g.gh - b * g.th < g.th ? g.gh - b * g.th : g.th;
    int c = (int)(r / ((int64_t)vt * vh * g.tw));
    c = c < g.nw - 1 ? c : g.nw - 1;
    return (a * g.nh + b) * g.nw + c;
}

// Calls f(r) for every partner row r of row i of a slab: for a video row
// the rows of its listed tiles, then the text rows; for a text row every
// row (MOD-DiT README, "Token-Type-Aware Masking").
template <typename F>
__device__ inline void for_partners(int64_t i, int h, const Geo &g, const int32_t *idx, const int32_t *cnt_,
                                    int max_e, F &&f)
{
    if (i >= g.N) {
        for (int64_t r = 0; r < g.S; ++r) f(r);
        return;
    }
    const int t = tile_of_row(g, i);
    const int cnt = cnt_[(int64_t)h * g.T + t];
    const int32_t *lst = idx + ((int64_t)h * g.T + t) * max_e;
    for (int e = 0; e < cnt; ++e) {
        const int len = tile_rows(g, lst[e]);
        for (int rr = 0; rr < len; ++rr) f(tile_row(g, lst[e], rr));
    }
    for (int64_t r = g.N; r < g.S; ++r) f(r);
}

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float *__restrict__ Q, const float *__restrict__ K,
                                                      const float *__restrict__ V, float *__restrict__ O,
                                                      float *__restrict__ LSE, const int32_t *__restrict__ kv_idx,
                                                      const int32_t *__restrict__ kv_cnt, int max_kv, int B,
                                                      int H, int IH, Geo g, float scale)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)B * H * g.S) return;
    const int64_t i = gid % g.S;
    const int64_t bh = gid / g.S;
    const int h = (int)(bh % IH);   // list set: the head's, or (b, h)'s
    const float *kb = K + bh * g.S * D;
    const float *vb = V + bh * g.S * D;
    float q[D], acc[D];
    for (int d = 0; d < D; ++d) {
        q[d] = Q[gid * D + d];
        acc[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for_partners(i, h, g, kv_idx, kv_cnt, max_kv, [&](int64_t j) {
        const float *kr = kb + j * D;
        float s = 0.f;
        for (int d = 0; d < D; ++d) s = fmaf(q[d], kr[d], s);
        s *= scale;
        const float mn = fmaxf(m, s);
        const float alpha = expf(m - mn);   // m = -inf on the first key: alpha = 0
        const float p = expf(s - mn);
        l = l * alpha + p;
        const float *vr = vb + j * D;
        for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vr[d], acc[d] * alpha);
        m = mn;
    });
    const float inv = 1.f / l;
    for (int d = 0; d < D; ++d) O[gid * D + d] = acc[d] * inv;
    LSE[gid] = m + logf(l);
}

template <int D>
__global__ __launch_bounds__(256) void delta_f32_kernel(const float *__restrict__ O, const float *__restrict__ dO,
                                                        float *__restrict__ delta, int64_t rows)
{
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    float s = 0.f;
    for (int d = 0; d < D; ++d) s = fmaf(O[r * D + d], dO[r * D + d], s);
    delta[r] = s;
}

template <int D>
__global__ __launch_bounds__(256) void dq_f32_kernel(const float *__restrict__ Q, const float *__restrict__ K,
                                                     const float *__restrict__ V, const float *__restrict__ LSE,
                                                     const float *__restrict__ dO, const float *__restrict__ delta,
                                                     float *__restrict__ dQ, const int32_t *__restrict__ kv_idx,
                                                     const int32_t *__restrict__ kv_cnt, int max_kv, int B, int H, int IH,
                                                     Geo g, float scale)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)B * H * g.S) return;
    const int64_t i = gid % g.S;
    const int64_t bh = gid / g.S;
    const int h = (int)(bh % IH);   // list set: the head's, or (b, h)'s
    const float *kb = K + bh * g.S * D;
    const float *vb = V + bh * g.S * D;
    float q[D], go[D], acc[D];
    for (int d = 0; d < D; ++d) {
        q[d] = Q[gid * D + d];
        go[d] = dO[gid * D + d];
        acc[d] = 0.f;
    }
    const float lse = LSE[gid], dl = delta[gid];
    for_partners(i, h, g, kv_idx, kv_cnt, max_kv, [&](int64_t j) {
        const float *kr = kb + j * D;
        const float *vr = vb + j * D;
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
            s = fmaf(q[d], kr[d], s);
            dp = fmaf(go[d], vr[d], dp);
        }
        const float p = expf(s * scale - lse);
        const float ds = p * (dp - dl);
        for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, kr[d], acc[d]);
    });
    for (int d = 0; d < D; ++d) dQ[gid * D + d] = acc[d] * scale;
}

template <int D>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(const float *__restrict__ Q, const float *__restrict__ K,
                                                       const float *__restrict__ V, const float *__restrict__ LSE,
                                                       const float *__restrict__ dO, const float *__restrict__ delta,
                                                       float *__restrict__ dK, float *__restrict__ dV,
                                                       const int32_t *__restrict__ q_idx,
                                                       const int32_t *__restrict__ q_cnt, int max_q, int B, int H, int IH,
                                                       Geo g, float scale)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)B * H * g.S) return;
    const int64_t j = gid % g.S;
    const int64_t bh = gid / g.S;
    const int h = (int)(bh % IH);   // list set: the head's, or (b, h)'s
    const float *qb = Q + bh * g.S * D;
    const float *ob = dO + bh * g.S * D;
    const float *lb = LSE + bh * g.S;
    const float *db = delta + bh * g.S;
    float k[D], v[D], ak[D], av[D];
    for (int d = 0; d < D; ++d) {
        k[d] = K[gid * D + d];
        v[d] = V[gid * D + d];
        ak[d] = 0.f;
        av[d] = 0.f;
    }
    for_partners(j, h, g, q_idx, q_cnt, max_q, [&](int64_t i) {
        const float *qr = qb + i * D;
        const float *gr = ob + i * D;
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
            s = fmaf(qr[d], k[d], s);
            dp = fmaf(gr[d], v[d], dp);
        }
        const float p = expf(s * scale - lb[i]);
        const float ds = p * (dp - db[i]);
        for (int d = 0; d < D; ++d) {
            av[d] = fmaf(p, gr[d], av[d]);
            ak[d] = fmaf(ds, qr[d], ak[d]);
        }
    });
    for (int d = 0; d < D; ++d) {
        dK[gid * D + d] = ak[d] * scale;
        dV[gid * D + d] = av[d];
    }
}

static dim3 grid_for(int64_t threads) { return dim3((unsigned)((threads + 255) / 256)); }

sta_status launch_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse, int B, int H,
                          int D, float scale, const Geo &g, const sta_index &idx, hipStream_t s)
{
    const int64_t rows = (int64_t)B * H * g.S;
    if (!grid_fits((rows + 255) / 256, 256))
        return fail(STA_ERR_UNSUPPORTED, "fp32 path: too many rows");
    if (D == 64)
        hipLaunchKernelGGL(fwd_f32_kernel<64>, grid_for(rows), dim3(256), 0, s, q, k, v, o, lse, idx.kv_idx,
                           idx.kv_cnt, idx.max_kv, B, H, idx.num_heads, g, scale);
    else
        hipLaunchKernelGGL(fwd_f32_kernel<128>, grid_for(rows), dim3(256), 0, s, q, k, v, o, lse, idx.kv_idx,
                           idx.kv_cnt, idx.max_kv, B, H, idx.num_heads, g, scale);
    return check_launch();
}

sta_status launch_bwd_f32(const float *q, const float *k, const float *v, const float *o, const float *lse,
                          const float *dout, float *dq, float *dk, float *dv, float *delta, int B, int H, int D,
                          float scale, const Geo &g, const sta_index &idx, int parts, hipStream_t s)
{
    const int64_t rows = (int64_t)B * H * g.S;
    if (!grid_fits((rows + 255) / 256, 256))
        return fail(STA_ERR_UNSUPPORTED, "fp32 path: too many rows");
    const dim3 grid = grid_for(rows), blk(256);
    if (parts & STA_BWD_DELTA) {
        if (D == 64) hipLaunchKernelGGL(delta_f32_kernel<64>, grid, blk, 0, s, o, dout, delta, rows);
        else hipLaunchKernelGGL(delta_f32_kernel<128>, grid, blk, 0, s, o, dout, delta, rows);
    }
    if (parts & STA_BWD_DKDV) {
        if (D == 64)
            hipLaunchKernelGGL(dkdv_f32_kernel<64>, grid, blk, 0, s, q, k, v, lse, dout, delta, dk, dv, idx.q_idx,
                               idx.q_cnt, idx.max_q, B, H, idx.num_heads, g, scale);
        else
            hipLaunchKernelGGL(dkdv_f32_kernel<128>, grid, blk, 0, s, q, k, v, lse, dout, delta, dk, dv, idx.q_idx,
                               idx.q_cnt, idx.max_q, B, H, idx.num_heads, g, scale);
    }
    if (parts & STA_BWD_DQ) {
        if (D == 64)
            hipLaunchKernelGGL(dq_f32_kernel<64>, grid, blk, 0, s, q, k, v, lse, dout, delta, dq, idx.kv_idx,
                               idx.kv_cnt, idx.max_kv, B, H, idx.num_heads, g, scale);
        else
            hipLaunchKernelGGL(dq_f32_kernel<128>, grid, blk, 0, s, q, k, v, lse, dout, delta, dq, idx.kv_idx,
                               idx.kv_cnt, idx.max_kv, B, H, idx.num_heads, g, scale);
    }
    return check_launch();
}

}  // namespace sta
