// Window-shift producer: chooses the shift of every query tile's key-tile
// window from the content.  3D Deformable Slide Attention moves the windows
// with the motion in the video ("MegaSlide-DiT: Memory-Centric Adaptation and
// Deformable Local Attention for Efficient Video Diffusion", abstract) but
// gives no rule; this library's rule is:
//   1. qbar, kbar: means of Q and K over the tokens of every tile (a tile cut
//      by the grid border over the tokens it holds), per (b, h); shared by
//      the batch as the mean of the per-batch means, or kept per batch item;
//   2. z_qk = scale * <qbar_q, kbar_k>;
//   3. mass(o) = sum over the key tiles k in the window of q shifted by o of
//      len_k * exp(z_qk - zmax_q), for every o of the search box
//      [-r_t, r_t] x [-r_h, r_h] x [-r_w, r_w], windows as the index builds
//      them (border rule included);
//   4. the shift of largest mass; among equal masses the smallest
//      |o_t| + |o_h| + |o_w|, then the first in raster order of o.
// zmax_q is taken over the search region (the union of the candidate
// windows): a factor common to one query tile's masses does not change its
// choice.
//
// Kernels:
//   tile_mean_kernel  one workgroup per (tensor, set, head, tile).  A tile's
//                     rows are one contiguous run of its tile-order slab (in
//                     the raster layout they are gathered row by row), so
//                     the workgroup streams it with 16-byte loads, rows
//                     spread over the threads, and reduces the partial sums
//                     in LDS in a fixed order (deterministic).  It reads Q
//                     and K once: bound by HBM bandwidth.
//   shift_kernel      one workgroup per (set, head, query tile): z over the
//                     search region into LDS (a wave per key tile, lanes
//                     across D), the exponentials, one thread per candidate
//                     summing its window in ascending tile order, and an
//                     argmax over the workgroup in the total order of step 4.
#include <limits.h>
#include <math.h>

#include <mutex>
#include <type_traits>

#include "common.h"

namespace sta {

namespace {

constexpr int kShiftHeadsPerLaunch = 64;
constexpr int kThreads = 256;

struct ShiftWindows {
    int w[kShiftHeadsPerLaunch][3];
};

template <typename E>
struct RowVec;

template <>
struct RowVec<__bf16> {
    using raw = uint4;
    static constexpr int n = 8;
    __device__ static void add(float *acc, const uint4 &u)
    {
        const unsigned x[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += __uint_as_float(x[i] << 16);
            acc[2 * i + 1] += __uint_as_float(x[i] & 0xffff0000u);
        }
    }
};

template <>
struct RowVec<float> {
    using raw = float4;
    static constexpr int n = 4;
    __device__ static void add(float *acc, const float4 &u)
    {
        acc[0] += u.x;
        acc[1] += u.y;
        acc[2] += u.z;
        acc[3] += u.w;
    }
};

// means[tensor][set][h][tile][d], tensor 0 = Q, 1 = K; set p covers the
// batch items p*nb .. p*nb + nb - 1 (nb = B when shared by the batch, 1 per
// batch item) and holds the mean of their per-item tile means.
template <int D, typename E>
__global__ __launch_bounds__(kThreads) void tile_mean_kernel(const E *__restrict__ Q, const E *__restrict__ K,
                                                             float *__restrict__ means, int H, int P, int nb,
                                                             Geo g)
{
    using V = RowVec<E>;
    constexpr int TPR = D / V::n;       // threads per row
    constexpr int RPP = kThreads / TPR; // rows per pass
    __shared__ float red[RPP][D];

    const int64_t w = blockIdx.x;       // ((tensor * P + p) * H + h) * T + tile
    const int tile = (int)(w % g.T);
    const int64_t rest = w / g.T;
    const int h = (int)(rest % H);
    const int p = (int)((rest / H) % P);
    const int tensor = (int)(rest / ((int64_t)H * P));
    const E *X = tensor ? K : Q;
    const Span sp = tile_span(g, tile);
    const int tid = threadIdx.x, col = tid % TPR, r0 = tid / TPR;

    float total = 0.f;
    for (int bi = 0; bi < nb; ++bi) {
        const int64_t b = (int64_t)p * nb + bi;
        float acc[V::n];
#pragma unroll
        for (int j = 0; j < V::n; ++j) acc[j] = 0.f;
        int r = r0;
        if (g.raster) {              // rows of the tile where its tokens sit
            const E *slab = X + (b * H + h) * g.S * D + col * V::n;
            for (; r < sp.len; r += RPP)
                V::add(acc, *reinterpret_cast<const typename V::raw *>(slab + tile_row(g, tile, r) * D));
        }
        const E *src = X + ((b * H + h) * g.S + sp.start) * D + col * V::n;
        for (; r + 3 * RPP < sp.len; r += 4 * RPP) {
            typename V::raw u[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                u[i] = *reinterpret_cast<const typename V::raw *>(src + (int64_t)(r + i * RPP) * D);
#pragma unroll
            for (int i = 0; i < 4; ++i) V::add(acc, u[i]);
        }
        for (; r < sp.len; r += RPP) V::add(acc, *reinterpret_cast<const typename V::raw *>(src + (int64_t)r * D));
#pragma unroll
        for (int j = 0; j < V::n; ++j) red[r0][col * V::n + j] = acc[j];
        __syncthreads();
        if (tid < D) {
            float s = 0.f;
            for (int rr = 0; rr < RPP; ++rr) s += red[rr][tid];
            total += s / (float)sp.len;
        }
        __syncthreads();
    }
    if (tid < D) means[w * D + tid] = total / (float)nb;
}

__device__ inline void shift_window(const Geo &g, int axis, int w, int q, int o, bool truncate, int &s, int &c)
{
    const int n = axis == 0 ? g.nt : axis == 1 ? g.nh : g.nw;
    if (truncate)
        axis_window_truncated(n, w, q, o, s, c);
    else
        axis_window(n, w, q, o, s, c);
}

// Step 4's order: larger mass first, then smaller |o|_1, then earlier in
// raster order.  A total order over the candidates (c is unique), so the
// argmax does not depend on the order of the reduction.
__device__ inline bool better(float m, int l1, int c, float bm, int bl1, int bc)
{
    return m > bm || (m == bm && (l1 < bl1 || (l1 == bl1 && c < bc)));
}

template <int D>
__global__ __launch_bounds__(kThreads) void shift_kernel(const float *__restrict__ means, int P, int H, int h0,
                                                         int nheads, ShiftWindows wins, Geo g, int rt, int rh,
                                                         int rw, bool truncate, float scale,
                                                         int32_t *__restrict__ offsets)
{
    extern __shared__ float e[];         // one entry per tile of the search region
    __shared__ float wmax[kThreads / 64];
    __shared__ float bmass[kThreads / 64];
    __shared__ int bl1s[kThreads / 64], bcs[kThreads / 64];

    const int q = blockIdx.x % g.T;
    const int rest = blockIdx.x / g.T;
    const int hl = rest % nheads, p = rest / nheads, h = h0 + hl;
    const int *win = wins.w[hl];
    const int rad[3] = {rt, rh, rw};
    const int qc[3] = {q / (g.nh * g.nw), (q / g.nw) % g.nh, q % g.nw};
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // search region: on each axis the windows start no earlier than at -r
    // and end no later than at +r, and consecutive shifts move a window by
    // at most one tile, so the union of the windows is this interval
    int lo[3], R[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        int s0, c0, s1, c1;
        shift_window(g, d, win[d], qc[d], -rad[d], truncate, s0, c0);
        shift_window(g, d, win[d], qc[d], rad[d], truncate, s1, c1);
        lo[d] = s0;
        R[d] = s1 + c1 - s0;
    }
    const int RT = R[0] * R[1] * R[2];

    constexpr int PER = D / 64;
    const float *qm = means + (((int64_t)p * H + h) * g.T + q) * D + lane * PER;
    const float *km = means + (((int64_t)(P + p) * H + h) * g.T) * D + lane * PER;
    float qv[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) qv[j] = qm[j];
    // four key tiles per wave and pass, so that four loads are in flight
    constexpr int WAVES = kThreads / 64, U = 4;
    for (int i0 = wave; i0 < RT; i0 += WAVES * U) {
        float sv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * WAVES;
            sv[u] = 0.f;
            if (i < RT) {
                const int a = i / (R[1] * R[2]), b = (i / R[2]) % R[1], c = i % R[2];
                const int k = ((lo[0] + a) * g.nh + lo[1] + b) * g.nw + lo[2] + c;
                const float *kr = km + (int64_t)k * D;
#pragma unroll
                for (int j = 0; j < PER; ++j) sv[u] = fmaf(qv[j], kr[j], sv[u]);
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1)
#pragma unroll
            for (int u = 0; u < U; ++u) sv[u] += __shfl_xor(sv[u], m);
        if (lane == 0)
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (i0 + u * WAVES < RT) e[i0 + u * WAVES] = scale * sv[u];
    }
    __syncthreads();

    float zm = -INFINITY;
    for (int i = tid; i < RT; i += kThreads) zm = fmaxf(zm, e[i]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) zm = fmaxf(zm, __shfl_xor(zm, m));
    if (lane == 0) wmax[wave] = zm;
    __syncthreads();
    zm = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    for (int i = tid; i < RT; i += kThreads) {
        const int a = i / (R[1] * R[2]), b = (i / R[2]) % R[1], c = i % R[2];
        const int k = ((lo[0] + a) * g.nh + lo[1] + b) * g.nw + lo[2] + c;
        e[i] = (float)tile_rows(g, k) * expf(e[i] - zm);
    }
    __syncthreads();

    const int C1 = 2 * rh + 1, C2 = 2 * rw + 1;
    const int NC = (2 * rt + 1) * C1 * C2;
    float best = -1.f;                   // masses are >= 0; a NaN mass is never taken
    int bl1 = INT_MAX, bc = INT_MAX;
    for (int c = tid; c < NC; c += kThreads) {
        const int o[3] = {c / (C1 * C2) - rt, (c / C2) % C1 - rh, c % C2 - rw};
        int s[3], n[3];
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            shift_window(g, d, win[d], qc[d], o[d], truncate, s[d], n[d]);
            s[d] -= lo[d];
        }
        float mass = 0.f;
        for (int a = s[0]; a < s[0] + n[0]; ++a)
            for (int b = s[1]; b < s[1] + n[1]; ++b) {
                const float *row = e + (a * R[1] + b) * R[2];
                for (int x = s[2]; x < s[2] + n[2]; ++x) mass += row[x];
            }
        const int l1 = abs(o[0]) + abs(o[1]) + abs(o[2]);
        if (better(mass, l1, c, best, bl1, bc)) {
            best = mass;
            bl1 = l1;
            bc = c;
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const float om = __shfl_xor(best, m);
        const int ol = __shfl_xor(bl1, m), oc = __shfl_xor(bc, m);
        if (better(om, ol, oc, best, bl1, bc)) {
            best = om;
            bl1 = ol;
            bc = oc;
        }
    }
    if (lane == 0) {
        bmass[wave] = best;
        bl1s[wave] = bl1;
        bcs[wave] = bc;
    }
    __syncthreads();
    if (tid == 0) {
        for (int x = 1; x < kThreads / 64; ++x)
            if (better(bmass[x], bl1s[x], bcs[x], best, bl1, bc)) {
                best = bmass[x];
                bl1 = bl1s[x];
                bc = bcs[x];
            }
        int32_t *out = offsets + (((int64_t)p * H + h) * g.T + q) * 3;
        if (bc == INT_MAX) {             // no finite mass (non-finite inputs): no shift
            out[0] = out[1] = out[2] = 0;
        } else {
            out[0] = bc / (C1 * C2) - rt;
            out[1] = (bc / C2) % C1 - rh;
            out[2] = bc % C2 - rw;
        }
    }
}

// Bytes of tile means the producer keeps: [2][P][H][T][D] fp32.
static size_t means_bytes(int B, int H, int D, const Geo &g, bool per_batch)
{
    return (size_t)2 * (per_batch ? B : 1) * H * g.T * D * sizeof(float);
}

// The two launches on a means buffer of means_bytes() (every value is
// written by the first before the second reads it).
template <int D, typename E>
sta_status run_shifts(const E *q, const E *k, int B, int H, float scale, const Geo &g, const int32_t *windows,
                      const int radius[3], bool truncate, bool per_batch, int region_max, int32_t *offsets,
                      float *means, hipStream_t s)
{
    const int P = per_batch ? B : 1, nb = per_batch ? 1 : B;
    sta_status st = STA_OK;
    const int64_t mean_blocks = (int64_t)2 * P * H * g.T;
    hipLaunchKernelGGL((tile_mean_kernel<D, E>), dim3((unsigned)mean_blocks), dim3(kThreads), 0, s, q, k, means,
                       H, P, nb, g);
    st = check_launch();
    for (int h0 = 0; st == STA_OK && h0 < H; h0 += kShiftHeadsPerLaunch) {
        const int nh = H - h0 < kShiftHeadsPerLaunch ? H - h0 : kShiftHeadsPerLaunch;
        ShiftWindows w;
        for (int i = 0; i < kShiftHeadsPerLaunch; ++i)
            for (int d = 0; d < 3; ++d) w.w[i][d] = i < nh ? windows[3 * (h0 + i) + d] : 1;
        const int64_t blocks = (int64_t)P * nh * g.T;
        hipLaunchKernelGGL((shift_kernel<D>), dim3((unsigned)blocks), dim3(kThreads),
                           (size_t)region_max * sizeof(float), s, means, P, H, h0, nh, w, g, radius[0], radius[1],
                           radius[2], truncate, scale, offsets);
        st = check_launch();
    }
    return st;
}

template <typename F>
sta_status dispatch(int D, sta_dtype dtype, const void *q, const void *k, F &&run)
{
    if (dtype == STA_BF16) {
        if (D == 128) return run(std::integral_constant<int, 128>{}, (const __bf16 *)q, (const __bf16 *)k);
        return run(std::integral_constant<int, 64>{}, (const __bf16 *)q, (const __bf16 *)k);
    }
    if (D == 128) return run(std::integral_constant<int, 128>{}, (const float *)q, (const float *)k);
    return run(std::integral_constant<int, 64>{}, (const float *)q, (const float *)k);
}

// Scratch of the allocation-free producer: room for the tile means of one
// call of up to kShiftScratchBytes (16 MiB: the 720P shape, 24 heads of 300
// tiles at D = 128, for up to two batch items with per-item shifts).  Every
// GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// host code uses only the per-device address from hipGetSymbolAddress.
constexpr size_t kShiftScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) float scratch[kShiftScratchBytes / sizeof(float)];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch[kMaxScratchDevices];

// Device address of `scratch` on the device of stream s, looked up once per
// device with that device current (restored afterwards).
sta_status scratch_for(hipStream_t s, float *&ptr)
{
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(s, &dev);
    if (e != hipSuccess) return fail(STA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices) return fail(STA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return fail(STA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(STA_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(e));
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return fail(STA_ERR_HIP, "hipGetSymbolAddress: %s", hipGetErrorString(e));
        if (back != hipSuccess) return fail(STA_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(back));
        g_scratch[dev] = (float *)p;
    }
    ptr = g_scratch[dev];
    return STA_OK;
}

}  // namespace

sta_status launch_window_shifts(const void *q, const void *k, int B, int H, int D, sta_dtype dtype, float scale,
                                const Geo &g, const int32_t *windows, const int radius[3], bool truncate,
                                bool per_batch, int region_max, int32_t *offsets, hipStream_t s)
{
    float *means = nullptr;
    sta_status st = workspace_alloc((void **)&means, means_bytes(B, H, D, g, per_batch), s);
    if (st != STA_OK) return st;
    st = dispatch(D, dtype, q, k, [&](auto dc, auto qp, auto kp) {
        return run_shifts<decltype(dc)::value>(qp, kp, B, H, scale, g, windows, radius, truncate, per_batch,
                                               region_max, offsets, means, s);
    });
    const sta_status fr = workspace_free(means, s);
    return st != STA_OK ? st : fr;
}

sta_status launch_window_shifts_scratch(const void *q, const void *k, int B, int H, int D, sta_dtype dtype,
                                        float scale, const Geo &g, const int32_t *windows, const int radius[3],
                                        bool truncate, bool per_batch, int region_max, int32_t *offsets,
                                        hipStream_t s)
{
    const size_t bytes = means_bytes(B, H, D, g, per_batch);
    if (bytes > kShiftScratchBytes)
        return fail(STA_ERR_UNSUPPORTED, "tile means of %zu bytes exceed the %zu-byte scratch of the allocation-free "
                                         "call (2 * P * H * num_tiles * D * 4 bytes)", bytes, kShiftScratchBytes);
    float *means = nullptr;
    const sta_status st = scratch_for(s, means);
    if (st != STA_OK) return st;
    return dispatch(D, dtype, q, k, [&](auto dc, auto qp, auto kp) {
        return run_shifts<decltype(dc)::value>(qp, kp, B, H, scale, g, windows, radius, truncate, per_batch,
                                               region_max, offsets, means, s);
    });
}

}  // namespace sta
