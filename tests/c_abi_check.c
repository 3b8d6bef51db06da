/*
 * Plain C consumer of libsta (no Python, no torch): HIP device memory from
 * hipMalloc, the four calls of the boundary (tile reorder, index build,
 * forward, backward) on a small shifted-window problem in fp32 and bf16, and
 * every output checked against the CPU oracle (test infrastructure; the
 * library never sees it).  Exits 0 and prints "c abi ok" when everything
 * matches.
 *
 * Problem: grid (4,8,12), tile (2,4,4) (2x2x3 tiles of 32 tokens), B = 1,
 * H = 2, D = 64, windows (3,3,3) and (1,3,3), one window shift per query
 * tile; inputs uniform in [-1, 1) from a xorshift generator.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "libsta.h"

int oracle_fwd(int B, int H, int D, const int grid[3], const int tile[3], const int *windows, const int *offsets,
               int flags, int ntext, double scale, const float *q, const float *k, const float *v, int64_t n_rows,
               const int64_t *rows, double *o, double *lse);
int oracle_bwd(int B, int H, int D, const int grid[3], const int tile[3], const int *windows, const int *offsets,
               int flags, int ntext, double scale, const float *q, const float *k, const float *v,
               const float *dout, int64_t n_q, const int64_t *qrows, double *dq, int64_t n_k,
               const int64_t *krows, double *dk, double *dv);

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                   \
            exit(2);                                                                  \
        }                                                                             \
    } while (0)
#define CHECK_STA(x)                                                                  \
    do {                                                                              \
        sta_status s_ = (x);                                                          \
        if (s_ != STA_OK) {                                                           \
            fprintf(stderr, "%s: %s (%s)\n", #x, sta_status_str(s_), sta_last_error()); \
            exit(3);                                                                  \
        }                                                                             \
    } while (0)

enum { B = 1, H = 2, D = 64, N = 4 * 8 * 12, T = 12 };

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static float uniform(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (float)((rng_state >> 40) * (1.0 / (1 << 24))) * 2.0f - 1.0f;
}

/* bf16 bits of x, nearest even (finite x) */
static uint16_t to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static float from_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, 4);
    return x;
}

static double max_abs_diff(const float *got, const double *want, int64_t n)
{
    double m = 0;
    for (int64_t i = 0; i < n; ++i) {
        double d = fabs((double)got[i] - want[i]);
        if (!(d <= m)) m = d;       /* NaN propagates */
    }
    return m;
}

/* One dtype: upload, reorder, forward, backward, reorder back, compare. */
static int run(sta_dtype dt, const float *q, const float *k, const float *v, const float *dout, const double *ro,
               const double *rl, const double *rq, const double *rk, const double *rv, const sta_geom *g,
               const sta_index *idx, double gate)
{
    const size_t n = (size_t)B * H * N * D, es = dt == STA_BF16 ? 2 : 4, bytes = n * es;
    void *host = malloc(bytes);
    void *raster[4], *tiled[4], *out_t[4], *out_r[4];
    float *lse_t, *lse_r, *delta;
    const float *src[4] = {q, k, v, dout};
    for (int t = 0; t < 4; ++t) {
        if (dt == STA_BF16)
            for (size_t i = 0; i < n; ++i) ((uint16_t *)host)[i] = to_bf16(src[t][i]);
        else
            memcpy(host, src[t], bytes);
        CHECK_HIP(hipMalloc(&raster[t], bytes));
        CHECK_HIP(hipMalloc(&tiled[t], bytes));
        CHECK_HIP(hipMalloc(&out_t[t], bytes));
        CHECK_HIP(hipMalloc(&out_r[t], bytes));
        CHECK_HIP(hipMemcpy(raster[t], host, bytes, hipMemcpyHostToDevice));
        CHECK_STA(sta_tile_reorder(raster[t], tiled[t], B * H, D * (int64_t)es, g, 0, 0));
    }
    CHECK_HIP(hipMalloc((void **)&lse_t, (size_t)B * H * N * 4));
    CHECK_HIP(hipMalloc((void **)&lse_r, (size_t)B * H * N * 4));
    CHECK_HIP(hipMalloc((void **)&delta, (size_t)B * H * N * 4));
    const float scale = 0.125f;
    /* out_t: 0 = O, 1 = dQ, 2 = dK, 3 = dV (tile order) */
    CHECK_STA(sta_fwd(tiled[0], tiled[1], tiled[2], out_t[0], lse_t, B, H, D, dt, scale, g, idx, 0));
    CHECK_STA(sta_bwd(tiled[0], tiled[1], tiled[2], out_t[0], lse_t, tiled[3], out_t[1], out_t[2], out_t[3], delta,
                      B, H, D, dt, scale, g, idx, 0));
    for (int t = 0; t < 4; ++t) CHECK_STA(sta_tile_reorder(out_t[t], out_r[t], B * H, D * (int64_t)es, g, 1, 0));
    CHECK_STA(sta_tile_reorder(lse_t, lse_r, B * H, 4, g, 1, 0));
    CHECK_HIP(hipDeviceSynchronize());

    int ok = 1;
    float *f = (float *)malloc(n * 4);
    const double *want[4] = {ro, rq, rk, rv};
    const char *name[4] = {"O", "dQ", "dK", "dV"};
    for (int t = 0; t < 4; ++t) {
        CHECK_HIP(hipMemcpy(host, out_r[t], bytes, hipMemcpyDeviceToHost));
        for (size_t i = 0; i < n; ++i) f[i] = dt == STA_BF16 ? from_bf16(((uint16_t *)host)[i]) : ((float *)host)[i];
        const double e = max_abs_diff(f, want[t], (int64_t)n);
        printf("%s %s max-abs %.3e\n", dt == STA_BF16 ? "bf16" : "fp32", name[t], e);
        ok &= e <= gate;
    }
    CHECK_HIP(hipMemcpy(f, lse_r, (size_t)B * H * N * 4, hipMemcpyDeviceToHost));
    const double el = max_abs_diff(f, rl, (int64_t)B * H * N);
    printf("%s LSE max-abs %.3e\n", dt == STA_BF16 ? "bf16" : "fp32", el);
    ok &= el <= (dt == STA_BF16 ? 2.5e-3 : 1e-4);
    for (int t = 0; t < 4; ++t) {
        hipFree(raster[t]);
        hipFree(tiled[t]);
        hipFree(out_t[t]);
        hipFree(out_r[t]);
    }
    hipFree(lse_t);
    hipFree(lse_r);
    hipFree(delta);
    free(f);
    free(host);
    return ok;
}

int main(void)
{
    const int grid[3] = {4, 8, 12}, tile[3] = {2, 4, 4};
    const int windows[2 * 3] = {3, 3, 3, 1, 3, 3};
    int offsets[T * 3];
    for (int i = 0; i < T * 3; ++i) offsets[i] = (int)((i * 7 + 3) % 3) - 1;   /* -1, 0, 1 */

    const size_t n = (size_t)B * H * N * D;
    float *in[4];
    for (int t = 0; t < 4; ++t) {
        in[t] = (float *)malloc(n * 4);
        for (size_t i = 0; i < n; ++i) in[t][i] = uniform();
    }
    /* the bf16 run rounds the inputs; the oracle sees the rounded values */
    float *inb[4];
    for (int t = 0; t < 4; ++t) {
        inb[t] = (float *)malloc(n * 4);
        for (size_t i = 0; i < n; ++i) inb[t][i] = from_bf16(to_bf16(in[t][i]));
    }

    int64_t *rows = (int64_t *)malloc(sizeof(int64_t) * B * H * N);
    for (int64_t i = 0; i < (int64_t)B * H * N; ++i) rows[i] = i;
    double *ref[2][5];
    for (int pass = 0; pass < 2; ++pass) {
        float **x = pass ? inb : in;
        for (int r = 0; r < 5; ++r) ref[pass][r] = (double *)malloc(sizeof(double) * n);
        if (!oracle_fwd(B, H, D, grid, tile, windows, offsets, 0, 0, 0.125, x[0], x[1], x[2], B * H * N, rows,
                        ref[pass][0], ref[pass][1]) ||
            !oracle_bwd(B, H, D, grid, tile, windows, offsets, 0, 0, 0.125, x[0], x[1], x[2], x[3], B * H * N, rows,
                        ref[pass][2], B * H * N, rows, ref[pass][3], ref[pass][4])) {
            fprintf(stderr, "oracle failed\n");
            return 4;
        }
    }

    sta_geom g = {{grid[0], grid[1], grid[2]}, {tile[0], tile[1], tile[2]}};
    sta_dim3 w[2] = {{3, 3, 3}, {1, 3, 3}};
    int32_t max_kv, max_q;
    CHECK_STA(sta_index_dims(&g, H, w, 1, &max_kv, &max_q));
    sta_index idx = {H, T, max_kv, max_q, NULL, NULL, NULL, NULL};
    int32_t *off_dev;
    CHECK_HIP(hipMalloc((void **)&idx.kv_idx, sizeof(int32_t) * H * T * max_kv));
    CHECK_HIP(hipMalloc((void **)&idx.kv_cnt, sizeof(int32_t) * H * T));
    CHECK_HIP(hipMalloc((void **)&idx.q_idx, sizeof(int32_t) * H * T * max_q));
    CHECK_HIP(hipMalloc((void **)&idx.q_cnt, sizeof(int32_t) * H * T));
    CHECK_HIP(hipMalloc((void **)&off_dev, sizeof(offsets)));
    CHECK_HIP(hipMemcpy(off_dev, offsets, sizeof(offsets), hipMemcpyHostToDevice));
    CHECK_STA(sta_build_index(&g, H, w, off_dev, &idx, 0));

    /* an error is reported on the host, before anything runs */
    if (sta_fwd(NULL, NULL, NULL, NULL, NULL, B, H, D, STA_F32, 0.125f, &g, &idx, 0) != STA_ERR_INVALID ||
        !sta_last_error()[0]) {
        fprintf(stderr, "NULL tensors were not rejected\n");
        return 5;
    }

    int ok = run(STA_F32, in[0], in[1], in[2], in[3], ref[0][0], ref[0][1], ref[0][2], ref[0][3], ref[0][4], &g, &idx,
                 1e-4);
    ok &= run(STA_BF16, inb[0], inb[1], inb[2], inb[3], ref[1][0], ref[1][1], ref[1][2], ref[1][3], ref[1][4], &g,
              &idx, 2e-2);
    printf(ok ? "c abi ok\n" : "c abi MISMATCH\n");
    return ok ? 0 : 1;
}
