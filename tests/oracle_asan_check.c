/*
 * Memory and undefined-behaviour check of the CPU oracle (test
 * infrastructure): tests/test_oracle_sanitized.py compiles this file
 * together with oracle/sta_oracle.c under AddressSanitizer and
 * UndefinedBehaviorSanitizer (abort on the first report) and runs it.
 *
 * Every entry point is driven on grids whose tiles are cut by the border,
 * with per-head windows and shifts, both border rules, joint text tokens,
 * lists sized exactly and one too small, and invalid arguments.  Beyond
 * "no report", the outputs are checked against what the definitions fix:
 *   - the token order is a permutation;
 *   - the list counts equal the number of entries before the -1 padding,
 *     and the transposed lists hold the same pairs as the forward lists;
 *   - sum_j dV_j = sum_i dO_i and sum_j dK_j = 0 per (batch, head), since
 *     each softmax row sums to one and dS has zero row sums.
 * Prints "oracle sanitized ok" and exits 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#define ORACLE_TRUNCATE 1
#define ORACLE_HEAD_OFFS 2

int oracle_perm(const int grid[3], const int tile[3], int64_t *perm);
int oracle_index(const int grid[3], const int tile[3], int H, const int *windows, const int *offsets, int flags,
                 int max_kv, int32_t *kv_idx, int32_t *kv_cnt, int max_q, int32_t *q_idx, int32_t *q_cnt);
int oracle_fwd(int B, int H, int D, const int grid[3], const int tile[3], const int *windows, const int *offsets,
               int flags, int ntext, double scale, const float *q, const float *k, const float *v, int64_t n_rows,
               const int64_t *rows, double *o, double *lse);
int oracle_bwd(int B, int H, int D, const int grid[3], const int tile[3], const int *windows, const int *offsets,
               int flags, int ntext, double scale, const float *q, const float *k, const float *v,
               const float *dout, int64_t n_q, const int64_t *qrows, double *dq, int64_t n_k,
               const int64_t *krows, double *dk, double *dv);

static int failures = 0;
#define EXPECT(c, ...)                      \
    do {                                    \
        if (!(c)) {                         \
            fprintf(stderr, __VA_ARGS__);   \
            fputc('\n', stderr);            \
            ++failures;                     \
        }                                   \
    } while (0)

static uint32_t rng = 12345u;
static float uniform(void)
{
    rng = rng * 1664525u + 1013904223u;
    return (float)(rng >> 8) * (1.0f / 16777216.0f) * 2.0f - 1.0f;
}

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

static void check_perm(const int grid[3], const int tile[3])
{
    const int64_t n = (int64_t)grid[0] * grid[1] * grid[2];
    int64_t *perm = malloc(sizeof(int64_t) * n);
    char *seen = calloc((size_t)n, 1);
    EXPECT(oracle_perm(grid, tile, perm), "perm rejected a valid geometry");
    for (int64_t r = 0; r < n; ++r) {
        EXPECT(perm[r] >= 0 && perm[r] < n, "perm[%lld] out of range", (long long)r);
        if (perm[r] >= 0 && perm[r] < n) {
            EXPECT(!seen[perm[r]], "perm hits %lld twice", (long long)perm[r]);
            seen[perm[r]] = 1;
        }
    }
    free(perm);
    free(seen);
}

/* Index with exact list sizes, then with the forward lists one short. */
static void check_index(const int grid[3], const int tile[3], int H, const int *windows, const int *offsets,
                        int flags)
{
    const int T = ceil_div(grid[0], tile[0]) * ceil_div(grid[1], tile[1]) * ceil_div(grid[2], tile[2]);
    int32_t *kv = malloc(sizeof(int32_t) * H * T * T), *kc = malloc(sizeof(int32_t) * H * T);
    int32_t *qi = malloc(sizeof(int32_t) * H * T * T), *qc = malloc(sizeof(int32_t) * H * T);
    EXPECT(oracle_index(grid, tile, H, windows, offsets, flags, T, kv, kc, T, qi, qc), "index rejected");
    int max_cnt = 0;
    for (int h = 0; h < H; ++h)
        for (int t = 0; t < T; ++t) {
            const int32_t *row = kv + ((int64_t)h * T + t) * T;
            int n = 0;
            while (n < T && row[n] >= 0) ++n;
            EXPECT(n == kc[h * T + t], "kv count %d vs %d entries", kc[h * T + t], n);
            if (n > max_cnt) max_cnt = n;
            for (int j = 0; j < n; ++j) {
                /* pair (t, row[j]) must appear in the transposed list of row[j] */
                const int32_t *tr = qi + ((int64_t)h * T + row[j]) * T;
                int found = 0;
                for (int a = 0; a < qc[h * T + row[j]]; ++a) found |= tr[a] == t;
                EXPECT(found, "pair (%d,%d) of head %d missing from the transposed list", t, row[j], h);
            }
        }
    int64_t fwd_pairs = 0, bwd_pairs = 0;
    for (int i = 0; i < H * T; ++i) {
        fwd_pairs += kc[i];
        bwd_pairs += qc[i];
    }
    EXPECT(fwd_pairs == bwd_pairs, "pair counts differ: %lld vs %lld", (long long)fwd_pairs, (long long)bwd_pairs);
    /* lists one entry too small: refused, and nothing written past them */
    if (max_cnt > 1) {
        const int m = max_cnt - 1;
        int32_t *small = malloc(sizeof(int32_t) * H * T * m);
        EXPECT(!oracle_index(grid, tile, H, windows, offsets, flags, m, small, kc, T, qi, qc),
               "index accepted lists of %d for %d entries", m, max_cnt);
        free(small);
    }
    free(kv);
    free(kc);
    free(qi);
    free(qc);
}

/* Forward and backward over every row of a small problem; the column-sum
 * identities of dK and dV; the forward's LSE is finite. */
static void check_attention(int B, int H, int D, const int grid[3], const int tile[3], const int *windows,
                            const int *offsets, int flags, int ntext)
{
    const int64_t N = (int64_t)grid[0] * grid[1] * grid[2] + ntext, rows = (int64_t)B * H * N;
    float *x[4];
    for (int t = 0; t < 4; ++t) {
        x[t] = malloc(sizeof(float) * rows * D);
        for (int64_t i = 0; i < rows * D; ++i) x[t][i] = uniform();
    }
    int64_t *ids = malloc(sizeof(int64_t) * rows);
    for (int64_t i = 0; i < rows; ++i) ids[i] = i;
    double *o = malloc(sizeof(double) * rows * D), *lse = malloc(sizeof(double) * rows);
    double *dq = malloc(sizeof(double) * rows * D), *dk = malloc(sizeof(double) * rows * D);
    double *dv = malloc(sizeof(double) * rows * D);
    const double scale = 1.0 / sqrt((double)D);
    EXPECT(oracle_fwd(B, H, D, grid, tile, windows, offsets, flags, ntext, scale, x[0], x[1], x[2], rows, ids, o,
                      lse),
           "fwd rejected");
    EXPECT(oracle_bwd(B, H, D, grid, tile, windows, offsets, flags, ntext, scale, x[0], x[1], x[2], x[3], rows, ids,
                      dq, rows, ids, dk, dv),
           "bwd rejected");
    for (int64_t i = 0; i < rows; ++i) EXPECT(isfinite(lse[i]), "lse[%lld] not finite", (long long)i);
    for (int bh = 0; bh < B * H; ++bh)
        for (int d = 0; d < D; ++d) {
            double sdk = 0, sdv = 0, sdo = 0, mag = 0;
            for (int64_t j = 0; j < N; ++j) {
                const int64_t r = (int64_t)bh * N + j;
                sdk += dk[r * D + d];
                sdv += dv[r * D + d];
                sdo += x[3][r * D + d];
                mag += fabs(dk[r * D + d]);
            }
            EXPECT(fabs(sdv - sdo) <= 1e-10 * (1 + fabs(sdo)), "sum dV %g vs sum dO %g", sdv, sdo);
            EXPECT(fabs(sdk) <= 1e-10 * (1 + mag), "sum dK %g (scale %g)", sdk, mag);
        }
    /* invalid arguments are refused before anything is read */
    EXPECT(!oracle_fwd(0, H, D, grid, tile, windows, offsets, flags, ntext, scale, x[0], x[1], x[2], rows, ids, o, lse),
           "fwd accepted B = 0");
    EXPECT(!oracle_bwd(B, H, D, grid, tile, windows, offsets, flags, -1, scale, x[0], x[1], x[2], x[3], rows, ids, dq,
                       rows, ids, dk, dv),
           "bwd accepted n_text = -1");
    for (int t = 0; t < 4; ++t) free(x[t]);
    free(ids);
    free(o);
    free(lse);
    free(dq);
    free(dk);
    free(dv);
}

int main(void)
{
    const int whole[3] = {4, 8, 8}, whole_tile[3] = {2, 4, 4};
    const int cut[3] = {5, 7, 9}, cut_tile[3] = {2, 4, 4};   /* 3 x 2 x 3 tiles, all axes cut */
    const int bad_tile[3] = {0, 4, 4};
    int64_t dummy[1];
    EXPECT(!oracle_perm(cut, bad_tile, dummy), "perm accepted a zero tile extent");

    check_perm(whole, whole_tile);
    check_perm(cut, cut_tile);

    const int H = 2, T = 3 * 2 * 3;
    const int windows[2 * 3] = {3, 1, 3, 2, 3, 1};          /* even and odd extents */
    int head_offs[2 * T * 3], offs[T * 3];
    for (int i = 0; i < 2 * T * 3; ++i) head_offs[i] = (i * 5 + 1) % 5 - 2;   /* -2 .. 2 */
    for (int i = 0; i < T * 3; ++i) offs[i] = (i * 7 + 3) % 3 - 1;            /* -1 .. 1 */
    for (int flags = 0; flags < 4; ++flags) {
        const int *o = flags & ORACLE_HEAD_OFFS ? head_offs : offs;
        check_index(cut, cut_tile, H, windows, o, flags);
        check_index(cut, cut_tile, H, windows, NULL, flags & ORACLE_TRUNCATE);
    }
    const int w8[2 * 3] = {3, 3, 3, 3, 3, 3};
    check_index(whole, whole_tile, H, w8, NULL, 0);

    check_attention(2, H, 8, cut, cut_tile, windows, head_offs, ORACLE_TRUNCATE | ORACLE_HEAD_OFFS, 0);
    check_attention(1, H, 8, cut, cut_tile, windows, offs, 0, 5);
    check_attention(1, 1, 16, whole, whole_tile, w8, NULL, 0, 3);

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitized ok\n");
    return 0;
}
