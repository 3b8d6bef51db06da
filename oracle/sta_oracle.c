/*
 * sta_oracle.c -- plain CPU oracle for sliding-tile attention (STA).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load this library.  It shares
 * no code, header, table or helper with the HIP library; it is written from
 * the method's definition only, and is deliberately slow and literal:
 * every attention row is computed on its own, from token coordinates, with
 * an explicit membership test for every (query, key) pair, in fp64.
 *
 * What is computed (sources):
 *   - "Fast Video Generation with Sliding Tile Attention" (pith.science
 *     record of arXiv 2502.04507, abstract): 3D full attention over the
 *     (T,H,W) video token grid is replaced by attention restricted to a
 *     local 3D window that slides with the query; STA does this at the
 *     granularity of tiles.
 *   - "MegaSlide-DiT: Memory-Centric Adaptation and Deformable Local
 *     Attention for Efficient Video Diffusion" (abstract): the window of
 *     the local operator is motion-adaptive (3D-DSA).  Here that is an
 *     integer per-query-tile shift of the window (an input; how offsets
 *     would be derived from motion is not stated: parity unpinned).
 *
 * Readings taken where the pages are silent (each is also listed in the
 * design notes):
 *   R1 border: the window keeps its full size and is shifted inward, i.e.
 *      its start is clamped to [0, n - c].
 *   R2 a window wider than the grid covers the whole axis.
 *   R3 window start = q + o - floor(w/2) before clamping (even w leans low).
 *   R4 offsets are integer tile units, one (dt,dh,dw) per query tile, shared
 *      by all heads and batch items, added before clamping.
 *   Options (the `flags` argument of the entry points), for the NEXT-ranked
 *   3D-DSA variants (motion-adaptive windows are not pinned by the pages):
 *   ORACLE_TRUNCATE  border rule instead of R1: per axis the shifted centre
 *                    q + o is clamped into [0, n-1] and the window
 *                    [centre - floor(w/2), centre - floor(w/2) + w - 1] is
 *                    cut at the grid border (so it always holds the clamped
 *                    centre and is never empty).
 *   ORACLE_HEAD_OFFS offsets are [H][T][3], one shift per head and query tile
 *                    (batch items still share them).
 *   Joint text + video sequences (token-type-aware masking, MOD-DiT README
 *   mirror, "Token-Type-Aware Masking"): the attention entry points take
 *   n_text >= 0 text tokens stored after the grid's video tokens; a text
 *   query attends every key and every query attends every text key, while
 *   video-video pairs keep the window rule.
 *   R6 raster order everywhere: t slowest, w fastest (tokens, tiles and the
 *      position inside a tile).
 *   R8 softmax scale is an argument (1/sqrt(D) in every workload).
 *   R9 LSE is the natural log of sum_j exp(scale * q.k_j) over allowed keys.
 *
 * Arithmetic: inputs are fp32 (bf16 inputs arrive upcast, which is exact);
 * every sum is accumulated in double; outputs are double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_TRUNCATE 1
#define ORACLE_HEAD_OFFS 2

/* ------------------------------------------------------------------ */
/* Geometry                                                            */
/* ------------------------------------------------------------------ */

/* Number of tiles along each axis, ceil(grid / tile): where the tile does
 * not divide the grid the last tile of the axis holds the remaining tokens
 * only (no padding tokens exist).  0 for non-positive extents. */
static int tiles_per_axis(const int grid[3], const int tile[3], int n[3])
{
    for (int d = 0; d < 3; ++d) {
        if (grid[d] <= 0 || tile[d] <= 0)
            return 0;
        n[d] = (grid[d] + tile[d] - 1) / tile[d];
    }
    return 1;
}

/* The window of query tile qc (tile coordinates) for window size win and
 * optional offset off: per axis the start s and count c of the allowed
 * tile range [s, s+c).  Readings R1-R4, or the truncating border rule. */
static void window_of(const int n[3], const int win[3], const int qc[3],
                      const int *off, int truncate, int s[3], int c[3])
{
    for (int d = 0; d < 3; ++d) {
        int o = off ? off[d] : 0;                    /* R4 */
        if (truncate) {
            int centre = qc[d] + o;
            if (centre < 0) centre = 0;
            if (centre > n[d] - 1) centre = n[d] - 1;
            int lo = centre - win[d] / 2;
            int hi = lo + win[d] - 1;
            if (lo < 0) lo = 0;
            if (hi > n[d] - 1) hi = n[d] - 1;
            s[d] = lo;
            c[d] = hi - lo + 1;
        } else {
            int cnt = win[d] < n[d] ? win[d] : n[d];     /* R2 */
            int start = qc[d] + o - win[d] / 2;          /* R3 */
            if (start < 0) start = 0;                    /* R1 */
            if (start > n[d] - cnt) start = n[d] - cnt;  /* R1 */
            s[d] = start;
            c[d] = cnt;
        }
    }
}

/* Offset triple of query tile q under head h (or NULL). */
static const int *offset_of(const int *offsets, int flags, int h, int T, int q)
{
    if (!offsets)
        return NULL;
    return offsets + 3 * ((int64_t)((flags & ORACLE_HEAD_OFFS) ? h * T : 0) + q);
}

static void tile_coords(int id, const int n[3], int tc[3])
{
    tc[2] = id % n[2];
    tc[1] = (id / n[2]) % n[1];
    tc[0] = id / (n[2] * n[1]);
}

static int tile_in_window(const int kc[3], const int s[3], const int c[3])
{
    for (int d = 0; d < 3; ++d)
        if (kc[d] < s[d] || kc[d] >= s[d] + c[d])
            return 0;
    return 1;
}

/* Tile coordinates of raster token r (R6). */
static void token_tile(int64_t r, const int grid[3], const int tile[3], int tc[3])
{
    int w = (int)(r % grid[2]);
    int h = (int)((r / grid[2]) % grid[1]);
    int t = (int)(r / ((int64_t)grid[2] * grid[1]));
    tc[0] = t / tile[0];
    tc[1] = h / tile[1];
    tc[2] = w / tile[2];
}

/* ------------------------------------------------------------------ */
/* Token permutation                                                   */
/* ------------------------------------------------------------------ */

/* perm[r] = position of raster token r in tile-contiguous order: tiles in
 * raster order of tile coordinates, tokens inside a tile in raster order of
 * their in-tile coordinates (R6).  Positions are handed out one by one in
 * that order, so a tile cut by the grid border holds exactly its tokens and
 * the next tile starts right after them. */
int oracle_perm(const int grid[3], const int tile[3], int64_t *perm)
{
    int n[3];
    if (!tiles_per_axis(grid, tile, n))
        return 0;
    int64_t pos = 0;
    for (int a = 0; a < n[0]; ++a)
        for (int b = 0; b < n[1]; ++b)
            for (int c = 0; c < n[2]; ++c)
                for (int t = a * tile[0]; t < (a + 1) * tile[0] && t < grid[0]; ++t)
                    for (int h = b * tile[1]; h < (b + 1) * tile[1] && h < grid[1]; ++h)
                        for (int w = c * tile[2]; w < (c + 1) * tile[2] && w < grid[2]; ++w)
                            perm[((int64_t)t * grid[1] + h) * grid[2] + w] = pos++;
    return 1;
}

/* ------------------------------------------------------------------ */
/* Block-sparse index                                                  */
/* ------------------------------------------------------------------ */

/* For every head h and query tile q: the ascending list of key tiles k in
 * the window of q (kv_idx[h][q][0..kv_cnt), padded with -1 to max_kv), and
 * the transposed lists: for every key tile k, the ascending query tiles q
 * whose window holds k (q_idx[h][k][0..q_cnt), padded -1 to max_q).
 * Brute force over all (q, k) pairs.  Returns 0 if a list would not fit or
 * the geometry is invalid, else 1.  windows: [H][3]; offsets: [T][3] (or
 * [H][T][3] with ORACLE_HEAD_OFFS) or NULL. */
int oracle_index(const int grid[3], const int tile[3], int H,
                 const int *windows, const int *offsets, int flags,
                 int max_kv, int32_t *kv_idx, int32_t *kv_cnt,
                 int max_q, int32_t *q_idx, int32_t *q_cnt)
{
    int n[3];
    if (!tiles_per_axis(grid, tile, n))
        return 0;
    int T = n[0] * n[1] * n[2];
    for (int h = 0; h < H; ++h) {
        const int *win = windows + 3 * h;
        for (int q = 0; q < T; ++q) {
            int qc[3], s[3], c[3], cnt = 0;
            tile_coords(q, n, qc);
            window_of(n, win, qc, offset_of(offsets, flags, h, T, q), flags & ORACLE_TRUNCATE, s, c);
            int32_t *row = kv_idx + ((int64_t)h * T + q) * max_kv;
            for (int j = 0; j < max_kv; ++j) row[j] = -1;
            for (int k = 0; k < T; ++k) {
                int kc[3];
                tile_coords(k, n, kc);
                if (tile_in_window(kc, s, c)) {
                    if (cnt >= max_kv) return 0;
                    row[cnt++] = k;
                }
            }
            kv_cnt[(int64_t)h * T + q] = cnt;
        }
        for (int k = 0; k < T; ++k) {
            int kc[3], cnt = 0;
            tile_coords(k, n, kc);
            int32_t *row = q_idx + ((int64_t)h * T + k) * max_q;
            for (int j = 0; j < max_q; ++j) row[j] = -1;
            for (int q = 0; q < T; ++q) {
                int qc[3], s[3], c[3];
                tile_coords(q, n, qc);
                window_of(n, win, qc, offset_of(offsets, flags, h, T, q), flags & ORACLE_TRUNCATE, s, c);
                if (tile_in_window(kc, s, c)) {
                    if (cnt >= max_q) return 0;
                    row[cnt++] = q;
                }
            }
            q_cnt[(int64_t)h * T + k] = cnt;
        }
    }
    return 1;
}

/* ------------------------------------------------------------------ */
/* Attention                                                           */
/* ------------------------------------------------------------------ */

typedef struct {
    int B, H, D;
    int grid[3], tile[3], n[3];
    int64_t N;                       /* rows per (b, h): Nv video + ntext text tokens */
    int64_t Nv;
    int ntext;
    const float *q, *k, *v, *dout;   /* [B][H][N][D], raster token order */
    const int *windows, *offsets;
    int flags;
    double scale;
} problem;

static int make_problem(problem *p, int B, int H, int D, const int grid[3],
                        const int tile[3], const int *windows, const int *offsets,
                        int flags, int ntext, double scale, const float *q, const float *k,
                        const float *v, const float *dout)
{
    if (B <= 0 || H <= 0 || D <= 0 || ntext < 0 || !tiles_per_axis(grid, tile, p->n))
        return 0;
    p->B = B; p->H = H; p->D = D;
    memcpy(p->grid, grid, sizeof p->grid);
    memcpy(p->tile, tile, sizeof p->tile);
    p->Nv = (int64_t)grid[0] * grid[1] * grid[2];
    p->ntext = ntext;
    p->N = p->Nv + ntext;
    p->q = q; p->k = k; p->v = v; p->dout = dout;
    p->windows = windows; p->offsets = offsets;
    p->flags = flags;
    p->scale = scale;
    return 1;
}

static const float *row_of(const problem *p, const float *x, int b, int h, int64_t i)
{
    return x + (((int64_t)b * p->H + h) * p->N + i) * p->D;
}

/* Is key token j allowed for query token i under head h?  A text token
 * (index >= Nv) on either side makes the pair allowed; between video tokens
 * the mask is M_h[i,j] = [tile(j) lies in the window of tile(i)]. */
static int allowed(const problem *p, int h, int64_t i, int64_t j)
{
    if (i >= p->Nv || j >= p->Nv)
        return 1;
    int qc[3], kc[3], s[3], c[3];
    token_tile(i, p->grid, p->tile, qc);
    token_tile(j, p->grid, p->tile, kc);
    int qid = (qc[0] * p->n[1] + qc[1]) * p->n[2] + qc[2];
    int T = p->n[0] * p->n[1] * p->n[2];
    window_of(p->n, p->windows + 3 * h, qc, offset_of(p->offsets, p->flags, h, T, qid),
              p->flags & ORACLE_TRUNCATE, s, c);
    return tile_in_window(kc, s, c);
}

static double dot(const float *a, const float *b, int D)
{
    double acc = 0.0;
    for (int d = 0; d < D; ++d)
        acc += (double)a[d] * (double)b[d];
    return acc;
}

/* Scores s_ij = scale * <q_i, k_j> for every allowed key j of query row i;
 * fills js[] and ss[] and returns how many. */
static int64_t row_scores(const problem *p, int b, int h, int64_t i,
                          int64_t *js, double *ss)
{
    const float *qi = row_of(p, p->q, b, h, i);
    int64_t m = 0;
    for (int64_t j = 0; j < p->N; ++j) {
        if (!allowed(p, h, i, j))
            continue;
        js[m] = j;
        ss[m] = p->scale * dot(qi, row_of(p, p->k, b, h, j), p->D);
        ++m;
    }
    return m;
}

/* Softmax normaliser of row i: LSE_i = m_i + ln sum_j exp(s_ij - m_i). */
static double row_lse(const double *ss, int64_t m)
{
    double mx = -INFINITY, sum = 0.0;
    for (int64_t a = 0; a < m; ++a)
        if (ss[a] > mx) mx = ss[a];
    for (int64_t a = 0; a < m; ++a)
        sum += exp(ss[a] - mx);
    return mx + log(sum);
}

static void split_row_id(const problem *p, int64_t id, int *b, int *h, int64_t *i)
{
    *i = id % p->N;
    *h = (int)((id / p->N) % p->H);
    *b = (int)(id / (p->N * p->H));
}

/*
 * Forward, for the requested rows only.  rows[r] is a flat row id
 * (b*H + h)*N + i with i a RASTER token index; o is [n_rows][D] and lse is
 * [n_rows] (double).  O_i = sum_j exp(s_ij - LSE_i) v_j over allowed j.
 * Returns 0 on invalid arguments, else 1.
 */
int oracle_fwd(int B, int H, int D, const int grid[3], const int tile[3],
               const int *windows, const int *offsets, int flags, int ntext, double scale,
               const float *q, const float *k, const float *v,
               int64_t n_rows, const int64_t *rows, double *o, double *lse)
{
    problem p;
    if (!make_problem(&p, B, H, D, grid, tile, windows, offsets, flags, ntext, scale, q, k, v, NULL))
        return 0;
    int ok = 1;
#pragma omp parallel
    {
        int64_t *js = (int64_t *)malloc(sizeof(int64_t) * p.N);
        double *ss = (double *)malloc(sizeof(double) * p.N);
        double *acc = (double *)malloc(sizeof(double) * D);
        if (!js || !ss || !acc) {
#pragma omp atomic write
            ok = 0;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < n_rows; ++r) {
                int b, h; int64_t i;
                split_row_id(&p, rows[r], &b, &h, &i);
                int64_t m = row_scores(&p, b, h, i, js, ss);
                double L = row_lse(ss, m);
                for (int d = 0; d < D; ++d) acc[d] = 0.0;
                for (int64_t a = 0; a < m; ++a) {
                    double pij = exp(ss[a] - L);
                    const float *vj = row_of(&p, p.v, b, h, js[a]);
                    for (int d = 0; d < D; ++d)
                        acc[d] += pij * (double)vj[d];
                }
                for (int d = 0; d < D; ++d) o[r * D + d] = acc[d];
                lse[r] = L;
            }
        }
        free(js); free(ss); free(acc);
    }
    return ok;
}

/* Per-row backward statistics of query row i: LSE_i and
 * Delta_i = sum_j P_ij dP_ij with P_ij = exp(s_ij - LSE_i) and
 * dP_ij = <dO_i, v_j>.  Leaves the row's allowed keys and scores in js/ss
 * and returns how many there are. */
static int64_t row_stats(const problem *p, int b, int h, int64_t i,
                         int64_t *js, double *ss, double *lse, double *delta)
{
    int64_t m = row_scores(p, b, h, i, js, ss);
    double L = row_lse(ss, m);
    const float *doi = row_of(p, p->dout, b, h, i);
    double dl = 0.0;
    for (int64_t a = 0; a < m; ++a)
        dl += exp(ss[a] - L) * dot(doi, row_of(p, p->v, b, h, js[a]), p->D);
    *lse = L;
    *delta = dl;
    return m;
}

/*
 * Backward, for the requested rows only.
 *   dS_ij = P_ij (dP_ij - Delta_i)
 *   dQ_i  = scale * sum_j dS_ij k_j              (qrows -> dq [n_q][D])
 *   dK_j  = scale * sum_i dS_ij q_i              (krows -> dk [n_k][D])
 *   dV_j  = sum_i P_ij dO_i                      (krows -> dv [n_k][D])
 * Row ids are flat (b*H + h)*N + raster index, as in oracle_fwd.  For a key
 * row j, the sums run over every query row i whose window holds tile(j);
 * their LSE_i and Delta_i are computed from the definition first.
 * Returns 0 on invalid arguments or allocation failure, else 1.
 */
int oracle_bwd(int B, int H, int D, const int grid[3], const int tile[3],
               const int *windows, const int *offsets, int flags, int ntext, double scale,
               const float *q, const float *k, const float *v, const float *dout,
               int64_t n_q, const int64_t *qrows, double *dq,
               int64_t n_k, const int64_t *krows, double *dk, double *dv)
{
    problem p;
    if (!make_problem(&p, B, H, D, grid, tile, windows, offsets, flags, ntext, scale, q, k, v, dout))
        return 0;
    int ok = 1;

    /* dQ rows */
#pragma omp parallel
    {
        int64_t *js = (int64_t *)malloc(sizeof(int64_t) * p.N);
        double *ss = (double *)malloc(sizeof(double) * p.N);
        double *acc = (double *)malloc(sizeof(double) * D);
        if (!js || !ss || !acc) {
#pragma omp atomic write
            ok = 0;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < n_q; ++r) {
                int b, h; int64_t i;
                split_row_id(&p, qrows[r], &b, &h, &i);
                double L, dl;
                int64_t m = row_stats(&p, b, h, i, js, ss, &L, &dl);
                const float *doi = row_of(&p, p.dout, b, h, i);
                for (int d = 0; d < D; ++d) acc[d] = 0.0;
                for (int64_t a = 0; a < m; ++a) {
                    double pij = exp(ss[a] - L);
                    double dpij = dot(doi, row_of(&p, p.v, b, h, js[a]), D);
                    double dsij = pij * (dpij - dl);
                    const float *kj = row_of(&p, p.k, b, h, js[a]);
                    for (int d = 0; d < D; ++d)
                        acc[d] += dsij * (double)kj[d];
                }
                for (int d = 0; d < D; ++d) dq[r * D + d] = scale * acc[d];
            }
        }
        free(js); free(ss); free(acc);
    }
    if (!ok || n_k == 0)
        return ok;

    /* Which query rows do the requested key rows need?  need[(b*H+h)*N+i]. */
    int64_t total = (int64_t)B * H * p.N;
    char *need = (char *)calloc((size_t)total, 1);
    double *lse = (double *)malloc(sizeof(double) * total);
    double *dlt = (double *)malloc(sizeof(double) * total);
    if (!need || !lse || !dlt) {
        free(need); free(lse); free(dlt);
        return 0;
    }
    for (int64_t r = 0; r < n_k; ++r) {
        int b, h; int64_t j;
        split_row_id(&p, krows[r], &b, &h, &j);
        for (int64_t i = 0; i < p.N; ++i)
            if (allowed(&p, h, i, j))
                need[((int64_t)b * H + h) * p.N + i] = 1;
    }
#pragma omp parallel
    {
        int64_t *js = (int64_t *)malloc(sizeof(int64_t) * p.N);
        double *ss = (double *)malloc(sizeof(double) * p.N);
        if (!js || !ss) {
#pragma omp atomic write
            ok = 0;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t id = 0; id < total; ++id) {
                if (!need[id]) continue;
                int b, h; int64_t i;
                split_row_id(&p, id, &b, &h, &i);
                row_stats(&p, b, h, i, js, ss, &lse[id], &dlt[id]);
            }
        }
        free(js); free(ss);
    }
    if (ok) {
#pragma omp parallel
        {
            double *ak = (double *)malloc(sizeof(double) * D);
            double *av = (double *)malloc(sizeof(double) * D);
            if (!ak || !av) {
#pragma omp atomic write
                ok = 0;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int64_t r = 0; r < n_k; ++r) {
                    int b, h; int64_t j;
                    split_row_id(&p, krows[r], &b, &h, &j);
                    const float *kj = row_of(&p, p.k, b, h, j);
                    const float *vj = row_of(&p, p.v, b, h, j);
                    for (int d = 0; d < D; ++d) { ak[d] = 0.0; av[d] = 0.0; }
                    for (int64_t i = 0; i < p.N; ++i) {
                        if (!allowed(&p, h, i, j)) continue;
                        int64_t id = ((int64_t)b * H + h) * p.N + i;
                        const float *qi = row_of(&p, p.q, b, h, i);
                        const float *doi = row_of(&p, p.dout, b, h, i);
                        double pij = exp(scale * dot(qi, kj, D) - lse[id]);
                        double dsij = pij * (dot(doi, vj, D) - dlt[id]);
                        for (int d = 0; d < D; ++d) {
                            ak[d] += dsij * (double)qi[d];
                            av[d] += pij * (double)doi[d];
                        }
                    }
                    for (int d = 0; d < D; ++d) {
                        dk[r * D + d] = scale * ak[d];
                        dv[r * D + d] = av[d];
                    }
                }
            }
            free(ak); free(av);
        }
    }
    free(need); free(lse); free(dlt);
    return ok;
}
