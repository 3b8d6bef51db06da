/*
 * Host code of libsta under AddressSanitizer and UndefinedBehaviorSanitizer
 * (test infrastructure): tests/test_host_sanitized.py compiles the
 * library's host-side sources with both sanitizers (device code as usual),
 * links them with the other objects of the build into a shared library and
 * runs this program against it, with no GPU.
 *
 * Only host work is called: status strings, the version, index sizing over
 * a sweep of geometries (whole and cut tiles, both border rules, huge and
 * overflowing extents), and every entry point with malformed arguments,
 * which must be refused before anything is launched (the pointers passed
 * are never dereferenced on the host).  Each refusal must come with a
 * reason from sta_last_error().  Prints "host sanitized ok" on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "libsta.h"

/* the C side of the ABI: enums are int-sized, as the library assumes */
_Static_assert(sizeof(sta_status) == 4 && sizeof(sta_dtype) == 4 && sizeof(sta_layout) == 4, "32-bit enums");

static int failures = 0;
#define EXPECT(c, ...)                      \
    do {                                    \
        if (!(c)) {                         \
            fprintf(stderr, __VA_ARGS__);   \
            fputc('\n', stderr);            \
            ++failures;                     \
        }                                   \
    } while (0)

/* A refused call: not OK, not a HIP error (nothing ran), with a reason. */
#define REFUSED(call)                                                                     \
    do {                                                                                  \
        sta_status s_ = (call);                                                           \
        EXPECT(s_ == STA_ERR_INVALID || s_ == STA_ERR_UNSUPPORTED, "%s returned %d", #call, \
               (int)s_);                                                                  \
        EXPECT(sta_last_error()[0] != 0, "%s left no reason", #call);                     \
    } while (0)

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int main(void)
{
    /* status strings, out-of-range codes included */
    for (int s = -1; s <= 5; ++s) EXPECT(sta_status_str((sta_status)s) != NULL, "no string for %d", s);
    EXPECT(strcmp(sta_status_str(STA_OK), "STA_OK") == 0, "STA_OK string");
    EXPECT(sta_version() >= 10000, "version");

    /* index sizing: valid geometries give sane sizes */
    const int grids[][3] = {{4, 8, 8}, {30, 48, 80}, {5, 7, 9}, {1, 1, 1}, {30, 45, 80}, {3, 100, 2}};
    const int tiles[][3] = {{2, 4, 4}, {6, 8, 8}, {2, 4, 4}, {1, 1, 1}, {6, 8, 8}, {4, 7, 1}};
    const int wins[][3] = {{1, 1, 1}, {3, 3, 5}, {2, 3, 4}, {5, 5, 5}, {99, 99, 99}};
    for (size_t gi = 0; gi < sizeof grids / sizeof grids[0]; ++gi) {
        sta_geom g = {{grids[gi][0], grids[gi][1], grids[gi][2]}, {tiles[gi][0], tiles[gi][1], tiles[gi][2]}};
        const int64_t T = ceil_div(grids[gi][0], tiles[gi][0]) * ceil_div(grids[gi][1], tiles[gi][1]) *
                          ceil_div(grids[gi][2], tiles[gi][2]);
        for (size_t wi = 0; wi < sizeof wins / sizeof wins[0]; ++wi)
            for (int border = 0; border < 2; ++border)
                for (int offs = 0; offs < 2; ++offs) {
                    sta_dim3 w[2] = {{wins[wi][0], wins[wi][1], wins[wi][2]}, {1, 1, 1}};
                    sta_index_opts o = {border, 0};
                    int32_t kv = -1, q = -1;
                    sta_status s = sta_index_dims_ex(&g, 2, w, offs, &o, &kv, &q);
                    EXPECT(s == STA_OK, "dims refused grid %zu window %zu: %s", gi, wi, sta_last_error());
                    EXPECT(kv >= 1 && kv <= T && q >= 1 && q <= T, "dims out of range: %d %d of %lld", kv, q,
                           (long long)T);
                }
    }

    sta_geom g = {{4, 8, 8}, {2, 4, 4}};
    sta_dim3 w[2] = {{3, 3, 3}, {1, 3, 3}};
    int32_t kv = 0, q = 0;
    EXPECT(sta_index_dims(&g, 2, w, 0, NULL, NULL) == STA_OK, "NULL outputs are allowed");

    /* malformed geometries and windows */
    sta_geom bad[] = {{{0, 8, 8}, {2, 4, 4}},   {{4, 8, 8}, {0, 4, 4}},     {{-4, 8, 8}, {2, 4, 4}},
                      {{4, 8, 8}, {2, -4, 4}},  {{1 << 20, 1 << 20, 1 << 20}, {1, 1, 1}},
                      {{2147483647, 2, 2}, {1, 1, 1}}, {{2147483647, 2147483647, 2147483647}, {7, 7, 7}},
                      {{64, 64, 64}, {64, 64, 64}}};   /* the last: 2^18 tokens per tile */
    for (size_t i = 0; i < sizeof bad / sizeof bad[0]; ++i) REFUSED(sta_index_dims(&bad[i], 2, w, 0, &kv, &q));
    REFUSED(sta_index_dims(NULL, 2, w, 0, &kv, &q));
    REFUSED(sta_index_dims(&g, 0, w, 0, &kv, &q));
    REFUSED(sta_index_dims(&g, 2, NULL, 0, &kv, &q));
    sta_dim3 w0[2] = {{3, 0, 3}, {1, 3, 3}};
    REFUSED(sta_index_dims(&g, 2, w0, 0, &kv, &q));
    sta_index_opts bad_border = {7, 0};
    REFUSED(sta_index_dims_ex(&g, 2, w, 0, &bad_border, &kv, &q));

    /* fake device pointers: the calls below must fail their checks first */
    char *p = (char *)(uintptr_t)0x100000;
    const int T = 8;
    EXPECT(sta_index_dims(&g, 2, w, 1, &kv, &q) == STA_OK, "dims");
    sta_index idx = {2, T, kv, q, (int32_t *)p, (int32_t *)p, (int32_t *)p, (int32_t *)p};

    REFUSED(sta_tile_reorder(NULL, p, 2, 256, &g, 0, 0));
    REFUSED(sta_tile_reorder(p, NULL, 2, 256, &g, 0, 0));
    REFUSED(sta_tile_reorder(p, p + 64, -1, 256, &g, 0, 0));
    REFUSED(sta_tile_reorder(p, p + 64, 2, 0, &g, 0, 0));
    REFUSED(sta_tile_reorder(p, p + 64, 2, 256, &bad[0], 0, 0));
    REFUSED(sta_tile_reorder(p, p + 64, INT64_MAX / 2, INT64_MAX / 2, &g, 0, 0));

    sta_index small = idx;
    small.max_kv = 1;
    REFUSED(sta_build_index(&g, 2, w, NULL, &small, 0));
    sta_index wrong_heads = idx;
    wrong_heads.num_heads = 3;
    REFUSED(sta_build_index(&g, 2, w, NULL, &wrong_heads, 0));
    sta_index wrong_tiles = idx;
    wrong_tiles.num_tiles = 9;
    REFUSED(sta_build_index(&g, 2, w, NULL, &wrong_tiles, 0));
    REFUSED(sta_build_index(&g, 2, w, NULL, NULL, 0));
    REFUSED(sta_build_index_ex(&g, 2, w, NULL, &bad_border, &idx, 0));

    const float scale = 0.125f;
    REFUSED(sta_fwd(NULL, p, p, p, (float *)p, 1, 2, 64, STA_BF16, scale, &g, &idx, 0));
    REFUSED(sta_fwd(p, p, p, p, (float *)p, 1, 2, 96, STA_BF16, scale, &g, &idx, 0));
    REFUSED(sta_fwd(p, p, p, p, (float *)p, 0, 2, 64, STA_BF16, scale, &g, &idx, 0));
    REFUSED(sta_fwd(p, p, p, p, (float *)p, 1, 3, 64, STA_BF16, scale, &g, &idx, 0));
    REFUSED(sta_fwd(p, p, p, p, (float *)p, 1, 2, 64, (sta_dtype)9, scale, &g, &idx, 0));
    REFUSED(sta_fwd(p + 1, p, p, p, (float *)p, 1, 2, 64, STA_BF16, scale, &g, &idx, 0));
    REFUSED(sta_fwd(p, p, p, p, (float *)p, 1, 2, 64, STA_BF16, scale, &g, NULL, 0));
    sta_attn_opts bad_text = {-1, 0, 0}, bad_prec = {0, 5, 0}, bad_layout = {0, 0, 9}, raster_text = {3, 0, 1};
    REFUSED(sta_fwd_ex(p, p, p, p, (float *)p, 1, 2, 64, STA_BF16, scale, &g, &idx, &bad_text, 0));
    REFUSED(sta_fwd_ex(p, p, p, p, (float *)p, 1, 2, 64, STA_BF16, scale, &g, &idx, &bad_prec, 0));
    REFUSED(sta_fwd_ex(p, p, p, p, (float *)p, 1, 2, 64, STA_BF16, scale, &g, &idx, &bad_layout, 0));
    REFUSED(sta_fwd_ex(p, p, p, p, (float *)p, 1, 2, 64, STA_BF16, scale, &g, &idx, &raster_text, 0));

    REFUSED(sta_bwd(p, p, p, p, (float *)p, p, p, p, NULL, (float *)p, 1, 2, 64, STA_BF16, scale, &g, &idx, 0));
    REFUSED(sta_bwd(p, p, p, p, (float *)p, p, p, p, p, (float *)p, 1, 2, 32, STA_BF16, scale, &g, &idx, 0));
    REFUSED(sta_bwd_parts(p, p, p, p, (float *)p, p, p, p, p, (float *)p, 1, 2, 64, STA_BF16, scale, &g, &idx, 0,
                          0));
    REFUSED(sta_bwd_parts(p, p, p, p, (float *)p, p, p, p, p, (float *)p, 1, 2, 64, STA_BF16, scale, &g, &idx, 8,
                          0));
    sta_attn_opts fp8 = {0, 1, 0};
    REFUSED(sta_bwd_ex(p, p, p, p, (float *)p, p, p, p, p, (float *)p, 1, 2, 64, STA_BF16, scale, &g, &idx,
                       STA_BWD_ALL, &fp8, 0));

    sta_dim3 r1 = {1, 1, 1}, rneg = {-1, 0, 0}, rbig = {10, 10, 10};
    sta_shift_opts so = {0, 0, 0, 0}, so_bad = {0, 2, 0, 0};
    int32_t *off = (int32_t *)p;
    REFUSED(sta_window_shifts(NULL, p, 1, 2, 64, STA_BF16, scale, &g, w, &r1, &so, off, 0));
    REFUSED(sta_window_shifts(p, p, 1, 2, 64, STA_BF16, scale, &g, w, &rneg, &so, off, 0));
    REFUSED(sta_window_shifts(p, p, 1, 2, 64, STA_BF16, scale, &g, w, &rbig, &so, off, 0));
    REFUSED(sta_window_shifts(p, p, 1, 2, 64, STA_BF16, -1.0f, &g, w, &r1, &so, off, 0));
    REFUSED(sta_window_shifts(p, p, 1, 2, 64, STA_BF16, scale, &g, w, &r1, &so_bad, off, 0));
    REFUSED(sta_window_shifts(p, p, 1, 2, 48, STA_BF16, scale, &g, w, &r1, &so, off, 0));

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("host sanitized ok\n");
    return 0;
}
