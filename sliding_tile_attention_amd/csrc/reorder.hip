// Raster <-> tile-contiguous token permutation (byte-generic gather).
//
// A run of consecutive tokens along w inside one tile (tw of them, fewer in
// a tile cut by the grid border) is contiguous in both orders, so the copy
// moves whole runs.  One
// thread owns one vector-sized chunk of one run and walks it through all
// `outer` slabs, so the index arithmetic is paid once per chunk position
// and every wave reads and writes contiguous, fully coalesced memory.
// Text rows that follow the grid's tokens in a slab are copied in place.
#include "common.h"

namespace sta {

template <typename V>
__global__ __launch_bounds__(256) void reorder_kernel(const V *__restrict__ src, V *__restrict__ dst,
                                                      int64_t outer, int64_t slab, int64_t row_vec,
                                                      int64_t run_vec, int64_t chunks, int64_t text_chunks, Geo g,
                                                      int inverse)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < chunks + text_chunks;
         gid += stride) {
        int64_t s0, d0;
        if (gid < chunks) {
            const int64_t u = gid / run_vec;     // run index, raster order of (t, h, w-tile)
            const int64_t c = gid - u * run_vec; // chunk inside the run
            const int jw = (int)(u % g.nw);
            const int64_t th_ = u / g.nw;
            const int h = (int)(th_ % g.gh);
            const int t = (int)(th_ / g.gh);
            const int vw = g.gw - jw * g.tw < g.tw ? g.gw - jw * g.tw : g.tw;   // tokens of this run
            if (c >= vw * row_vec) continue;     // past a run cut by the grid border
            const int64_t raster = ((int64_t)t * g.gh + h) * g.gw + (int64_t)jw * g.tw;
            const int tile_id = ((t / g.tt) * g.nh + h / g.th) * g.nw + jw;
            const Span sp = tile_span(g, tile_id);
            const int vh = g.gh - (h / g.th) * g.th < g.th ? g.gh - (h / g.th) * g.th : g.th;
            const int64_t tiled = sp.start + ((int64_t)(t % g.tt) * vh + h % g.th) * vw;
            s0 = (inverse ? tiled : raster) * row_vec + c;
            d0 = (inverse ? raster : tiled) * row_vec + c;
        } else {                                 // text rows keep their place
            s0 = d0 = g.N * row_vec + (gid - chunks);
        }
        int64_t o = 0;
        for (; o + 4 <= outer; o += 4) {
            V a0 = __builtin_nontemporal_load(src + s0 + (o + 0) * slab);
            V a1 = __builtin_nontemporal_load(src + s0 + (o + 1) * slab);
            V a2 = __builtin_nontemporal_load(src + s0 + (o + 2) * slab);
            V a3 = __builtin_nontemporal_load(src + s0 + (o + 3) * slab);
            __builtin_nontemporal_store(a0, dst + d0 + (o + 0) * slab);
            __builtin_nontemporal_store(a1, dst + d0 + (o + 1) * slab);
            __builtin_nontemporal_store(a2, dst + d0 + (o + 2) * slab);
            __builtin_nontemporal_store(a3, dst + d0 + (o + 3) * slab);
        }
        for (; o < outer; ++o)
            __builtin_nontemporal_store(__builtin_nontemporal_load(src + s0 + o * slab), dst + d0 + o * slab);
    }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// V is the copy unit; the caller picks one that divides row_bytes and the
// pointers' alignment, so token offsets are whole numbers of V.
template <typename V>
static sta_status run(const void *src, void *dst, int64_t outer, int64_t row_bytes, const Geo &g,
                      bool inverse, hipStream_t s)
{
    const int64_t vb = sizeof(V);
    const int64_t row_vec = row_bytes / vb;      // units per token row
    const int64_t run_vec = g.tw * row_vec;      // units per run of tw tokens
    const int64_t chunks = (int64_t)g.gt * g.gh * g.nw * run_vec;   // runs of the (t, h, w-tile) grid
    const int64_t text_chunks = (int64_t)g.text * row_vec;
    const int64_t slab = g.S * row_vec;
    int64_t blocks = (chunks + text_chunks + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;    // grid-stride loop covers the rest
    hipLaunchKernelGGL(reorder_kernel<V>, dim3((unsigned)blocks), dim3(256), 0, s, (const V *)src, (V *)dst,
                       outer, slab, row_vec, run_vec, chunks, text_chunks, g, inverse ? 1 : 0);
    return check_launch();
}

sta_status launch_reorder(const void *src, void *dst, int64_t outer, int64_t row_bytes, const Geo &g,
                          bool inverse, hipStream_t s)
{
    const uintptr_t a = (uintptr_t)src | (uintptr_t)dst;
    if (row_bytes % 16 == 0 && (a & 15) == 0)
        return run<u32x4>(src, dst, outer, row_bytes, g, inverse, s);
    if (row_bytes % 4 == 0 && (a & 3) == 0)
        return run<unsigned int>(src, dst, outer, row_bytes, g, inverse, s);
    return run<unsigned char>(src, dst, outer, row_bytes, g, inverse, s);
}

}  // namespace sta
