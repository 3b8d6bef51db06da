// Work split of the attention kernels over the chip's 8 XCDs.
//
// A query- or key-stationary kernel has rblocks row blocks of every tile and
// text pseudo-tile of every (b, h) slab, ordered slab by slab (work index
// = (bh * TT + tile slot) * rblocks + rb).  Workgroups go to XCD (block
// index mod 8), each XCD with an L2 of its own.  XCD x takes one contiguous
// range of that order -- neighbouring windows of one head share its L2 --
// and the ranges are cut at equal COST rather than equal item counts: the
// cost of a slab is the number of key tiles its row blocks walk (its list
// set's listed tile pairs, plus the text pseudo-tiles), which differs between
// heads with different window sizes (up to 4.6x between 3x3x3 and 5x5x5
// windows).  The slabs are first ordered by descending cost (ties keep
// their order), so that every XCD starts on its heaviest slabs and ends on
// its lightest: the longest items never trail at the end of a launch.
// Equal slabs keep their order and get equal ranges, the plain contiguous
// split.  Within a slab the cost is taken as uniform per item.  A launch has
// G blocks per XCD (twice the mean share, work_blocks); a range is capped
// at G items, and the ranges after it take up what the cap leaves.
//
// A key-stationary walk (dK/dV) also gets an order of the video tiles inside
// a slab: by descending length of their transposed lists, ties in tile
// order.  Those lengths differ between key tiles (the windows moved inward
// at the grid border overlap there: 12 to 140 query tiles at the 720p
// workload); in plain tile order the workgroups sharing an XCD walk lists
// of different lengths, drift out of step and stop sharing the query blocks
// they copy through L2.  Sorted, the workgroups that run together walk
// equally long lists of neighbouring tiles in step, and the heaviest tiles
// start first.  Text pseudo-tiles keep their place before the video tiles.
//
// Workspace layout (plan_bytes): int split[9] at 0 and at int 9 the offset
// (in ints) of the tile order or -1 (plan_tile), int order[BH] at 64 bytes
// (order[r] = the slab of rank r), int64 cost[IH] after it, then (with a
// tile order) int tiles[IH][T] (tiles[h][i] = the video tile at position i)
// and int64 prefix[IH][TT + 1] (running cost of the slots in walk order).
#include "common.h"

namespace sta {

// Plan layout: split[9] and the tile-order offset in the first 64 bytes,
// the slab order, the slab costs, then (with a tile order) the tiles and the
// per-list-set running cost of the slots in walk order (text slots first).
struct PlanLayout {
    size_t order, cost, tiles, prefix, bytes;
};

static bool orders_tiles(const Geo &g, int IH) { return g.T <= kMaxOrderedTiles && (int64_t)IH * g.TT < (1LL << 26); }

static PlanLayout plan_layout(int IH, int64_t BH, const Geo *tile_order)
{
    PlanLayout l;
    l.order = 64;
    l.cost = l.order + (((size_t)BH * 4 + 7) & ~(size_t)7);
    l.tiles = l.cost + (size_t)IH * 8;
    l.prefix = l.bytes = l.tiles;
    if (tile_order && orders_tiles(*tile_order, IH)) {
        l.prefix = l.tiles + (((size_t)IH * tile_order->T * 4 + 7) & ~(size_t)7);
        l.bytes = l.prefix + (size_t)IH * (tile_order->TT + 1) * 8;
    }
    return l;
}

// One workgroup per list set h: the rank of every video tile by (descending
// list length, tile index), each thread counting over the set's lengths in
// LDS (T <= kMaxOrderedTiles: at most T^2 / 256 steps per thread), then the
// running cost of the walk's slots: a text slot walks all TT tiles, the
// video tile at position i its list plus the Tt text pseudo-tiles.
__global__ __launch_bounds__(256) void tile_order_kernel(const int32_t *__restrict__ walk_cnt, Geo g,
                                                         int *__restrict__ tiles, long long *__restrict__ prefix)
{
    extern __shared__ int lds[];
    int *len = lds, *sorted = lds + g.T;              // T lengths; the same in walk order
    __shared__ long long part[257];
    const int T = g.T, h = blockIdx.x;
    const int32_t *c = walk_cnt + (int64_t)h * T;
    for (int t = threadIdx.x; t < T; t += blockDim.x) len[t] = c[t];
    __syncthreads();
    for (int t = threadIdx.x; t < T; t += blockDim.x) {
        const int lt = len[t];
        int r = 0;
        for (int m = 0; m < T; ++m) r += (len[m] > lt) | ((len[m] == lt) & (m < t));
        tiles[(int64_t)h * T + r] = t;
        sorted[r] = lt;
    }
    __syncthreads();
    // running cost: each thread sums one chunk of slots, thread 0 scans the
    // chunk sums, each thread then writes its chunk's running values
    const int TT = g.TT, chunk = (TT + blockDim.x - 1) / blockDim.x;
    const int s0 = threadIdx.x * chunk, s1 = s0 + chunk < TT ? s0 + chunk : TT;
    auto slot_cost = [&](int sl) -> long long { return sl < g.Tt ? TT : (long long)sorted[sl - g.Tt] + g.Tt; };
    long long sum = 0;
    for (int sl = s0; sl < s1; ++sl) sum += slot_cost(sl);
    part[threadIdx.x + 1] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        part[0] = 0;
        for (int i = 1; i <= (int)blockDim.x; ++i) part[i] += part[i - 1];
    }
    __syncthreads();
    long long *pre = prefix + (int64_t)h * (TT + 1);
    long long run = part[threadIdx.x];
    if (threadIdx.x == 0) pre[0] = 0;
    for (int sl = s0; sl < s1; ++sl) {
        run += slot_cost(sl);
        pre[sl + 1] = run;
    }
}

// One workgroup: per list set the walked key tiles, the slab order, then
// the 9 cut points.  A cut inside a slab falls at its share of the slab's
// cost: by the running slot costs when the plan orders tiles (the slots'
// costs then fall along the slab), else spread evenly over the items.
// Costs and order are worked on in LDS when they fit (the slab order is
// then written out for the kernels), in the workspace otherwise.
constexpr int kLdsSets = 1024, kLdsSlabs = 2048;
__global__ __launch_bounds__(256) void split_kernel(const int32_t *__restrict__ cnt, int IH, int BH, Geo g,
                                                    int rblocks, int G, int tiles_at,
                                                    const long long *__restrict__ prefix, int *__restrict__ split,
                                                    int *__restrict__ order, long long *__restrict__ cost)
{
    __shared__ long long s_cost[kLdsSets];
    __shared__ int s_order[kLdsSlabs];
    long long *cst = IH <= kLdsSets ? s_cost : cost;
    int *ord = BH <= kLdsSlabs ? s_order : order;
    // one wave per list set at a time: lanes stride over its tiles, then a
    // butterfly sum (exact: integers)
    const int lane = threadIdx.x & 63, nwaves = blockDim.x >> 6;
    for (int h = threadIdx.x >> 6; h < IH; h += nwaves) {
        long long c = 0;
        for (int t = lane; t < g.T; t += 64) c += cnt[(int64_t)h * g.T + t];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, 64);
        // every video row block also walks the text pseudo-tiles; every text
        // row block walks every tile
        if (lane == 0) cst[h] = c + (long long)g.T * g.Tt + (long long)g.Tt * g.TT;
    }
    __syncthreads();
    // rank of slab b: the slabs of higher cost, and the earlier ones of
    // equal cost, come before it.  Slab a has list set a mod IH: of the
    // slabs below n, (n - j + IH - 1) / IH have list set j.  (Very many
    // slabs and list sets together keep the given order.)
    const bool sort = (long long)BH * IH <= (1LL << 26);
    for (int b = threadIdx.x; b < BH; b += blockDim.x) {
        const long long cb = cst[b % IH];
        long long r = 0;
        for (int j = 0; sort && j < IH; ++j) {
            const long long cj = cst[j];
            if (cj > cb) r += (BH - j + IH - 1) / IH;
            else if (cj == cb) r += (b - j + IH - 1) / IH;
        }
        ord[sort ? r : b] = b;
    }
    __syncthreads();
    if (ord != order)
        for (int b = threadIdx.x; b < BH; b += blockDim.x) order[b] = ord[b];
    if (threadIdx.x != 0) return;
    long long C = 0;
    for (int b = 0; b < BH; ++b) C += cst[b % IH];
    const long long per = (long long)g.TT * rblocks;    // items of a slab
    const long long total = (long long)BH * per;
    int cut[9];
    cut[0] = 0;
    long long cum = 0;
    int r = 0;                                          // slab rank
    for (int x = 1; x < 8; ++x) {
        const long long target = C * x / 8;
        while (r < BH && cum + cst[ord[r] % IH] <= target) cum += cst[ord[r++] % IH];
        long long item = (long long)r * per;
        if (r < BH && cst[ord[r] % IH] > 0) {
            const long long rem = target - cum;
            if (prefix) {
                // last slot whose running cost is <= rem, then the share of
                // its row blocks
                const long long *pre = prefix + (int64_t)(ord[r] % IH) * (g.TT + 1);
                int lo = 0, hi = g.TT;
                while (hi - lo > 1) {
                    const int mid = (lo + hi) / 2;
                    if (pre[mid] <= rem) lo = mid;
                    else hi = mid;
                }
                const long long sc = pre[lo + 1] - pre[lo];
                item += (long long)lo * rblocks + (sc > 0 ? (rem - pre[lo]) * rblocks / sc : 0);
            } else {
                item += (long long)((double)rem / (double)cst[ord[r] % IH] * (double)per);
            }
        }
        // at most G items per range, and no more left than the later
        // ranges can take
        long long lo = cut[x - 1], hi = lo + G;
        lo = total - (long long)(8 - x) * G > lo ? total - (long long)(8 - x) * G : lo;
        hi = hi < total ? hi : total;
        cut[x] = (int)(item < lo ? lo : item > hi ? hi : item);
    }
    cut[8] = (int)total;
#pragma unroll
    for (int x = 0; x < 9; ++x) split[x] = cut[x];
    split[9] = tiles_at;
}

size_t plan_bytes(int IH, int64_t BH, const Geo *tile_order) { return plan_layout(IH, BH, tile_order).bytes; }

sta_status plan_work(const Geo &g, const int32_t *kv_cnt, int IH, int64_t BH, int rblocks, int64_t blocks, void *ws,
                     hipStream_t s, const int **split, const int32_t *walk_cnt)
{
    const bool tiles = walk_cnt && orders_tiles(g, IH) && g.T > 0;
    const PlanLayout l = plan_layout(IH, BH, tiles ? &g : nullptr);
    char *base = (char *)ws;
    long long *prefix = tiles ? (long long *)(base + l.prefix) : nullptr;
    if (tiles)
        hipLaunchKernelGGL(tile_order_kernel, dim3((unsigned)IH), dim3(256), (size_t)g.T * 8, s, walk_cnt, g,
                           (int *)(base + l.tiles), prefix);
    hipLaunchKernelGGL(split_kernel, dim3(1), dim3(256), 0, s, kv_cnt, IH, (int)BH, g, rblocks, (int)(blocks / 8),
                       tiles ? (int)(l.tiles / 4) : -1, (const long long *)prefix, (int *)base, (int *)(base + l.order),
                       (long long *)(base + l.cost));
    *split = (const int *)base;
    return check_launch();
}

}  // namespace sta
