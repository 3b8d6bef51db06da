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
// Workspace layout (plan_bytes): int split[9] at 0, int order[BH] at 64
// bytes (order[r] = the slab of rank r), int64 cost[IH] after it.
#include "common.h"

namespace sta {

// One workgroup: per list set the walked key tiles, the slab order, then
// the 9 cut points.
__global__ __launch_bounds__(256) void split_kernel(const int32_t *__restrict__ cnt, int IH, int BH, Geo g,
                                                    int rblocks, int G, int *__restrict__ split,
                                                    int *__restrict__ order, long long *__restrict__ cost)
{
    for (int h = threadIdx.x; h < IH; h += blockDim.x) {
        long long c = 0;
        for (int t = 0; t < g.T; ++t) c += cnt[(int64_t)h * g.T + t];
        // every video row block also walks the text pseudo-tiles; every text
        // row block walks every tile
        c += (long long)g.T * g.Tt + (long long)g.Tt * g.TT;
        cost[h] = c;
    }
    __syncthreads();
    // rank of slab b: the slabs of higher cost, and the earlier ones of
    // equal cost, come before it.  Slab a has list set a mod IH: of the
    // slabs below n, (n - j + IH - 1) / IH have list set j.  (Very many
    // slabs and list sets together keep the given order.)
    const bool sort = (long long)BH * IH <= (1LL << 26);
    for (int b = threadIdx.x; b < BH; b += blockDim.x) {
        const long long cb = cost[b % IH];
        long long r = 0;
        for (int j = 0; sort && j < IH; ++j) {
            const long long cj = cost[j];
            if (cj > cb) r += (BH - j + IH - 1) / IH;
            else if (cj == cb) r += (b - j + IH - 1) / IH;
        }
        order[sort ? r : b] = b;
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    long long C = 0;
    for (int b = 0; b < BH; ++b) C += cost[b % IH];
    const long long per = (long long)g.TT * rblocks;    // items of a slab
    const long long total = (long long)BH * per;
    split[0] = 0;
    long long cum = 0;
    int r = 0;                                          // slab rank
    for (int x = 1; x < 8; ++x) {
        const long long target = C * x / 8;
        while (r < BH && cum + cost[order[r] % IH] <= target) cum += cost[order[r++] % IH];
        long long item = (long long)r * per;
        if (r < BH && cost[order[r] % IH] > 0)
            item += (long long)((double)(target - cum) / (double)cost[order[r] % IH] * (double)per);
        // at most G items per range, and no more left than the later
        // ranges can take
        long long lo = split[x - 1], hi = lo + G;
        lo = total - (long long)(8 - x) * G > lo ? total - (long long)(8 - x) * G : lo;
        hi = hi < total ? hi : total;
        split[x] = (int)(item < lo ? lo : item > hi ? hi : item);
    }
    split[8] = (int)total;
}

size_t plan_bytes(int IH, int64_t BH) { return 64 + (((size_t)BH * 4 + 7) & ~(size_t)7) + (size_t)IH * 8; }

sta_status plan_work(const Geo &g, const int32_t *kv_cnt, int IH, int64_t BH, int rblocks, int64_t blocks, void *ws,
                     hipStream_t s, const int **split)
{
    int *out = (int *)ws;
    int *order = (int *)((char *)ws + 64);
    long long *cost = (long long *)((char *)ws + 64 + (((size_t)BH * 4 + 7) & ~(size_t)7));
    hipLaunchKernelGGL(split_kernel, dim3(1), dim3(256), 0, s, kv_cnt, IH, (int)BH, g, rblocks, (int)(blocks / 8),
                       out, order, cost);
    *split = out;
    return check_launch();
}

}  // namespace sta
