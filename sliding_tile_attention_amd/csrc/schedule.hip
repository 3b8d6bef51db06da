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
// windows).  Equal slabs give equal ranges, the plain contiguous split.
// Within a slab the cost is taken as uniform per item.  A launch has G
// blocks per XCD (twice the mean share, work_blocks); a range is capped at G
// items, and the ranges after it take up what the cap leaves.
#include "common.h"

namespace sta {

// One workgroup: per list set the walked key tiles, then the 9 cut points.
// cost[IH] (int64) is scratch in the same workspace.
__global__ __launch_bounds__(256) void split_kernel(const int32_t *__restrict__ cnt, int IH, int BH, Geo g,
                                                    int rblocks, int G, long long *__restrict__ cost,
                                                    int *__restrict__ split)
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
    if (threadIdx.x != 0) return;
    long long C = 0;
    for (int bh = 0; bh < BH; ++bh) C += cost[bh % IH];
    const long long per = (long long)g.TT * rblocks;    // items of a slab
    split[0] = 0;
    long long cum = 0;
    int bh = 0;
    for (int x = 1; x < 8; ++x) {
        const long long target = C * x / 8;
        while (bh < BH && cum + cost[bh % IH] <= target) cum += cost[bh++ % IH];
        long long item = (long long)bh * per;
        if (bh < BH && cost[bh % IH] > 0)
            item += (long long)((double)(target - cum) / (double)cost[bh % IH] * (double)per);
        // at most G items per range, and no more left than the later
        // ranges can take
        const long long total = (long long)BH * per;
        long long lo = split[x - 1], hi = lo + G;
        lo = total - (long long)(8 - x) * G > lo ? total - (long long)(8 - x) * G : lo;
        hi = hi < total ? hi : total;
        split[x] = (int)(item < lo ? lo : item > hi ? hi : item);
    }
    split[8] = (int)((long long)BH * per);
}

size_t plan_bytes(int IH) { return 64 + (size_t)IH * sizeof(long long); }

sta_status plan_work(const Geo &g, const int32_t *kv_cnt, int IH, int64_t BH, int rblocks, int64_t blocks, void *ws,
                     hipStream_t s, const int **split)
{
    int *out = (int *)ws;
    hipLaunchKernelGGL(split_kernel, dim3(1), dim3(256), 0, s, kv_cnt, IH, (int)BH, g, rblocks, (int)(blocks / 8),
                       (long long *)((char *)ws + 64), out);
    *split = out;
    return check_launch();
}

}  // namespace sta
