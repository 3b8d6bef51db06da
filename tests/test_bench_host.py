"""Host arithmetic of the benchmark (CPU only): the bytes an attention
kernel copies into LDS per launch, against closed forms at the 720P
training shape, and on a grid with cut border tiles against a brute-force
count of the workgroups' copies."""
import numpy as np

import bench
from oracle import oracle

GRID, TILE, H, D = (30, 48, 80), (6, 8, 8), 24, 128


def _lens(grid, tile):
    axes = [[min(t, g - i * t) for i in range(-(-g // t))] for g, t in zip(grid, tile)]
    return np.einsum("a,b,c->abc", *[np.array(x, np.float64) for x in axes]).ravel()


def test_copy_bytes_closed_form_720p():
    kv_idx, kv_cnt, q_idx, q_cnt = oracle.index(GRID, TILE, [(3, 3, 5)] * H)
    lens = _lens(GRID, TILE)
    pairs = H * 300 * 45                       # every query tile lists 45 key tiles, 324 000 pairs
    assert kv_cnt.sum() == pairs and q_cnt.sum() == pairs
    # 3 workgroups of 128 rows per 384-row tile, each copying 384 listed rows per pair
    assert bench.block_copy_bytes(lens, kv_idx, kv_cnt, 1, 4 * D) == pairs * 3 * 384 * 4 * D
    assert bench.block_copy_bytes(lens, q_idx, q_cnt, 2, 4 * D + 8) == 2 * pairs * 3 * 384 * (4 * D + 8)


def test_copy_bytes_cut_tiles_brute_force():
    grid, tile = (7, 12, 13), (4, 8, 8)        # tiles of 256 rows, cut ones of 96 to 160 rows
    kv_idx, kv_cnt, _, _ = oracle.index(grid, tile, [(3, 3, 3), (1, 3, 5)])
    lens = _lens(grid, tile)
    expect = 0
    for h in range(2):
        for t in range(kv_cnt.shape[1]):
            for wg_start in range(0, int(lens[t]), 128):          # one workgroup per 128 rows of the tile
                for kt in kv_idx[h, t, :kv_cnt[h, t]]:
                    expect += int(lens[kt]) * 40
    assert bench.block_copy_bytes(lens, kv_idx, kv_cnt, 1, 40) == expect
