"""The allocation-free window-shift producer (sta_window_shifts_noalloc,
for callers that cannot allocate) against the pool-backed entry point
sta_window_shifts: two calls in a row, the second on a smaller input (so the
static scratch still holds the first call's larger contents), each equal to
the pool-backed result exactly (integer shifts)."""
import pytest
import torch

import sliding_tile_attention_amd as sta
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

CASES = [
    # name, grid, tile, B, H, D, windows, radius, per_batch, border
    ("720p-B2-per-item", (30, 48, 80), (6, 8, 8), 2, 24, 128, [(3, 3, 3), (3, 3, 5), (5, 5, 5)] * 8, (1, 1, 1), True,
     "shift"),
    ("small-D64-truncate", (8, 16, 24), (2, 8, 8), 1, 3, 64, [(3, 3, 3), (1, 3, 5), (3, 1, 1)], (1, 1, 2), False,
     "truncate"),
]


def _inputs(B, H, grid, tile, D, seed):
    """Seeded q, k [B, H, N, D] bf16 in tile order: N(0,1) draws plus one
    N(0,1) vector per tile (q and k independent), so that tiles differ and
    the chosen shifts vary."""
    geom = sta.Geometry(grid, tile)
    T, L = geom.num_tiles, geom.tile_tokens
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(B, H, T, L, D, device="cuda", generator=g) + torch.randn(B, H, T, 1, D, device="cuda", generator=g)
    k = torch.randn(B, H, T, L, D, device="cuda", generator=g) + torch.randn(B, H, T, 1, D, device="cuda", generator=g)
    return geom, q.reshape(B, H, T * L, D).to(torch.bfloat16), k.reshape(B, H, T * L, D).to(torch.bfloat16)


def test_noalloc_shifts_equal_the_pool_backed_call():
    data, got = [], []
    for i, (name, grid, tile, B, H, D, windows, radius, per_batch, border) in enumerate(CASES):
        geom, q, k = _inputs(B, H, grid, tile, D, 300 + i)
        data.append((geom, q, k, windows, radius, per_batch, border))
    for (name, *_), (geom, q, k, windows, radius, per_batch, border) in zip(CASES, data):
        say("noalloc window shifts " + name)
        got.append(sta.window_shifts(q, k, geom, windows, radius, border=border, per_batch=per_batch, noalloc=True))
    torch.cuda.synchronize()
    for (name, *_), (geom, q, k, windows, radius, per_batch, border), g in zip(CASES, data, got):
        ref = sta.window_shifts(q, k, geom, windows, radius, border=border, per_batch=per_batch)
        torch.cuda.synchronize()
        assert g.shape == ref.shape and torch.equal(g, ref), name
        assert int(g.abs().sum()) > 0, name + ": every shift is zero"
        say("  %s: %d shifts equal, %d nonzero" % (name, g.numel() // 3, int((g != 0).any(-1).sum())))
