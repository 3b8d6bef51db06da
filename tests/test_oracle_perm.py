"""Pins of the oracle's raster -> tile-contiguous token permutation (CPU)."""
import numpy as np
import pytest

from oracle import oracle
from tests.conftest import read_golden
from tests.inputs import CONFIGS


@pytest.mark.parametrize("name", ["perm_small.txt", "perm_asym.txt", "perm_ragged.txt"])
def test_golden_small(name):
    rows = {r[0]: list(map(int, r[1:])) for r in read_golden(name)}
    assert oracle.perm(rows["grid"], rows["tile"]).tolist() == rows["perm"]


@pytest.mark.parametrize("cfg", ["tiny-fp32", "mid-7680", "720p", "asym"])
def test_bijection_and_tile_contiguity(cfg):
    grid, tile = ((4, 6, 6), (2, 3, 2)) if cfg == "asym" else (CONFIGS[cfg]["grid"], CONFIGS[cfg]["tile"])
    p = oracle.perm(grid, tile)
    N = int(np.prod(grid))
    assert np.array_equal(np.sort(p), np.arange(N))
    # every block of L consecutive tile-order slots holds exactly one tile's tokens
    L = int(np.prod(tile))
    t, h, w = np.unravel_index(np.arange(N), grid)
    n = oracle.tiles_per_axis(grid, tile)
    tid = ((t // tile[0]) * n[1] + h // tile[1]) * n[2] + w // tile[2]
    assert np.array_equal(p // L, tid)


@pytest.mark.parametrize("grid,tile", [((3, 4, 5), (1, 1, 1)), ((3, 4, 5), (3, 4, 5)),
                                       ((4, 6, 10), (2, 6, 10)), ((6, 1, 7), (3, 1, 7))])
def test_identity_cases(grid, tile):
    """Unit tiles, one tile, and tiles spanning whole (H,W) planes keep raster order."""
    assert np.array_equal(oracle.perm(grid, tile), np.arange(int(np.prod(grid))))


def test_rows_of_tw_tokens_stay_contiguous():
    """A run of tw tokens along w inside one tile is contiguous in both orders."""
    grid, tile = (30, 48, 80), (6, 8, 8)
    p = oracle.perm(grid, tile)
    runs = p.reshape(-1, tile[2])
    assert np.all(np.diff(runs, axis=1) == 1)


def test_non_positive_extents_rejected():
    with pytest.raises(ValueError):
        oracle.perm((5, 4, 4), (2, 0, 2))


RAGGED = [((5, 4, 4), (2, 2, 2)), ((3, 5, 3), (2, 2, 2)), ((7, 9, 10), (3, 4, 4)), ((30, 45, 80), (6, 8, 8)),
          ((2, 3, 5), (4, 4, 8))]


@pytest.mark.parametrize("grid,tile", RAGGED)
def test_ragged_tiles_are_contiguous_and_ordered(grid, tile):
    """Cut border tiles: the permutation is a bijection onto 0..N-1; every
    tile's tokens fill one contiguous range, tiles follow in raster order of
    tile coordinates, each range as long as the tile's tokens inside the grid,
    and tokens inside a tile keep their raster order."""
    p = oracle.perm(grid, tile)
    N = int(np.prod(grid))
    assert np.array_equal(np.sort(p), np.arange(N))
    t, h, w = np.unravel_index(np.arange(N), grid)
    n = oracle.tiles_per_axis(grid, tile)
    tid = ((t // tile[0]) * n[1] + h // tile[1]) * n[2] + w // tile[2]
    order = np.argsort(p)                          # raster tokens in tile order
    assert np.all(np.diff(tid[order]) >= 0)        # tiles in order, each contiguous
    for k in np.unique(tid)[:: max(1, len(np.unique(tid)) // 50)]:
        toks = np.flatnonzero(tid == k)            # raster order
        assert np.array_equal(p[toks], p[toks].min() + np.arange(len(toks)))
        a, b, c = np.unravel_index(k, n)
        size = np.prod([min(tl, g - i * tl) for g, tl, i in zip(grid, tile, (a, b, c))])
        assert len(toks) == size


def test_divisible_part_unchanged_by_a_cut_border():
    """Cutting only the last tile plane leaves the positions of every token
    before it as on the grid without that plane."""
    assert np.array_equal(oracle.perm((7, 8, 8), (3, 4, 4))[: 6 * 64], oracle.perm((6, 8, 8), (3, 4, 4)))
