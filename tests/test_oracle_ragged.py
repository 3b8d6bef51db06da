"""Pins of the oracle on grids that the tile does not divide (CPU only).

Reading: the last tile of such an axis is cut by the grid border and holds
only the tokens inside the grid; no padding tokens exist, and the window
rule works on the ceil(grid / tile) tiles per axis.  Pins: dense masked
attention (torch SDPA + autograd, float64) under a mask built independently;
a reduction to the divisible case (the grid padded to whole tiles, padding
keys pushed to probability zero through an extra feature, padding queries
given zero gradient); the index depends only on the tile grid; a window
covering the whole tile grid is full attention."""
import numpy as np
import pytest
import torch

from oracle import dense_ref, oracle
from tests.inputs import tensors

CASES = [
    # grid, tile, windows, border, per-head offsets?, n_text
    ((5, 6, 7), (2, 4, 4), [(1, 3, 3), (3, 1, 3)], "shift", False, 0),
    ((3, 5, 9), (2, 2, 4), [(3, 3, 1), (1, 3, 3)], "truncate", True, 0),
    ((4, 7, 6), (4, 3, 4), [(1, 1, 1), (3, 3, 3)], "shift", True, 5),
    ((2, 3, 5), (4, 4, 8), [(1, 1, 1), (3, 3, 3)], "shift", False, 0),      # one tile, cut on every axis
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_ragged_matches_torch_dense(case):
    grid, tile, windows, border, per_head, nt = CASES[case]
    H, D = len(windows), 8
    T = int(np.prod(oracle.tiles_per_axis(grid, tile)))
    g = np.random.default_rng(60 + case)
    off = g.integers(-1, 1, endpoint=True, size=(H, T, 3)).astype(np.int32) if per_head else None
    S = int(np.prod(grid)) + nt
    q, k, v, do = tensors(1, H, S, D, "f32", 70 + case, with_dout=True)
    o, lse = oracle.fwd(q, k, v, grid, tile, windows, off, border=border, n_text=nt)
    dq, dk, dv = oracle.bwd(q, k, v, do, grid, tile, windows, off, border=border, n_text=nt)
    ref = dense_ref.attention(q, k, v, grid, tile, windows, off, dout=do, border=border, n_text=nt)
    for got, want in zip((o, lse, dq, dk, dv), ref):
        assert np.max(np.abs(got - want)) < 1e-10


def _padded(x, grid, pgrid, fill):
    """[B,H,N,D] raster tensor on grid -> the same on pgrid (>= grid per
    axis), new tokens filled with `fill`."""
    B, H, _, D = x.shape
    out = np.full((B, H) + tuple(pgrid) + (D,), fill, x.dtype)
    out[:, :, : grid[0], : grid[1], : grid[2]] = x.reshape((B, H) + tuple(grid) + (D,))
    return out.reshape(B, H, -1, D)


@pytest.mark.parametrize("case", [0, 1])
def test_ragged_equals_padded_grid_with_padding_masked(case):
    """Attention on a cut grid equals attention on the grid padded to whole
    tiles (a divisible problem), where the padding keys are pushed to
    probability zero by an extra feature: queries carry 1 there, real keys 0
    and padding keys -1e30 (exp underflows to exactly 0 in fp64); padding
    queries get dO = 0, so they add nothing to dK and dV."""
    grid, tile, windows, border, per_head, _ = CASES[case]
    H, D = len(windows), 8
    n = oracle.tiles_per_axis(grid, tile)
    pgrid = tuple(a * b for a, b in zip(n, tile))
    T = int(np.prod(n))
    g = np.random.default_rng(80 + case)
    off = g.integers(-1, 1, endpoint=True, size=(H, T, 3)).astype(np.int32) if per_head else None
    N = int(np.prod(grid))
    q, k, v, do = tensors(1, H, N, D, "f32", 90 + case, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    o, lse = oracle.fwd(q, k, v, grid, tile, windows, off, scale=scale, border=border)
    dq, dk, dv = oracle.bwd(q, k, v, do, grid, tile, windows, off, scale=scale, border=border)

    real = np.zeros(pgrid, bool)
    real[: grid[0], : grid[1], : grid[2]] = True
    real = real.ravel()
    pq = _padded(np.concatenate([q, np.ones(q.shape[:-1] + (1,), np.float32)], -1), grid, pgrid, 0.0)
    pq[:, :, ~real, -1] = 1.0
    pk = _padded(np.concatenate([k, np.zeros(k.shape[:-1] + (1,), np.float32)], -1), grid, pgrid, 0.0)
    pk[:, :, ~real, -1] = -1e30
    pv = _padded(np.concatenate([v, np.zeros(v.shape[:-1] + (1,), np.float32)], -1), grid, pgrid, 0.0)
    pdo = _padded(np.concatenate([do, np.zeros(do.shape[:-1] + (1,), np.float32)], -1), grid, pgrid, 0.0)
    po, pl = oracle.fwd(pq, pk, pv, pgrid, tile, windows, off, scale=scale, border=border)
    pdq, pdk, pdv = oracle.bwd(pq, pk, pv, pdo, pgrid, tile, windows, off, scale=scale, border=border)
    np.testing.assert_allclose(o, po[:, :, real, :D], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, pl[:, :, real], rtol=1e-12, atol=1e-13)
    for got, want in ((dq, pdq), (dk, pdk), (dv, pdv)):
        np.testing.assert_allclose(got, want[:, :, real, :D], rtol=1e-11, atol=1e-13)


def test_ragged_index_is_that_of_the_tile_grid():
    """The lists depend only on the tile grid: a cut grid has the lists of the
    grid rounded up to whole tiles."""
    for grid, tile, windows, border, per_head, _ in CASES:
        n = oracle.tiles_per_axis(grid, tile)
        pgrid = tuple(a * b for a, b in zip(n, tile))
        a = oracle.index(grid, tile, windows, border=border)
        b = oracle.index(pgrid, tile, windows, border=border)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_ragged_whole_window_is_full_attention():
    grid, tile = (3, 5, 7), (2, 2, 4)
    q, k, v, do = tensors(1, 1, 105, 8, "f32", 99, with_dout=True)
    o, lse = oracle.fwd(q, k, v, grid, tile, [(5, 5, 5)])
    dq, dk, dv = oracle.bwd(q, k, v, do, grid, tile, [(5, 5, 5)])
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    to.backward(torch.tensor(do, dtype=torch.float64))
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-11, atol=1e-12)
    for got, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-10, atol=1e-12)
