"""Pins of the window-shift producer's oracle (oracle/shift.py; CPU only).

The rule is this library's reading of the motion-adaptive windows of
3D-DSA ("MegaSlide-DiT", abstract), so the pins fix the rule itself: no
search radius gives no shift; a planted displacement between query and key
tiles is recovered with one-tile windows (block matching); equal key tiles
tie everywhere and the tie goes to the zero shift; the masses agree with an
independent count over the dense token mask; batch pooling is the mean of
the per-batch tile means."""
import numpy as np
import pytest

from oracle import dense_ref, oracle, shift
from tests.inputs import tensors


def test_zero_radius_gives_zero_shifts():
    q, k, _ = tensors(1, 2, 4 * 8 * 12, 16, "f32", 300)
    off, _, cands = shift.shifts(q, k, (4, 8, 12), (2, 4, 4), [(3, 3, 3), (1, 3, 5)], (0, 0, 0))
    assert len(cands) == 1 and np.all(off == 0)


@pytest.mark.parametrize("d", [(0, 1, -2), (1, -1, 1), (0, 0, 0)])
def test_planted_displacement_is_recovered(d):
    """Key tile q + d carries the direction of query tile q, every other key
    tile an orthogonal one: with one-tile windows the producer must return d
    for every query tile whose partner lies inside the grid."""
    grid, tile = (6, 8, 12), (2, 4, 4)
    n = oracle.tiles_per_axis(grid, tile)
    T = int(np.prod(n))
    N = int(np.prod(grid))
    D = T
    t, h, w = np.unravel_index(np.arange(N), grid)
    tc = np.stack([t // tile[0], h // tile[1], w // tile[2]], 1)
    tid = (tc[:, 0] * n[1] + tc[:, 1]) * n[2] + tc[:, 2]
    q = np.zeros((1, 1, N, D), np.float32)
    k = np.zeros((1, 1, N, D), np.float32)
    q[0, 0, np.arange(N), tid] = 8.0
    src = tc - np.array(d)                          # key tile c holds the direction of query tile c - d
    inside = np.all((src >= 0) & (src < np.array(n)), axis=1)
    sid = (src[:, 0] * n[1] + src[:, 1]) * n[2] + src[:, 2]
    k[0, 0, np.flatnonzero(inside), sid[inside]] = 8.0
    off, _, _ = shift.shifts(q, k, grid, tile, [(1, 1, 1)], (1, 1, 2), scale=1.0)
    qc = np.stack(np.unravel_index(np.arange(T), n), 1)
    partner_in = np.all((qc + d >= 0) & (qc + d < np.array(n)), axis=1)
    assert np.all(off[0, partner_in] == np.array(d))


@pytest.mark.parametrize("border", ["shift", "truncate"])
def test_equal_keys_tie_and_the_tie_goes_to_zero(border):
    """Equal key tiles give every candidate window mass = its token count: with
    the shifting border rule all windows hold the same tiles' worth and every
    shift ties, so the zero shift is chosen; with truncation a border window
    grows by pointing inward, which the producer then prefers."""
    grid, tile = (4, 8, 12), (2, 4, 4)
    g = np.random.default_rng(1)
    q = g.standard_normal((1, 1, int(np.prod(grid)), 16)).astype(np.float32)
    k = np.ones_like(q)
    off, tab, cands = shift.shifts(q, k, grid, tile, [(1, 3, 3)], (1, 1, 1), border=border)
    if border == "shift":
        assert np.all(off == 0)
    else:
        n = oracle.tiles_per_axis(grid, tile)
        qc = np.stack(np.unravel_index(np.arange(int(np.prod(n))), n), 1)
        # along h (window 3, 2 tiles) every window is cut to the whole axis;
        # along w (window 3, 3 tiles) the edge tiles point inward
        assert np.all(off[0][qc[:, 2] == 0, 2] == 1) and np.all(off[0][qc[:, 2] == 2, 2] == -1)
        assert np.all(off[0][qc[:, 2] == 1, 2] == 0)


@pytest.mark.parametrize("border", ["shift", "truncate"])
def test_masses_match_dense_token_mask(border):
    grid, tile, window, radius = (4, 8, 12), (2, 4, 4), (1, 3, 3), (1, 1, 1)
    q, k, _ = tensors(1, 1, int(np.prod(grid)), 16, "f32", 301)
    tab, cands = shift.masses(q, k, grid, tile, window, radius, 0.25, border)
    qm, lens = shift.tile_means(q, grid, tile)
    km, _ = shift.tile_means(k, grid, tile)
    z = 0.25 * qm[0, 0] @ km[0, 0].T
    e = lens[None, :] * np.exp(z - z.max(axis=1, keepdims=True))
    n = oracle.tiles_per_axis(grid, tile)
    T = int(np.prod(n))
    N = int(np.prod(grid))
    t, h, w = np.unravel_index(np.arange(N), grid)
    tid = ((t // tile[0]) * n[1] + h // tile[1]) * n[2] + w // tile[2]
    first = np.array([np.flatnonzero(tid == x)[0] for x in range(T)])
    for c, o in enumerate(cands):
        m = dense_ref.token_mask(grid, tile, window, np.tile(o, (T, 1)), border)
        for qq in range(T):
            allowed = np.unique(tid[m[first[qq]]])
            assert np.isclose(tab[0, 0, qq, c], e[qq, allowed].sum(), rtol=1e-12)


def test_pooling_is_the_batch_mean():
    grid, tile = (4, 8, 12), (2, 4, 4)
    q, k, _ = tensors(2, 1, int(np.prod(grid)), 16, "f32", 302)
    pooled, _, _ = shift.shifts(q, k, grid, tile, [(1, 3, 3)], (1, 1, 1))
    mq = q.mean(axis=0, keepdims=True)
    mk = k.mean(axis=0, keepdims=True)
    one, _, _ = shift.shifts(mq, mk, grid, tile, [(1, 3, 3)], (1, 1, 1))
    assert np.array_equal(pooled, one)
    per, _, _ = shift.shifts(q, k, grid, tile, [(1, 3, 3)], (1, 1, 1), pooled=False)
    assert per.shape == (2, 1, int(np.prod(oracle.tiles_per_axis(grid, tile))), 3)
    alone, _, _ = shift.shifts(q[1:], k[1:], grid, tile, [(1, 3, 3)], (1, 1, 1))
    assert np.array_equal(per[1], alone)
