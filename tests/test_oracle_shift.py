"""Pins of the window-shift producer's oracle (oracle/shift.py; CPU only).

The rule is this library's reading of the motion-adaptive windows of
3D-DSA ("MegaSlide-DiT", abstract), so the pins fix the rule itself: tile
means against their closed form on coordinate-valued tokens; no search
radius gives no shift; a planted displacement between query and key tiles
is recovered with one-tile windows (block matching); equal key tiles tie
everywhere and the tie goes to the zero shift, and a tie between shifts of
equal size goes to the first in raster order; the masses agree with an
independent count over the dense token mask; batch pooling is the mean of
the per-batch tile means.

Each check takes the module under test, so that planted mistakes in copies
of it (tests/test_oracle_shift_mutants.py) run through the same checks."""
import numpy as np
import pytest

from oracle import dense_ref, oracle, shift
from tests.inputs import tensors

PLANTED = [(0, 1, -2), (1, -1, 1), (0, 0, 0)]


def check_tile_means_closed_form(mod):
    """Tokens valued by their own (t, h, w) coordinates: a tile's mean is the
    centre of the box of its tokens and its length the box's volume (tiles
    cut by the grid border included)."""
    grid, tile = (5, 7, 10), (2, 4, 4)
    N = int(np.prod(grid))
    coords = np.stack(np.unravel_index(np.arange(N), grid), 1).astype(np.float32)
    means, lens = mod.tile_means(coords[None, None], grid, tile)
    n = oracle.tiles_per_axis(grid, tile)
    for tid, (a, b, c) in enumerate(np.ndindex(*n)):
        lo = np.array([a, b, c]) * tile
        hi = np.minimum(lo + tile, grid)
        assert lens[tid] == np.prod(hi - lo)
        np.testing.assert_allclose(means[0, 0, tid], (lo + hi - 1) / 2.0, rtol=0, atol=1e-12)


def check_zero_radius(mod):
    q, k, _ = tensors(1, 2, 4 * 8 * 12, 16, "f32", 300)
    off, _, cands = mod.shifts(q, k, (4, 8, 12), (2, 4, 4), [(3, 3, 3), (1, 3, 5)], (0, 0, 0))
    assert len(cands) == 1 and np.all(off == 0)


def check_planted_displacement(mod, d):
    """Key tile c carries the direction of query tile c - d, every other key
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
    off, _, _ = mod.shifts(q, k, grid, tile, [(1, 1, 1)], (1, 1, 2), scale=1.0)
    qc = np.stack(np.unravel_index(np.arange(T), n), 1)
    partner_in = np.all((qc + d >= 0) & (qc + d < np.array(n)), axis=1)
    assert np.all(off[0, partner_in] == np.array(d))


def check_equal_keys(mod, border):
    """Equal key tiles give every candidate window mass = its token count: with
    the shifting border rule all windows hold the same tiles' worth and every
    shift ties, so the zero shift is chosen; with truncation a border window
    grows by pointing inward, which the producer then prefers."""
    grid, tile = (4, 8, 12), (2, 4, 4)
    g = np.random.default_rng(1)
    q = g.standard_normal((1, 1, int(np.prod(grid)), 16)).astype(np.float32)
    k = np.ones_like(q)
    off, tab, cands = mod.shifts(q, k, grid, tile, [(1, 3, 3)], (1, 1, 1), border=border)
    if border == "shift":
        assert np.all(off == 0)
    else:
        n = oracle.tiles_per_axis(grid, tile)
        qc = np.stack(np.unravel_index(np.arange(int(np.prod(n))), n), 1)
        # along h (window 3, 2 tiles) every window is cut to the whole axis;
        # along w (window 3, 3 tiles) the edge tiles point inward
        assert np.all(off[0][qc[:, 2] == 0, 2] == 1) and np.all(off[0][qc[:, 2] == 2, 2] == -1)
        assert np.all(off[0][qc[:, 2] == 1, 2] == 0)


def check_raster_order_tie(mod):
    """Key tiles (0,1,0) and (0,0,1) both carry the direction of query tile
    (0,0,0) and nothing else does: with one-tile windows the shifts (0,1,0)
    and (0,0,1) tie exactly with equal |o|_1, and the first in raster order
    of (o_t, o_h, o_w), (0,0,1), is chosen."""
    grid, tile = (6, 8, 12), (2, 4, 4)
    n = oracle.tiles_per_axis(grid, tile)
    N = int(np.prod(grid))
    t, h, w = np.unravel_index(np.arange(N), grid)
    tid = ((t // tile[0]) * n[1] + h // tile[1]) * n[2] + w // tile[2]
    q = np.zeros((1, 1, N, 4), np.float32)
    k = np.zeros((1, 1, N, 4), np.float32)
    q[0, 0, tid == 0, 0] = 3.0
    for c in ((0, 1, 0), (0, 0, 1)):
        k[0, 0, tid == (c[0] * n[1] + c[1]) * n[2] + c[2], 0] = 3.0
    off, tab, cands = mod.shifts(q, k, grid, tile, [(1, 1, 1)], (1, 1, 1), scale=1.0)
    assert tuple(off[0, 0]) == (0, 0, 1)


def check_masses_match_dense_mask(mod, border):
    """Every candidate's mass against a sum over the tiles that the dense token
    mask (an independent window characterisation) lets a query tile see, with
    the tile means and lengths formed here from the tokens directly."""
    grid, tile, window, radius = (5, 7, 10), (2, 4, 4), (1, 3, 3), (1, 1, 1)
    N = int(np.prod(grid))
    q, k, _ = tensors(1, 1, N, 16, "f32", 301)
    tab, cands = mod.masses(q, k, grid, tile, window, radius, 0.25, border)
    n = oracle.tiles_per_axis(grid, tile)
    T = int(np.prod(n))
    t, h, w = np.unravel_index(np.arange(N), grid)
    tid = ((t // tile[0]) * n[1] + h // tile[1]) * n[2] + w // tile[2]
    lens = np.bincount(tid, minlength=T).astype(np.float64)
    qm = np.stack([q[0, 0, tid == x].astype(np.float64).mean(0) for x in range(T)])
    km = np.stack([k[0, 0, tid == x].astype(np.float64).mean(0) for x in range(T)])
    z = 0.25 * qm @ km.T
    e = lens[None, :] * np.exp(z - z.max(axis=1, keepdims=True))
    first = np.array([np.flatnonzero(tid == x)[0] for x in range(T)])
    for c, o in enumerate(cands):
        m = dense_ref.token_mask(grid, tile, window, np.tile(o, (T, 1)), border)
        for qq in range(T):
            allowed = np.unique(tid[m[first[qq]]])
            assert np.isclose(tab[0, 0, qq, c], e[qq, allowed].sum(), rtol=1e-12)


def check_pooling(mod):
    grid, tile = (4, 8, 12), (2, 4, 4)
    q, k, _ = tensors(2, 1, int(np.prod(grid)), 16, "f32", 302)
    pooled, _, _ = mod.shifts(q, k, grid, tile, [(1, 3, 3)], (1, 1, 1))
    mq = q.mean(axis=0, keepdims=True)
    mk = k.mean(axis=0, keepdims=True)
    one, _, _ = mod.shifts(mq, mk, grid, tile, [(1, 3, 3)], (1, 1, 1))
    assert np.array_equal(pooled, one)
    per, _, _ = mod.shifts(q, k, grid, tile, [(1, 3, 3)], (1, 1, 1), pooled=False)
    assert per.shape == (2, 1, int(np.prod(oracle.tiles_per_axis(grid, tile))), 3)
    alone, _, _ = mod.shifts(q[1:], k[1:], grid, tile, [(1, 3, 3)], (1, 1, 1))
    assert np.array_equal(per[1], alone)


def all_checks():
    """(name, callable(mod)) for every check, parameters bound."""
    out = [("tile-means", check_tile_means_closed_form), ("zero-radius", check_zero_radius),
           ("pooling", check_pooling), ("raster-order-tie", check_raster_order_tie)]
    out += [("planted-%s" % (d,), lambda m, d=d: check_planted_displacement(m, d)) for d in PLANTED]
    for b in ("shift", "truncate"):
        out += [("equal-keys-" + b, lambda m, b=b: check_equal_keys(m, b)),
                ("dense-mask-" + b, lambda m, b=b: check_masses_match_dense_mask(m, b))]
    return out


@pytest.mark.parametrize("name,check", all_checks(), ids=[n for n, _ in all_checks()])
def test_shift_oracle_pin(name, check):
    check(shift)
