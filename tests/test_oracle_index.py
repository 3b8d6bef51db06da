"""Pins of the oracle's block-sparse index (CPU only).

The window rule has no worked example on the pages ("Fast Video Generation
with Sliding Tile Attention", abstract: attention slides over a local 3D
window).  The oracle's lists are pinned here by hand-derived tables, by a
second characterisation of the window (enumeration, in dense_ref), and by
invariants that any correct list must satisfy.
"""
import itertools

import numpy as np
import pytest

from oracle import oracle, dense_ref
from tests.conftest import read_golden
from tests.inputs import CONFIGS, offsets_for, windows_for


def _axis_case(n, w, q, o):
    """One-axis window through the 3D oracle: grid (1,1,n) of 1-token tiles."""
    off = np.zeros((n, 3), np.int32)
    off[q, 2] = o
    kv_idx, kv_cnt, _, _ = oracle.index((1, 1, n), (1, 1, 1), [(1, 1, w)], off)
    lst = kv_idx[0, q, : kv_cnt[0, q]]
    return int(lst[0]), int(kv_cnt[0, q]), lst


@pytest.mark.parametrize("row", read_golden("window_axis.txt"), ids=lambda r: "-".join(r))
def test_window_axis_golden(row):
    n, w, q, o, start, count = map(int, row)
    s, c, lst = _axis_case(n, w, q, o)
    assert (s, c) == (start, count)
    assert list(lst) == list(range(start, start + count))


def test_attendee_counts_720p_golden():
    rows = {r[0]: list(map(int, r[1:])) for r in read_golden("attendee_counts_720p.txt")}
    c = CONFIGS["720p"]
    _, kv_cnt, q_idx, q_cnt = oracle.index(c["grid"], c["tile"], windows_for("720p")[:1])
    n = (5, 6, 10)
    expect = np.einsum("i,j,k->ijk", rows["t"], rows["h"], rows["w"]).reshape(-1)
    assert np.array_equal(q_cnt[0], expect)
    assert q_cnt.min() == 12 and q_cnt.max() == 140 and q_cnt.sum() == 13500
    assert np.all(kv_cnt == 45)
    assert int(np.prod(n)) == q_cnt.shape[1]


def _random_geometries(count, seed):
    g = np.random.default_rng(seed)
    for _ in range(count):
        n = tuple(int(x) for x in g.integers(1, 7, size=3))
        tile = tuple(int(x) for x in g.integers(1, 3, size=3))
        grid = tuple(a * b for a, b in zip(n, tile))
        H = int(g.integers(1, 4))
        windows = g.integers(1, 8, size=(H, 3)).astype(np.int32)
        off = g.integers(-3, 4, size=(int(np.prod(n)), 3)).astype(np.int32) if g.random() < 0.5 else None
        yield grid, tile, windows, off


@pytest.mark.parametrize("case", range(12))
def test_lists_match_enumerated_token_mask(case):
    """The tile lists, expanded to tokens, equal dense_ref's mask, whose
    windows are found by enumerating placements (not by the clamp)."""
    grid, tile, windows, off = list(_random_geometries(12, 99))[case]
    kv_idx, kv_cnt, _, _ = oracle.index(grid, tile, windows, off)
    n = oracle.tiles_per_axis(grid, tile)
    coords = np.array(list(itertools.product(*[range(x) for x in grid])))
    tc = coords // np.array(tile)
    tid = (tc[:, 0] * n[1] + tc[:, 1]) * n[2] + tc[:, 2]
    for h in range(len(windows)):
        m = dense_ref.token_mask(grid, tile, tuple(windows[h]), off)
        allowed_tiles = [set(kv_idx[h, q, : kv_cnt[h, q]].tolist()) for q in range(int(np.prod(n)))]
        from_lists = np.array([[tid[j] in allowed_tiles[tid[i]] for j in range(len(tid))]
                               for i in range(len(tid))])
        assert np.array_equal(m, from_lists)


@pytest.mark.parametrize("case", range(12))
def test_list_invariants(case):
    grid, tile, windows, off = list(_random_geometries(12, 7))[case]
    n = oracle.tiles_per_axis(grid, tile)
    T = int(np.prod(n))
    kv_idx, kv_cnt, q_idx, q_cnt = oracle.index(grid, tile, windows, off)
    for h, w in enumerate(windows):
        # every query tile gets the full window (windows are moved, not cut)
        assert np.all(kv_cnt[h] == np.prod(np.minimum(w, n)))
        for q in range(T):
            lst = kv_idx[h, q]
            c = kv_cnt[h, q]
            assert np.all(np.diff(lst[:c]) > 0) and np.all(lst[c:] == -1)
        for k in range(T):
            lst = q_idx[h, k]
            c = q_cnt[h, k]
            assert np.all(np.diff(lst[:c]) > 0) and np.all(lst[c:] == -1)
        # transpose consistency: k in KV(q) <=> q in QT(k)
        fw = {(q, int(k)) for q in range(T) for k in kv_idx[h, q, : kv_cnt[h, q]]}
        bw = {(int(q), k) for k in range(T) for q in q_idx[h, k, : q_cnt[h, k]]}
        assert fw == bw
        assert kv_cnt[h].sum() == q_cnt[h].sum()


def test_interior_tiles_get_chebyshev_ball():
    """Away from the borders and without shifts the window is the set of
    tiles within floor(w/2) of the query tile on every axis."""
    grid, tile, w = (16, 16, 20), (2, 2, 2), (3, 5, 7)
    n = oracle.tiles_per_axis(grid, tile)
    kv_idx, kv_cnt, _, _ = oracle.index(grid, tile, [w])
    r = [x // 2 for x in w]
    for qc in itertools.product(*[range(r[d], n[d] - r[d]) for d in range(3)]):
        q = (qc[0] * n[1] + qc[1]) * n[2] + qc[2]
        ball = sorted((a * n[1] + b) * n[2] + c
                      for a in range(qc[0] - r[0], qc[0] + r[0] + 1)
                      for b in range(qc[1] - r[1], qc[1] + r[1] + 1)
                      for c in range(qc[2] - r[2], qc[2] + r[2] + 1))
        assert kv_idx[0, q, : kv_cnt[0, q]].tolist() == ball


def test_mirror_symmetry():
    """Odd windows without shifts: the window of the mirrored tile is the
    mirrored window."""
    grid, tile, w = (10, 12, 14), (2, 3, 2), (3, 3, 5)
    n = oracle.tiles_per_axis(grid, tile)
    kv_idx, kv_cnt, _, _ = oracle.index(grid, tile, [w])

    def coords(i):
        return (i // (n[1] * n[2]), (i // n[2]) % n[1], i % n[2])

    def mirror(i):
        a, b, c = coords(i)
        return ((n[0] - 1 - a) * n[1] + (n[1] - 1 - b)) * n[2] + (n[2] - 1 - c)

    T = int(np.prod(n))
    for q in range(T):
        mine = {mirror(int(k)) for k in kv_idx[0, q, : kv_cnt[0, q]]}
        theirs = set(kv_idx[0, mirror(q), : kv_cnt[0, mirror(q)]].tolist())
        assert mine == theirs


def test_zero_offsets_equal_no_offsets_and_large_offsets_saturate():
    grid, tile = (12, 12, 20), (2, 2, 2)
    n = oracle.tiles_per_axis(grid, tile)
    T = int(np.prod(n))
    w = [(3, 3, 5), (5, 1, 3)]
    a = oracle.index(grid, tile, w, None)
    b = oracle.index(grid, tile, w, np.zeros((T, 3), np.int32))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    far = np.full((T, 3), 1000, np.int32)
    kv_idx, kv_cnt, _, _ = oracle.index(grid, tile, w, far)
    # every query gets the window pressed against the high border
    for h, wh in enumerate(w):
        c = np.minimum(wh, n)
        top = sorted((a_ * n[1] + b_) * n[2] + c_
                     for a_ in range(n[0] - c[0], n[0])
                     for b_ in range(n[1] - c[1], n[1])
                     for c_ in range(n[2] - c[2], n[2]))
        for q in range(T):
            assert kv_idx[h, q, : kv_cnt[h, q]].tolist() == top


def test_tiny_fp32_workload_is_dense():
    """Window (3,3,3) over a 2x2x2 tile grid covers everything."""
    c = CONFIGS["tiny-fp32"]
    kv_idx, kv_cnt, q_idx, q_cnt = oracle.index(c["grid"], c["tile"], windows_for("tiny-fp32"))
    assert np.all(kv_cnt == 8) and np.all(q_cnt == 8)
    assert np.all(kv_idx[:, :, :8] == np.arange(8))


def test_offsets_workload_counts():
    """Per-head windows of the offsets workload: 27/45/125 tiles per query."""
    c = CONFIGS["720p-shifted-perhead"]
    w = windows_for("720p-shifted-perhead")
    kv_idx, kv_cnt, q_idx, q_cnt = oracle.index(c["grid"], c["tile"], w, offsets_for("720p-shifted-perhead"))
    for h in range(c["H"]):
        assert np.all(kv_cnt[h] == np.prod(w[h]))
        assert q_cnt[h].sum() == kv_cnt[h].sum()


def test_capacity_too_small_is_rejected():
    with pytest.raises(ValueError):
        oracle.index((4, 4, 4), (1, 1, 1), [(3, 3, 3)], max_kv=26)
    with pytest.raises(ValueError):
        oracle.index((5, 0, 4), (2, 1, 1), [(3, 3, 3)])
