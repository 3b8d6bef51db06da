"""Pins of the oracle's window options (CPU only): the truncating border
rule and per-head window shifts, the 3D-DSA variants of "MegaSlide-DiT"
(abstract: motion-adaptive local windows; the pages give no rule, so both
options are readings and offsets are inputs).

The truncating rule is pinned by hand-worked fixtures, by a second
characterisation (enumeration of the nearest centre and of the window's
members, in dense_ref), and by invariants; per-head shifts by reduction to
the shared-shift and single-head cases; attention with both options by the
dense masked-attention reference (torch routines)."""
import numpy as np
import pytest

from oracle import dense_ref, oracle
from tests.conftest import read_golden


def _axis_truncate(n, w, q, o):
    off = np.zeros((n, 3), np.int32)
    off[q, 2] = o
    kv_idx, kv_cnt, _, _ = oracle.index((1, 1, n), (1, 1, 1), [(1, 1, w)], off, border="truncate")
    lst = kv_idx[0, q, : kv_cnt[0, q]]
    return int(lst[0]), int(kv_cnt[0, q]), lst


@pytest.mark.parametrize("row", read_golden("window_axis_truncate.txt"), ids=lambda r: "-".join(r))
def test_truncate_axis_golden(row):
    n, w, q, o, start, count = map(int, row)
    s, c, lst = _axis_truncate(n, w, q, o)
    assert (s, c) == (start, count)
    assert list(lst) == list(range(start, start + count))


CASES = [
    # grid of 1-token tiles (tile coords = token coords), window, offset range
    ((3, 4, 7), (3, 3, 5), 0),
    ((4, 5, 6), (1, 3, 4), 2),
    ((2, 6, 3), (5, 1, 3), 3),
    ((5, 5, 5), (3, 3, 3), 1),
]


def _tile_windows_by_enumeration(n, win, offsets):
    """[T] list of sets: the truncated window of every query tile, built
    from dense_ref's enumeration (no clamp formula)."""
    T = n[0] * n[1] * n[2]
    out = []
    for q in range(T):
        qc = (q // (n[1] * n[2]), (q // n[2]) % n[1], q % n[2])
        o = (0, 0, 0) if offsets is None else offsets[q]
        axes = [dense_ref.window_truncated_by_enumeration(n[d], win[d], qc[d], int(o[d])) for d in range(3)]
        out.append({(a * n[1] + b) * n[2] + c
                    for a in range(axes[0][0], axes[0][0] + axes[0][1])
                    for b in range(axes[1][0], axes[1][0] + axes[1][1])
                    for c in range(axes[2][0], axes[2][0] + axes[2][1])})
    return out


@pytest.mark.parametrize("case", range(len(CASES)))
def test_truncate_lists_match_enumeration_and_transpose(case):
    n, win, orange = CASES[case]
    T = int(np.prod(n))
    g = np.random.default_rng(10 + case)
    off = g.integers(-orange, orange, endpoint=True, size=(T, 3)).astype(np.int32) if orange else None
    kv_idx, kv_cnt, q_idx, q_cnt = oracle.index(n, (1, 1, 1), [win], off, border="truncate")
    want = _tile_windows_by_enumeration(n, win, off)
    for q in range(T):
        lst = kv_idx[0, q, : kv_cnt[0, q]]
        assert list(lst) == sorted(want[q]), q
        assert np.all(kv_idx[0, q, kv_cnt[0, q]:] == -1)
    for k in range(T):
        attendees = [q for q in range(T) if k in want[q]]
        assert list(q_idx[0, k, : q_cnt[0, k]]) == attendees
    assert kv_cnt.sum() == q_cnt.sum()


def test_truncate_holds_clamped_centre_and_never_exceeds_window():
    n, win = (4, 5, 6), (3, 1, 5)
    T = int(np.prod(n))
    off = np.random.default_rng(3).integers(-4, 4, endpoint=True, size=(T, 3)).astype(np.int32)
    kv_idx, kv_cnt, _, _ = oracle.index(n, (1, 1, 1), [win], off, border="truncate")
    for q in range(T):
        qc = np.array([q // (n[1] * n[2]), (q // n[2]) % n[1], q % n[2]])
        centre = np.clip(qc + off[q], 0, np.array(n) - 1)
        cid = (centre[0] * n[1] + centre[1]) * n[2] + centre[2]
        assert cid in set(kv_idx[0, q, : kv_cnt[0, q]])
        assert 1 <= kv_cnt[0, q] <= np.prod(win)


def test_truncate_interior_equals_shift_and_border_is_smaller():
    """Away from the borders both rules give the same window; at a border
    the truncated window is a strict subset of the shifted one."""
    n, win = (5, 6, 10), (3, 3, 5)
    kv_t, cnt_t, _, _ = oracle.index(n, (1, 1, 1), [win], border="truncate")
    kv_s, cnt_s, _, _ = oracle.index(n, (1, 1, 1), [win])
    for q in range(int(np.prod(n))):
        qc = (q // (n[1] * n[2]), (q // n[2]) % n[1], q % n[2])
        interior = all(win[d] // 2 <= qc[d] <= n[d] - 1 - win[d] // 2 for d in range(3))
        a = set(kv_t[0, q, : cnt_t[0, q]])
        b = set(kv_s[0, q, : cnt_s[0, q]])
        if interior:
            assert a == b
        else:
            assert a < b


def test_truncate_mirror_symmetry_and_wide_window():
    n, win = (3, 4, 7), (3, 3, 5)
    kv, cnt, _, _ = oracle.index(n, (1, 1, 1), [win], border="truncate")
    T = int(np.prod(n))

    def mirror(t):
        a, b, c = t // (n[1] * n[2]), (t // n[2]) % n[1], t % n[2]
        return ((n[0] - 1 - a) * n[1] + (n[1] - 1 - b)) * n[2] + (n[2] - 1 - c)

    for q in range(T):
        assert set(mirror(k) for k in kv[0, q, : cnt[0, q]]) == set(kv[0, mirror(q), : cnt[0, mirror(q)]])
    # a window twice the grid (plus one) covers every tile from any centre
    kv, cnt, _, _ = oracle.index(n, (1, 1, 1), [tuple(2 * x + 1 for x in n)], border="truncate")
    assert np.all(cnt == T)


@pytest.mark.parametrize("border", ["shift", "truncate"])
def test_head_offsets_reduce_to_shared_and_single_head(border):
    n, tile = (3, 4, 6), (1, 1, 1)
    T = int(np.prod(n))
    windows = [(3, 3, 3), (1, 3, 5), (3, 1, 3)]
    H = len(windows)
    g = np.random.default_rng(21)
    per = g.integers(-2, 2, endpoint=True, size=(H, T, 3)).astype(np.int32)
    got = oracle.index(n, tile, windows, per, border=border)
    for h in range(H):
        one = oracle.index(n, tile, [windows[h]], per[h], border=border)
        for a, b in zip(got, one):
            assert np.array_equal(a[h], b[0]), h
    shared = per[0]
    rep = np.broadcast_to(shared, (H, T, 3)).copy()
    for a, b in zip(oracle.index(n, tile, windows, rep, border=border),
                    oracle.index(n, tile, windows, shared, border=border)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("border", ["shift", "truncate"])
def test_attention_options_match_torch_dense(border):
    """Forward and backward with per-head shifts (and either border rule)
    against dense masked attention (SDPA + autograd, float64)."""
    grid, tile = (4, 4, 6), (2, 2, 2)
    windows = [(1, 3, 3), (3, 1, 5)]
    B, H, D = 1, 2, 8
    N = int(np.prod(grid))
    T = int(np.prod([a // b for a, b in zip(grid, tile)]))
    g = np.random.default_rng(31)
    q, k, v, do = (g.standard_normal((B, H, N, D)).astype(np.float32) for _ in range(4))
    per = g.integers(-1, 1, endpoint=True, size=(H, T, 3)).astype(np.int32)
    o, lse = oracle.fwd(q, k, v, grid, tile, windows, per, border=border)
    dq, dk, dv = oracle.bwd(q, k, v, do, grid, tile, windows, per, border=border)
    ro, rl, rq, rk, rv = dense_ref.attention(q, k, v, grid, tile, windows, per, dout=do, border=border)
    for got, ref in ((o, ro), (lse, rl), (dq, rq), (dk, rk), (dv, rv)):
        assert np.max(np.abs(got - ref)) < 1e-10
