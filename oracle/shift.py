"""Oracle of the window-shift producer (test infrastructure only: loaded by
tests/, never by the library).

3D Deformable Slide Attention moves each query tile's window with the
content ("MegaSlide-DiT", abstract: motion-adaptive local windows); the
pages give no rule for the shift.  This library's reading: the shift of a
query tile's window is the one, within a search radius, whose window holds
the most tile-level attention mass.

  1. Tile means of Q and K over each tile's tokens (a tile cut by the grid
     border over the tokens it holds), per (b, h); pooled over the batch by
     their mean unless the shifts are wanted per batch item.
  2. z_qk = scale * <qbar_q, kbar_k> for every pair of tiles.
  3. For every candidate shift o in [-r_t, r_t] x [-r_h, r_h] x [-r_w, r_w]:
     mass(o) = sum over the tiles k of window(q, o) of len_k * exp(z_qk - zmax_q),
     zmax_q = max_k z_qk, with the window rule of the index (shift or
     truncate border).
  4. The shift with the largest mass; among candidates of equal mass the
     one with the smallest |o_t| + |o_h| + |o_w|, then the first in raster
     order of (o_t, o_h, o_w).

Everything here is float64; the GPU decides the argmax in fp32, so parity
compares the masses (a shift whose mass is within a relative 1e-5 of the
largest is a valid choice) and the shifts where the choice is clear.
"""
import itertools

import numpy as np

from oracle import oracle


def tile_means(x, grid, tile):
    """[B,H,N,D] raster-order tokens -> ([B,H,T,D] tile means, [T] lengths)."""
    B, H, N, D = np.shape(x)
    t, h, w = np.unravel_index(np.arange(N), grid)
    n = oracle.tiles_per_axis(grid, tile)
    tid = ((t // tile[0]) * n[1] + h // tile[1]) * n[2] + w // tile[2]
    T = int(np.prod(n))
    lens = np.bincount(tid, minlength=T).astype(np.float64)
    sums = np.zeros((B, H, T, D))
    np.add.at(sums, (slice(None), slice(None), tid), np.asarray(x, np.float64))
    return sums / lens[None, None, :, None], lens


def candidates(radius):
    """Candidate shifts in raster order."""
    return [np.array(o, np.int32) for o in itertools.product(*[range(-r, r + 1) for r in radius])]


def window_lists(grid, tile, window, o, border):
    """[T] lists of the key tiles in the window of every query tile shifted by o."""
    T = int(np.prod(oracle.tiles_per_axis(grid, tile)))
    off = np.tile(np.asarray(o, np.int32), (T, 1))
    kv_idx, kv_cnt, _, _ = oracle.index(grid, tile, [window], off, border=border)
    return [kv_idx[0, q, : kv_cnt[0, q]] for q in range(T)]


def masses(q, k, grid, tile, window, radius, scale, border="shift", pooled=True):
    """mass[b or 0][h][q][candidate] for one window size shared by the heads
    given (callers pass one head's window)."""
    qm, lens = tile_means(q, grid, tile)
    km, _ = tile_means(k, grid, tile)
    if pooled:
        qm, km = qm.mean(axis=0, keepdims=True), km.mean(axis=0, keepdims=True)
    z = scale * np.einsum("bhqd,bhkd->bhqk", qm, km)
    z = z - z.max(axis=3, keepdims=True)
    e = lens[None, None, None, :] * np.exp(z)
    cands = candidates(radius)
    out = np.zeros(z.shape[:3] + (len(cands),))
    for c, o in enumerate(cands):
        lists = window_lists(grid, tile, window, o, border)
        for qq, lst in enumerate(lists):
            out[:, :, qq, c] = e[:, :, qq, lst].sum(axis=-1)
    return out, cands


def choose(mass, cands):
    """Step 4 on mass[..., candidate] -> offsets [..., 3] and the chosen masses."""
    l1 = np.array([np.abs(o).sum() for o in cands])
    order = np.lexsort((np.arange(len(cands)), l1))             # by |o|_1, then raster order
    best = mass.max(axis=-1, keepdims=True)
    pick = np.zeros(mass.shape[:-1], np.int64)
    done = np.zeros(mass.shape[:-1], bool)
    for c in order:
        hit = (mass[..., c] == best[..., 0]) & ~done
        pick[hit] = c
        done |= hit
    return np.stack([cands[c] for c in pick.ravel()]).reshape(mass.shape[:-1] + (3,)), best[..., 0]


def shifts(q, k, grid, tile, windows, radius, scale=None, border="shift", pooled=True):
    """Offsets [H,T,3] (pooled) or [B,H,T,3], plus the mass tables [.., H, T, C]
    and the candidate list, for [B,H,N,D] raster-order q, k (video tokens)."""
    B, H, N, D = np.shape(q)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out, tables = [], []
    for h in range(H):
        m, cands = masses(np.asarray(q)[:, h:h + 1], np.asarray(k)[:, h:h + 1], grid, tile, windows[h], radius,
                          scale, border, pooled)
        off, _ = choose(m, cands)
        out.append(off[:, 0])
        tables.append(m[:, 0])
    off = np.stack(out, axis=1)
    tab = np.stack(tables, axis=1)
    return (off[0], tab[0], cands) if pooled else (off, tab, cands)
