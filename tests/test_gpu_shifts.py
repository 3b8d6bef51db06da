"""GPU parity of the window-shift producer (sta_window_shifts) and of
attention whose windows are shifted per batch item.

The producer's rule is this library's reading of the motion-adaptive windows
of 3D-DSA ("MegaSlide-DiT", abstract), written out in oracle/shift.py.  The
GPU decides in fp32 and the oracle in fp64, so a GPU choice is valid when its
oracle mass is within a relative MASS_TOL of the largest, and it must be the
oracle's own choice wherever the largest mass leads every different one by
more than 2 * MASS_TOL (candidates whose windows coincide have bit-equal
masses on both sides, so their tie-break is compared exactly).  Planted
displacements with one-tile windows must be recovered exactly.

MASS_TOL: the GPU's masses differ from exact ones by the fp32 rounding of
the tile means (sums of <= 384 rows: relative error ~1e-6 of the row
magnitudes), of the logits (D <= 128 terms), of exp (a few ulp) and of sums
of <= 125 window terms (<= 125 * 2^-24 = 7.5e-6); with logits below 25 in
these inputs, 1e-4 bounds the relative mass error with margin."""
import numpy as np
import pytest
import torch

import sliding_tile_attention_amd as sta
from oracle import oracle, shift
from tests.gpu_util import Layer, assert_close, assert_fp8, assert_lse, say, to_dev, to_host
from tests.inputs import tensors, tile_signal, windows_for

pytestmark = pytest.mark.gpu

MASS_TOL = 1e-4


def _gpu_shifts(q, k, grid, tile, windows, radius, dtype, border="shift", per_batch=False, n_text=0):
    geom = sta.Geometry(tuple(grid), tuple(tile))
    tq, tk = (sta.tile_reorder(to_dev(x, dtype), geom, n_text=n_text) for x in (q, k))
    off = sta.window_shifts(tq, tk, geom, [tuple(int(a) for a in w) for w in windows], radius, border=border,
                            per_batch=per_batch, n_text=n_text)
    torch.cuda.synchronize()
    return off.cpu().numpy()


def _check(got, q, k, grid, tile, windows, radius, border="shift", per_batch=False, n_text=0, what=""):
    """Validity of every choice and exactness where the oracle's is clear.
    Returns (number of query tiles, number compared exactly)."""
    nv = int(np.prod(grid))
    windows = [tuple(int(a) for a in w) for w in windows]
    ref, tab, cands = shift.shifts(q[:, :, :nv], k[:, :, :nv], grid, tile, windows, radius, border=border,
                                   pooled=not per_batch)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    where = {tuple(int(x) for x in c): i for i, c in enumerate(cands)}
    g, t, r = got.reshape(-1, 3), tab.reshape(-1, len(cands)), ref.reshape(-1, 3)
    exact = 0
    for i in range(g.shape[0]):
        c = where.get(tuple(int(x) for x in g[i]))
        assert c is not None, "%s: tile %d shift %s outside the search box" % (what, i, g[i])
        m = t[i]
        best = m.max()
        assert m[c] >= best * (1 - MASS_TOL), "%s: tile %d mass %.9g, best %.9g" % (what, i, m[c], best)
        distinct = np.unique(m)
        if len(distinct) == 1 or distinct[-1] > distinct[-2] * (1 + 2 * MASS_TOL):
            assert np.array_equal(g[i], r[i]), "%s: tile %d shift %s, oracle %s" % (what, i, g[i], r[i])
            exact += 1
    return g.shape[0], exact


DISP = [(0, 1, -1), (1, 0, 1), (-1, -1, 0)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("grid", [(6, 8, 12), (5, 7, 10)], ids=["whole", "cut"])
@pytest.mark.parametrize("D", [64, 128])
def test_planted_displacement_is_recovered(dtype, grid, D):
    """Key tile c carries the content of query tile c - d_h: with one-tile
    windows the producer returns d_h wherever that partner lies in the grid."""
    tile, B, H = (2, 4, 4), 2, 3
    say("shifts planted %s %s D=%d" % (dtype, grid, D))
    q, k = tile_signal(B, H, grid, tile, D, dtype, 70, amp=2.0, disp=DISP)
    windows, radius = [(1, 1, 1)] * H, (1, 1, 1)
    got = _gpu_shifts(q, k, grid, tile, windows, radius, dtype)
    n = oracle.tiles_per_axis(grid, tile)
    qc = np.stack(np.unravel_index(np.arange(int(np.prod(n))), n), 1)
    for h in range(H):
        inside = np.all((qc + DISP[h] >= 0) & (qc + DISP[h] < np.array(n)), axis=1)
        assert inside.sum() >= 4
        assert np.all(got[h, inside] == np.array(DISP[h])), (h, got[h, inside])
    _check(got, q, k, grid, tile, windows, radius, what="planted")


CASES = [
    # name, grid, tile, B, H, D, windows, radius, border, per_batch, n_text, dtype
    ("L128-pooled", (8, 16, 16), (2, 8, 8), 2, 2, 128, [(3, 1, 1), (1, 3, 3)], (1, 1, 1), "shift", False, 0, "bf16"),
    ("cut-truncate-text-per-batch", (5, 9, 11), (2, 4, 4), 2, 2, 128, [(3, 3, 3), (1, 3, 5)], (1, 2, 1),
     "truncate", True, 37, "bf16"),
    ("f32-pooled-B3", (6, 8, 12), (2, 4, 4), 3, 2, 64, [(1, 1, 1), (3, 3, 3)], (2, 1, 1), "shift", False, 0, "f32"),
    ("64-tiles-per-head-windows", (16, 32, 32), (4, 8, 8), 1, 4, 128, [(3, 3, 3), (3, 3, 5), (5, 5, 5), (1, 3, 3)],
     (1, 2, 2), "shift", False, 0, "bf16"),
    ("truncate-D64-text", (8, 16, 24), (4, 8, 8), 2, 2, 64, [(3, 3, 3), (1, 1, 3)], (1, 1, 2), "truncate", False,
     19, "bf16"),
    ("window-over-grid", (6, 8, 12), (2, 4, 4), 1, 2, 128, [(5, 5, 5), (3, 9, 1)], (1, 1, 1), "shift", False, 0,
     "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_shifts_match_oracle(case):
    name, grid, tile, B, H, D, windows, radius, border, per_batch, nt, dtype = case
    say("shifts " + name)
    q, k = tile_signal(B, H, grid, tile, D, dtype, 71, amp=1.0, n_text=nt)
    got = _gpu_shifts(q, k, grid, tile, windows, radius, dtype, border, per_batch, nt)
    total, exact = _check(got, q, k, grid, tile, windows, radius, border, per_batch, nt, what=name)
    say("  %d query tiles, %d compared exactly" % (total, exact))
    assert exact >= total // 2


def test_zero_radius_and_equal_keys():
    """No search radius: every shift is zero.  Equal key tiles (k = 1): every
    window of the shifting border rule holds the same mass and the tie goes
    to the zero shift."""
    grid, tile, B, H, D = (6, 8, 12), (2, 4, 4), 2, 2, 128
    q, k = tile_signal(B, H, grid, tile, D, "bf16", 72)
    got = _gpu_shifts(q, k, grid, tile, [(3, 3, 3)] * H, (0, 0, 0), "bf16")
    assert not got.any()
    ones = np.ones_like(k)
    got = _gpu_shifts(q, ones, grid, tile, [(1, 3, 3), (3, 1, 1)], (1, 1, 1), "bf16")
    assert not got.any()
    _check(got, q, ones, grid, tile, [(1, 3, 3), (3, 1, 1)], (1, 1, 1), what="equal keys")


def test_raster_order_tie():
    """Two shifts of equal size with bit-equal masses (key tiles (0,1,0) and
    (0,0,1) carry query tile 0's content, one-tile windows): the first in
    raster order, (0,0,1), is chosen, as in the oracle."""
    grid, tile, D = (6, 8, 12), (2, 4, 4), 64
    n = oracle.tiles_per_axis(grid, tile)
    N = int(np.prod(grid))
    t, h, w = np.unravel_index(np.arange(N), grid)
    tid = ((t // tile[0]) * n[1] + h // tile[1]) * n[2] + w // tile[2]
    q = np.zeros((1, 1, N, D), np.float32)
    k = np.zeros((1, 1, N, D), np.float32)
    q[0, 0, tid == 0, 0] = 3.0
    for c in ((0, 1, 0), (0, 0, 1)):
        k[0, 0, tid == (c[0] * n[1] + c[1]) * n[2] + c[2], 0] = 3.0
    for dtype in ("bf16", "f32"):
        got = _gpu_shifts(q, k, grid, tile, [(1, 1, 1)], (1, 1, 1), dtype)
        assert tuple(got[0, 0]) == (0, 0, 1), (dtype, got[0, 0])
        _check(got, q, k, grid, tile, [(1, 1, 1)], (1, 1, 1), what="raster tie " + dtype)


def test_shifts_720p_full_size():
    """The 720p per-head workload's shapes (24 heads, windows 3x3x3 / 3x3x5 /
    5x5x5, bf16, D 128; tiles carrying content of their own on top of the
    N(0,1) draws) with a search radius of one tile: every choice against
    the oracle's masses."""
    grid, tile = (30, 48, 80), (6, 8, 8)
    windows = windows_for("720p-shifted-perhead")
    say("shifts 720p full size")
    q, k = tile_signal(1, 24, grid, tile, 128, "bf16", 74, amp=1.0)
    got = _gpu_shifts(q, k, grid, tile, windows, (1, 1, 1), "bf16")
    total, exact = _check(got, q, k, grid, tile, windows, (1, 1, 1), what="720p")
    say("  %d query tiles, %d compared exactly" % (total, exact))
    assert exact >= total // 2


def test_shifts_deterministic():
    grid, tile = (16, 32, 32), (4, 8, 8)
    q, k = tile_signal(1, 4, grid, tile, 128, "bf16", 73)
    a = _gpu_shifts(q, k, grid, tile, [(3, 3, 3)] * 4, (1, 1, 1), "bf16")
    b = _gpu_shifts(q, k, grid, tile, [(3, 3, 3)] * 4, (1, 1, 1), "bf16")
    assert np.array_equal(a, b)


# ---- attention with windows shifted per batch item ---------------------

def _per_batch_offsets(B, H, grid, tile, seed):
    T = int(np.prod(oracle.tiles_per_axis(grid, tile)))
    return np.random.default_rng(seed).integers([-1, -1, -2], [1, 1, 2], endpoint=True,
                                                size=(B, H, T, 3)).astype(np.int32)


@pytest.mark.parametrize("border", ["shift", "truncate"])
def test_per_batch_index_lists(border):
    grid, tile, B, H = (5, 9, 11), (2, 4, 4), 3, 2
    windows = [(3, 3, 3), (1, 3, 5)]
    off = _per_batch_offsets(B, H, grid, tile, 80)
    geom = sta.Geometry(grid, tile)
    idx = sta.StaIndex(geom, windows, torch.from_numpy(off).cuda(), border=border)
    torch.cuda.synchronize()
    assert idx.num_heads == B * H and idx.batch == B
    for b in range(B):
        kv_idx, kv_cnt, q_idx, q_cnt = oracle.index(grid, tile, windows, off[b], idx.max_kv, idx.max_q,
                                                    border=border)
        s = slice(b * H, (b + 1) * H)
        assert np.array_equal(idx.kv_cnt[s].cpu().numpy(), kv_cnt)
        assert np.array_equal(idx.kv_idx[s].cpu().numpy(), kv_idx)
        assert np.array_equal(idx.q_cnt[s].cpu().numpy(), q_cnt)
        assert np.array_equal(idx.q_idx[s].cpu().numpy(), q_idx)


PB_CASES = [
    # name, grid, tile, B, H, D, windows, border, n_text, dtype
    ("bf16-D128", (6, 8, 12), (2, 4, 4), 2, 2, 128, [(3, 3, 3), (1, 3, 3)], "shift", 0, "bf16"),
    ("bf16-cut-truncate-text", (5, 9, 11), (2, 4, 4), 2, 2, 64, [(3, 3, 3), (1, 1, 3)], "truncate", 21, "bf16"),
    ("f32-B3", (4, 8, 8), (2, 4, 4), 3, 1, 64, [(1, 3, 3)], "shift", 0, "f32"),
]


@pytest.mark.parametrize("case", PB_CASES, ids=lambda c: c[0])
def test_per_batch_attention_matches_oracle(case):
    """Forward and backward with one list set per (b, h): every batch item
    against the oracle run with that item's shifts."""
    name, grid, tile, B, H, D, windows, border, nt, dtype = case
    say("per-batch attention " + name)
    off = _per_batch_offsets(B, H, grid, tile, 81)
    S = int(np.prod(grid)) + nt
    q, k, v, do = tensors(B, H, S, D, dtype, 82, with_dout=True)
    layer = Layer(grid, tile, windows, off, q, k, v, dtype, dout=do, border=border, n_text=nt)
    assert layer.index.num_heads == B * H
    o, lse = layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    for b in range(B):
        sl = slice(b, b + 1)
        ro, rl = oracle.fwd(q[sl], k[sl], v[sl], grid, tile, windows, off[b], border=border, n_text=nt)
        rq, rk, rv = oracle.bwd(q[sl], k[sl], v[sl], do[sl], grid, tile, windows, off[b], border=border, n_text=nt)
        tag = "%s b=%d " % (name, b)
        assert_close(to_host(o[sl]), ro, dtype, tag + "O")
        if dtype == "bf16":
            assert_lse(to_host(lse[sl]), rl, dtype, tag + "LSE")
        else:
            assert_close(to_host(lse[sl]), rl, dtype, tag + "LSE")
        for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
            assert_close(to_host(got[sl]), ref, dtype, tag + nm)


def test_per_batch_index_with_equal_shifts_equals_shared_index():
    """B*H list sets holding the same shifts for every batch item give
    bit-identical outputs to one shared list set (same kernels, same lists)."""
    grid, tile, B, H, D = (6, 8, 12), (2, 4, 4), 2, 2, 128
    T = int(np.prod(oracle.tiles_per_axis(grid, tile)))
    off_h = np.random.default_rng(83).integers(-1, 1, endpoint=True, size=(H, T, 3)).astype(np.int32)
    q, k, v, do = tensors(B, H, int(np.prod(grid)), D, "bf16", 84, with_dout=True)
    windows = [(3, 3, 3), (1, 3, 5)]
    shared = Layer(grid, tile, windows, off_h, q, k, v, "bf16", dout=do)
    per_b = Layer(grid, tile, windows, np.stack([off_h] * B), q, k, v, "bf16", dout=do)
    a = shared.forward() + shared.backward()
    b = per_b.forward() + per_b.backward()
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_producer_feeds_per_batch_attention():
    """The whole adaptive path on device: shifts chosen per batch item from
    q and k, the B*H-set index built from them, attention; against the
    oracle run with the shifts the GPU chose (checked valid above)."""
    grid, tile, B, H, D = (8, 16, 16), (2, 8, 8), 2, 2, 128
    windows = [(3, 1, 1), (1, 3, 3)]
    disp = np.array([[(0, 1, 0), (1, 0, -1)], [(-1, 0, 1), (0, -1, 0)]])
    # unit variance: the bf16 gates are those of N(0,1) inputs
    q, k = tile_signal(B, H, grid, tile, D, "bf16", 85, amp=1.0, disp=disp, unit=True)
    _, _, v, do = tensors(B, H, int(np.prod(grid)), D, "bf16", 86, with_dout=True)
    geom = sta.Geometry(grid, tile)
    layer = Layer(grid, tile, windows, None, q, k, v, "bf16", dout=do)
    off = sta.window_shifts(layer.q, layer.k, geom, windows, (1, 1, 1), per_batch=True)
    layer.index = sta.StaIndex(geom, windows, off)
    o, lse = layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    offs = off.cpu().numpy()
    _check(offs, q, k, grid, tile, windows, (1, 1, 1), per_batch=True, what="producer")
    for b in range(B):
        sl = slice(b, b + 1)
        ro, rl = oracle.fwd(q[sl], k[sl], v[sl], grid, tile, windows, offs[b])
        rq, rk, rv = oracle.bwd(q[sl], k[sl], v[sl], do[sl], grid, tile, windows, offs[b])
        assert_close(to_host(o[sl]), ro, "bf16", "O b=%d" % b)
        assert_lse(to_host(lse[sl]), rl, "bf16")
        for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
            assert_close(to_host(got[sl]), ref, "bf16", "%s b=%d" % (nm, b))


def test_per_batch_index_with_quantized_forward():
    """The quantized forward with one list set per (b, h): every batch item
    against the quantized method's oracle run with that item's shifts."""
    from oracle import quant
    grid, tile, B, H, D = (6, 8, 16), (2, 8, 8), 2, 2, 128
    windows = [(3, 1, 3), (1, 3, 1)]
    say("per-batch quantized forward")
    off = _per_batch_offsets(B, H, grid, tile, 87)
    q, k, v = tensors(B, H, int(np.prod(grid)), D, "bf16", 88)
    layer = Layer(grid, tile, windows, off, q, k, v, "bf16")
    o, lse = layer.forward(precision="fp8")
    torch.cuda.synchronize()
    for b in range(B):
        sl = slice(b, b + 1)
        assert_fp8(to_host(o[sl]), to_host(lse[sl]), quant.fwd(q[sl], k[sl], v[sl], grid, tile, windows, off[b],
                                                             bound=True), "fp8 b=%d" % b)
