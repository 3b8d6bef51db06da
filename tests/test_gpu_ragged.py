"""GPU parity on grids the tile does not divide: border tiles cut by the
grid hold only their tokens (compact tile order).  Permutation and index
bit-exact, attention (bf16 and fp32, forward and backward) against the CPU
oracle, and the 720p latent grid (30,45,80) at full size."""
import numpy as np
import pytest
import torch

import sliding_tile_attention_amd as sta
from oracle import oracle
from tests.gpu_util import Layer, assert_close, assert_lse, say, to_host
from tests.inputs import tensors

pytestmark = pytest.mark.gpu

REORDER = [
    # grid, tile, outer, row_bytes
    ((5, 6, 7), (2, 4, 4), 3, 256),        # cut on every axis, 16-byte path
    ((30, 45, 80), (6, 8, 8), 24, 256),    # 720p latent grid, bf16 D=128
    ((30, 45, 80), (6, 8, 8), 24, 4),      # its LSE
    ((7, 9, 10), (3, 4, 4), 2, 6),         # byte path
    ((3, 5, 3), (2, 2, 2), 2, 12),         # 4-byte path (the hand-worked fixture's grid)
    ((2, 3, 5), (4, 4, 8), 4, 32),         # tile longer than the grid on every axis
]


@pytest.mark.parametrize("case", REORDER, ids=lambda c: "%s-%s-%d-%d" % c)
def test_ragged_reorder_bit_exact_and_round_trip(case):
    grid, tile, outer, row_bytes = case
    say("ragged reorder %s" % (case,))
    N = int(np.prod(grid))
    geom = sta.Geometry(grid, tile)
    g = torch.Generator(device="cpu").manual_seed(8)
    src_h = torch.randint(0, 256, (outer, N, row_bytes), dtype=torch.uint8, generator=g)
    src = src_h.cuda()
    dst = torch.empty_like(src)
    sta.sta_tile_reorder(src, dst, outer, row_bytes, geom, False)
    back = torch.empty_like(src)
    sta.sta_tile_reorder(dst, back, outer, row_bytes, geom, True)
    torch.cuda.synchronize()
    expect = np.empty_like(src_h.numpy())
    expect[:, oracle.perm(grid, tile), :] = src_h.numpy()
    assert np.array_equal(dst.cpu().numpy(), expect)
    assert torch.equal(back.cpu(), src_h)


@pytest.mark.parametrize("seed", range(8))
def test_ragged_index_random_geometries(seed):
    g = np.random.default_rng(200 + seed)
    grid = tuple(int(x) for x in g.integers(1, 14, size=3))
    tile = tuple(int(x) for x in g.integers(1, 6, size=3))
    windows = [tuple(int(x) for x in w) for w in g.integers(1, 6, size=(2, 3))]
    geom = sta.Geometry(grid, tile)
    say("ragged index %s %s" % (grid, tile))
    T = geom.num_tiles
    off = g.integers(-2, 2, endpoint=True, size=(T, 3)).astype(np.int32) if seed % 2 else None
    idx = sta.StaIndex(geom, windows, None if off is None else torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    kv_idx, kv_cnt, q_idx, q_cnt = oracle.index(grid, tile, windows, off, idx.max_kv, idx.max_q)
    assert np.array_equal(idx.kv_cnt.cpu().numpy(), kv_cnt)
    assert np.array_equal(idx.kv_idx.cpu().numpy(), kv_idx)
    assert np.array_equal(idx.q_cnt.cpu().numpy(), q_cnt)
    assert np.array_equal(idx.q_idx.cpu().numpy(), q_idx)


CASES = [
    # name, grid, tile, B, H, D, windows, offsets kind, border, n_text
    ("cut-all-L32-D128", (5, 7, 9), (2, 4, 4), 1, 2, 128, [(3, 3, 3), (1, 3, 3)], None, "shift", 0),
    ("cut-w-L384-D128", (12, 16, 21), (6, 8, 8), 1, 2, 128, [(3, 3, 3), (1, 1, 3)], "shared", "shift", 0),
    ("cut-h-L384-D64", (12, 13, 16), (6, 8, 8), 2, 1, 64, [(3, 3, 3)], None, "shift", 0),
    ("cut-t-L128-D128-text", (5, 16, 16), (2, 8, 8), 1, 2, 128, [(3, 1, 1), (1, 3, 3)], "head", "truncate", 70),
    ("cut-all-L48-D64", (7, 9, 10), (3, 4, 4), 1, 2, 64, [(1, 3, 3), (3, 3, 5)], "head", "shift", 0),
    ("tile-over-grid-D128", (2, 5, 9), (4, 8, 8), 1, 1, 128, [(1, 1, 1)], None, "shift", 9),
]


def _offsets(kind, H, T, seed=11):
    if kind is None:
        return None
    shape = (T, 3) if kind == "shared" else (H, T, 3)
    return np.random.default_rng(seed).integers([-1, -2, -2], [1, 2, 2], endpoint=True,
                                                size=shape).astype(np.int32)


def _run(case, dtype, seed):
    name, grid, tile, B, H, D, windows, kind, border, nt = case
    T = int(np.prod(oracle.tiles_per_axis(grid, tile)))
    off = _offsets(kind, H, T)
    S = int(np.prod(grid)) + nt
    q, k, v, do = tensors(B, H, S, D, dtype, seed, with_dout=True)
    layer = Layer(grid, tile, windows, off, q, k, v, dtype, dout=do, border=border, n_text=nt)
    o, lse = layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, off, border=border, n_text=nt)
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, off, border=border, n_text=nt)
    return (o, lse, dq, dk, dv), (ro, rl, rq, rk, rv)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_ragged_bf16_forward_backward(case):
    say("ragged bf16 " + case[0])
    (o, lse, dq, dk, dv), (ro, rl, rq, rk, rv) = _run(case, "bf16", 140)
    assert_close(to_host(o), ro, "bf16", case[0] + " O")
    assert_lse(to_host(lse), rl, "bf16")
    for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_close(to_host(got), ref, "bf16", case[0] + " " + nm)


@pytest.mark.parametrize("case", [CASES[0], CASES[4]], ids=lambda c: c[0])
def test_ragged_f32_forward_backward(case):
    say("ragged f32 " + case[0])
    got, ref = _run(case, "f32", 141)
    for a, b, nm in zip(got, ref, ("O", "LSE", "dQ", "dK", "dV")):
        assert_close(to_host(a), b, "f32", case[0] + " " + nm)


def test_ragged_720p_latent_grid_sampled():
    """The 720p latent grid (30,45,80) with tile (6,8,8): the last tile row
    along h holds 5 of 8 rows.  24 heads, window 3x3x5, forward and backward
    whole on the GPU; sampled rows of whole and cut tiles against the oracle,
    plus the whole-tensor identities."""
    grid, tile, windows = (30, 45, 80), (6, 8, 8), [(3, 3, 5)] * 24
    B, H, D = 1, 24, 128
    N = int(np.prod(grid))
    say("ragged bf16 720p latent grid (full size)")
    q, k, v, do = tensors(B, H, N, D, "bf16", 150, with_dout=True)
    layer = Layer(grid, tile, windows, None, q, k, v, "bf16", dout=do)
    o, lse = layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    p = oracle.perm(grid, tile)
    inv = np.argsort(p)                          # tile-order slot -> raster token
    t, h, w = np.unravel_index(np.arange(N), grid)
    n = oracle.tiles_per_axis(grid, tile)
    tid = ((t // tile[0]) * n[1] + h // tile[1]) * n[2] + w // tile[2]
    g = np.random.default_rng(151)
    cut = [5 * 10 + 0, 5 * 10 + 9, 4 * 60 + 5 * 10 + 4]           # tiles of the cut tile row (ih = 5)
    whole = [0, 299 - 50, int(g.integers(0, 50))]
    qrows, krows = [], []
    for hh in (0, 12, 23):
        for tl in cut + whole:
            toks = np.flatnonzero(tid == tl)
            qrows += [hh * N + int(x) for x in g.choice(toks, 3, replace=False)]
    for tl in (cut[0], 0):
        toks = np.flatnonzero(tid == tl)
        krows += [7 * N + int(x) for x in g.choice(toks, 2, replace=False)]
    qrows, krows = np.array(qrows, np.int64), np.array(krows, np.int64)
    say("oracle: %d query rows, %d key rows" % (len(qrows), len(krows)))
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, rows=qrows)
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, qrows=qrows, krows=krows)
    pick = lambda x, rows: to_host(x.reshape(-1, D)[torch.from_numpy(rows).cuda()])
    assert_close(pick(o, qrows), ro, "bf16", "O")
    assert_lse(to_host(lse.reshape(-1)[torch.from_numpy(qrows).cuda()]), rl, "bf16")
    assert_close(pick(dq, qrows), rq, "bf16", "dQ")
    assert_close(pick(dk, krows), rk, "bf16", "dK")
    assert_close(pick(dv, krows), rv, "bf16", "dV")
    sdv, sdo = dv.float().sum(2), torch.from_numpy(do).cuda().sum(2)
    assert (torch.linalg.norm(sdv - sdo) / torch.linalg.norm(sdo)).item() < 1e-3
    sdk = dk.float().sum(2)
    assert (sdk.abs() / torch.sqrt((dk.float() ** 2).sum(2) * N).clamp_min(1e-30)).max().item() < 1e-2
    assert inv.shape == (N,)
