"""GPU parity on the degenerate shapes of the method: a grid of one tile,
tiles of one token, an axis of extent one, one-tile windows (block-diagonal
attention), and more heads than one launch of the index builder or the shift
producer covers (launches are split by 64 heads)."""
import numpy as np
import pytest
import torch

import sliding_tile_attention_amd as sta
from oracle import oracle, shift
from tests.gpu_util import Layer, assert_close, assert_lse, say, to_dev, to_host
from tests.inputs import tensors, tile_signal

pytestmark = pytest.mark.gpu


def _layer_vs_oracle(name, grid, tile, B, H, D, windows, dtype, seed, offsets=None):
    say("edge " + name)
    q, k, v, do = tensors(B, H, int(np.prod(grid)), D, dtype, seed, with_dout=True)
    layer = Layer(grid, tile, windows, offsets, q, k, v, dtype, dout=do)
    o, lse = layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, offsets)
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, offsets)
    assert_close(to_host(o), ro, dtype, name + " O")
    if dtype == "bf16":
        assert_lse(to_host(lse), rl, dtype)
    else:
        assert_close(to_host(lse), rl, dtype, name + " LSE")
    for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_close(to_host(got), ref, dtype, name + " " + nm)
    return q, k, v, o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_tile_grid_is_dense_attention(dtype):
    """One tile (T = 1): every window holds it, so the result is dense
    attention over the 32 tokens."""
    q, k, v, o, lse = _layer_vs_oracle("one tile " + dtype, (2, 4, 4), (2, 4, 4), 1, 2, 64, [(3, 3, 3), (1, 1, 1)],
                                       dtype, 170)
    ref = torch.nn.functional.scaled_dot_product_attention(*(torch.from_numpy(x).double() for x in (q, k, v)))
    assert_close(to_host(o), ref.numpy(), dtype, "one tile vs dense")


def test_one_token_tiles_attend_themselves():
    """Tiles of one token with one-tile windows: each query sees only its own
    key, so O = V and LSE = scale * <q, k> exactly in fp32 arithmetic."""
    grid, tile, D = (3, 2, 2), (1, 1, 1), 64
    q, k, v, o, lse = _layer_vs_oracle("one-token tiles", grid, tile, 1, 1, D, [(1, 1, 1)], "f32", 171)
    np.testing.assert_array_equal(to_host(o), v.astype(np.float64))
    want = (q.astype(np.float64) * k).sum(-1) / np.sqrt(D)
    np.testing.assert_allclose(to_host(lse), want, rtol=0, atol=1e-5)


def test_axis_of_extent_one():
    _layer_vs_oracle("flat grid", (1, 8, 12), (1, 4, 4), 2, 2, 128, [(3, 3, 3), (1, 1, 3)], "bf16", 172)


def test_one_tile_windows_are_block_diagonal():
    """Window (1,1,1): each tile attends to itself only: per-tile dense
    attention, checked against SDPA tile by tile."""
    grid, tile, D = (4, 8, 8), (2, 4, 4), 128
    q, k, v, o, lse = _layer_vs_oracle("block diagonal", grid, tile, 1, 1, D, [(1, 1, 1)], "bf16", 173)
    p = oracle.perm(grid, tile)
    L = int(np.prod(tile))
    inv = np.argsort(p)
    got = to_host(o)[0, 0]
    for t in range(int(np.prod(oracle.tiles_per_axis(grid, tile)))):
        toks = inv[t * L:(t + 1) * L]
        ref = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(x[0, 0, toks]).double()[None] for x in (q, k, v)))[0].numpy()
        assert_close(got[toks], ref, "bf16", "tile %d" % t)


def test_more_heads_than_one_launch():
    """70 heads: the index builder and the shift producer split their
    launches by 64 heads; lists bit-exact, shifts valid against the oracle,
    attention of the first and last heads against the oracle."""
    grid, tile, H, D = (4, 8, 12), (2, 4, 4), 70, 64
    g = np.random.default_rng(174)
    windows = [tuple(int(x) for x in w) for w in g.integers(1, 4, size=(H, 3))]
    geom = sta.Geometry(grid, tile)
    T = geom.num_tiles
    say("edge 70 heads")
    off = g.integers(-1, 1, endpoint=True, size=(H, T, 3)).astype(np.int32)
    idx = sta.StaIndex(geom, windows, torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    kv_idx, kv_cnt, q_idx, q_cnt = oracle.index(grid, tile, windows, off, idx.max_kv, idx.max_q)
    assert np.array_equal(idx.kv_idx.cpu().numpy(), kv_idx)
    assert np.array_equal(idx.q_idx.cpu().numpy(), q_idx)
    q, k = tile_signal(1, H, grid, tile, D, "bf16", 175, unit=True)
    qd, kd = (sta.tile_reorder(to_dev(x, "bf16"), geom) for x in (q, k))
    got = sta.window_shifts(qd, kd, geom, windows, (1, 1, 1)).cpu().numpy()
    ref, tab, cands = shift.shifts(q, k, grid, tile, windows, (1, 1, 1))
    where = {tuple(int(x) for x in c): i for i, c in enumerate(cands)}
    for h in range(H):
        for t in range(T):
            m = tab[h, t]
            assert m[where[tuple(int(x) for x in got[h, t])]] >= m.max() * (1 - 1e-4), (h, t)
    _, _, v, do = tensors(1, H, int(np.prod(grid)), D, "bf16", 176, with_dout=True)
    layer = Layer(grid, tile, windows, off, q, k, v, "bf16", dout=do)
    o, lse = layer.forward()
    torch.cuda.synchronize()
    for h in (0, H - 1):
        ro, rl = oracle.fwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], grid, tile, [windows[h]], off[h:h + 1])
        assert_close(to_host(o[:, h:h + 1]), ro, "bf16", "head %d O" % h)
        assert_lse(to_host(lse[:, h:h + 1]), rl, "bf16")


@pytest.mark.parametrize("border", ["shift", "truncate"])
def test_even_window_sizes(border):
    """Even window sizes start half a window below the centre (the start
    q + o - floor(w/2)); with both border rules and shifts, attention against
    the oracle."""
    grid, tile, B, H, D = (6, 8, 12), (2, 4, 4), 1, 2, 64
    T = int(np.prod(oracle.tiles_per_axis(grid, tile)))
    off = np.random.default_rng(177).integers(-1, 1, endpoint=True, size=(T, 3)).astype(np.int32)
    say("edge even windows " + border)
    q, k, v, do = tensors(B, H, int(np.prod(grid)), D, "bf16", 178, with_dout=True)
    windows = [(2, 2, 2), (2, 1, 4)]
    layer = Layer(grid, tile, windows, off, q, k, v, "bf16", dout=do, border=border)
    o, lse = layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, off, border=border)
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, off, border=border)
    assert_close(to_host(o), ro, "bf16", "even O")
    assert_lse(to_host(lse), rl, "bf16")
    for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_close(to_host(got), ref, "bf16", "even " + nm)


def test_batch_of_four():
    """B = 4 (16 slabs with H = 4) sharing one index: every slab against the
    oracle."""
    _layer_vs_oracle("batch of four", (4, 8, 12), (2, 4, 4), 4, 4, 128, [(3, 3, 3), (1, 3, 3), (3, 1, 1), (1, 1, 3)],
                     "bf16", 179)


@pytest.mark.parametrize("tiles_w", [64, 68])
def test_key_tile_order_at_and_past_its_limit(tiles_w):
    """The work plan orders dK/dV's key tiles by transposed-list length on
    grids of up to 4096 tiles and keeps tile order beyond: 4 x 16 x 64 = 4096
    tiles (ordered) and 4 x 16 x 68 = 4352 (plain order), 16-token tiles,
    moved-inward 3x3x5 windows whose transposed lists differ in length at
    the border.  dK/dV on whole key tiles (the least and the most attended,
    and two seeded), dQ on rows of corner and seeded tiles, against the
    oracle."""
    grid, tile, windows, D = (4, 64, 4 * tiles_w), (1, 4, 4), [(3, 3, 5)], 64
    name = "key-tile order, %d tiles" % (4 * 16 * tiles_w)
    say("edge " + name)
    N = int(np.prod(grid))
    q, k, v, do = tensors(1, 1, N, D, "bf16", 181, with_dout=True)
    layer = Layer(grid, tile, windows, None, q, k, v, "bf16", dout=do)
    layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    L, T = 16, 4 * 16 * tiles_w
    inv = np.argsort(oracle.perm(grid, tile))                    # tile-order slot -> raster token
    q_cnt = np.asarray(oracle.index(grid, tile, windows, None)[3])[0]
    g = np.random.default_rng(182)
    ktiles = [int(np.argmin(q_cnt)), int(np.argmax(q_cnt))] + [int(x) for x in g.choice(T, 2, replace=False)]
    krows = np.sort(np.concatenate([inv[t * L:(t + 1) * L] for t in ktiles]))
    qtiles = [0, T - 1] + [int(x) for x in g.choice(T, 2, replace=False)]
    qrows = np.sort(np.concatenate([inv[t * L:(t + 1) * L] for t in qtiles]))
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, None, qrows=qrows, krows=krows)
    pick = lambda t, rows: to_host(t.reshape(-1, D)[torch.from_numpy(rows).cuda()])
    assert_close(pick(dq, qrows), rq, "bf16", name + " dQ")
    assert_close(pick(dk, krows), rk, "bf16", name + " dK")
    assert_close(pick(dv, krows), rv, "bf16", name + " dV")
