"""GPU parity on seeded random geometries: tile shapes with 16 to 64 tokens,
1 to 3 tiles per axis with the last tile cut by the grid or whole, per-head
windows of odd and even sizes, no / shared / per-head window shifts, both
border rules, text tokens or none, D = 64 or 128, B of 1 or 2 and H of 1
to 3, bf16 and fp32 (fp32 wherever a tile clipped by the grid holds a number
of tokens the bf16 kernels do not take).  Forward and backward in full
against the oracle."""
import numpy as np
import pytest
import torch

from oracle import oracle
from tests.gpu_util import Layer, assert_close, assert_lse, say, to_host
from tests.inputs import tensors

pytestmark = pytest.mark.gpu

TILES = [(1, 4, 4), (2, 2, 4), (1, 2, 8), (2, 4, 4), (3, 4, 4), (1, 4, 8), (2, 4, 8), (3, 2, 8)]


def case(i):
    g = np.random.default_rng(7000 + i)
    tile = TILES[int(g.integers(len(TILES)))]
    n = [int(g.integers(1, 4)) for _ in range(3)]
    grid = tuple((nd - 1) * td + int(g.integers(1, td + 1)) for nd, td in zip(n, tile))
    B, H = int(g.integers(1, 3)), int(g.integers(1, 4))
    D = int(g.choice([64, 128]))
    windows = [tuple(int(x) for x in g.choice([1, 2, 3, 5], size=3)) for _ in range(H)]
    T = int(np.prod([-(-a // b) for a, b in zip(grid, tile)]))
    kind = int(g.integers(3))
    offsets = None
    if kind == 1:
        offsets = g.integers(-1, 2, size=(T, 3)).astype(np.int32)
    elif kind == 2:
        offsets = g.integers(-1, 2, size=(H, T, 3)).astype(np.int32)
    border = "truncate" if g.integers(2) else "shift"
    n_text = int(g.integers(1, 41)) if g.integers(2) else 0
    dtype = "f32" if i % 4 == 3 else "bf16"
    # a tile longer than the grid on an axis holds the grid's extent there;
    # the bf16 kernels take tiles of a multiple of 16 tokens
    if int(np.prod([min(a, b) for a, b in zip(grid, tile)])) % 16:
        dtype = "f32"
    return grid, tile, B, H, D, windows, offsets, border, n_text, dtype


@pytest.mark.parametrize("i", range(48))
def test_random_geometry_forward_and_backward(i):
    grid, tile, B, H, D, windows, offsets, border, n_text, dtype = case(i)
    name = "random %d: grid %s tile %s B%d H%d D%d windows %s shifts %s %s text %d %s" % (
        i, grid, tile, B, H, D, windows, None if offsets is None else offsets.shape, border, n_text, dtype)
    say(name)
    N = int(np.prod(grid)) + n_text
    q, k, v, do = tensors(B, H, N, D, dtype, 7100 + i, with_dout=True)
    layer = Layer(grid, tile, windows, offsets, q, k, v, dtype, dout=do, border=border, n_text=n_text)
    o, lse = layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, offsets, border=border, n_text=n_text)
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, offsets, border=border, n_text=n_text)
    assert_close(to_host(o), ro, dtype, name + " O")
    if dtype == "bf16":
        assert_lse(to_host(lse), rl, dtype)
    else:
        assert_close(to_host(lse), rl, dtype, name + " LSE")
    for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_close(to_host(got), ref, dtype, name + " " + nm)
