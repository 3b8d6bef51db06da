"""GPU parity of the raster layout (sta_attn_opts.layout = STA_LAYOUT_RASTER):
the attention kernels read and write raster-order tensors directly, with no
reorder pass.

Against the oracle (which works in raster order itself): bf16 and fp32
forward and backward, with shifted, per-head, truncated and per-batch
windows.  Against the tile-order path: the same kernels do the same
arithmetic on the same rows in the same order, only the addresses differ,
so every output must equal the tile-order output permuted to raster order
bit for bit (bf16, fp32, the window-shift producer); at the 720P shape this
is checked on whole tensors.  The quantized forward's smoothing mean sums
the rows in the layout's order, so there the two agree to rounding."""
import numpy as np
import pytest
import torch

import sliding_tile_attention_amd as sta
from oracle import oracle
from tests.gpu_util import Layer, assert_close, assert_fp8, assert_lse, say, to_dev, to_host
from tests.inputs import tensors, tile_signal, windows_for

pytestmark = pytest.mark.gpu


def _offsets(kind, B, H, T, seed=91):
    g = np.random.default_rng(seed)
    shape = {None: None, "shared": (T, 3), "head": (H, T, 3), "batch": (B, H, T, 3)}[kind]
    if shape is None:
        return None
    return g.integers([-1, -1, -2], [1, 1, 2], endpoint=True, size=shape).astype(np.int32)


class Raster:
    """Raster-order device tensors and the index."""

    def __init__(self, grid, tile, windows, offsets, q, k, v, dtype, dout=None, border="shift"):
        self.geom = sta.Geometry(tuple(grid), tuple(tile))
        self.windows = [tuple(int(x) for x in w) for w in windows]
        off = None if offsets is None else torch.from_numpy(np.ascontiguousarray(offsets, np.int32)).cuda()
        self.index = sta.StaIndex(self.geom, self.windows, off, border=border)
        self.q, self.k, self.v = (to_dev(x, dtype) for x in (q, k, v))
        self.dout = None if dout is None else to_dev(dout, dtype)

    def forward(self, precision="default"):
        self.o, self.lse = sta.forward(self.q, self.k, self.v, self.geom, self.index, precision=precision,
                                       layout="raster")
        return self.o, self.lse

    def backward(self):
        return sta.backward(self.q, self.k, self.v, self.o, self.lse, self.dout, self.geom, self.index,
                            layout="raster")


CASES = [
    # name, grid, tile, B, H, D, windows, offsets, border
    ("L32-plane16-D64", (4, 8, 12), (2, 4, 4), 1, 2, 64, [(3, 3, 3), (1, 3, 1)], None, "shift"),
    ("L128-D128-head-shifts", (8, 16, 24), (2, 8, 8), 1, 2, 128, [(3, 1, 3), (1, 3, 3)], "head", "shift"),
    ("L256-D128-truncate", (8, 24, 24), (4, 8, 8), 1, 2, 128, [(3, 3, 3), (1, 1, 3)], "shared", "truncate"),
    ("L64-per-batch", (6, 8, 16), (1, 8, 8), 2, 2, 128, [(3, 1, 3), (1, 3, 1)], "batch", "shift"),
    ("plane32-D64", (4, 16, 16), (4, 4, 8), 2, 1, 64, [(1, 3, 3)], "shared", "shift"),
    # the walk's other branches: planes of 8 rows (a block spans four planes), tw = 16, tw = 1
    ("plane8-L32", (8, 4, 12), (4, 2, 4), 1, 2, 64, [(3, 3, 3), (1, 1, 3)], "head", "shift"),
    ("tw16-plane128-L256", (4, 16, 32), (2, 8, 16), 1, 2, 128, [(3, 1, 1), (1, 3, 1)], None, "truncate"),
    ("tw1-plane16-L64", (8, 32, 3), (4, 16, 1), 1, 1, 64, [(1, 3, 3)], "shared", "shift"),
]


def _run(case, dtype, seed):
    name, grid, tile, B, H, D, windows, kind, border = case
    T = int(np.prod(oracle.tiles_per_axis(grid, tile)))
    off = _offsets(kind, B, H, T)
    q, k, v, do = tensors(B, H, int(np.prod(grid)), D, dtype, seed, with_dout=True)
    r = Raster(grid, tile, windows, off, q, k, v, dtype, dout=do, border=border)
    o, lse = r.forward()
    dq, dk, dv = r.backward()
    torch.cuda.synchronize()
    refs = []
    for b in range(B):
        sl = slice(b, b + 1)
        ob = off[b] if kind == "batch" else off
        ro, rl = oracle.fwd(q[sl], k[sl], v[sl], grid, tile, windows, ob, border=border)
        rq, rk, rv = oracle.bwd(q[sl], k[sl], v[sl], do[sl], grid, tile, windows, ob, border=border)
        refs.append((ro, rl, rq, rk, rv))
    ref = [np.concatenate([x[i] for x in refs]) for i in range(5)]
    return (o, lse, dq, dk, dv), ref, (q, k, v, do, off)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_raster_bf16_matches_oracle_and_tile_order(case):
    say("raster bf16 " + case[0])
    got, ref, (q, k, v, do, off) = _run(case, "bf16", 160)
    names = ("O", "LSE", "dQ", "dK", "dV")
    for a, b, nm in zip(got, ref, names):
        if nm == "LSE":
            assert_lse(to_host(a), b, "bf16", case[0] + " LSE")
        else:
            assert_close(to_host(a), b, "bf16", case[0] + " " + nm)
    # the tile-order path, permuted back to raster order: bit-identical
    name, grid, tile, B, H, D, windows, kind, border = case
    layer = Layer(grid, tile, windows, off, q, k, v, "bf16", dout=do, border=border)
    t = layer.forward() + layer.backward()
    torch.cuda.synchronize()
    for a, b, nm in zip(got, t, names):
        assert torch.equal(a, b), case[0] + " " + nm + " differs from the tile-order path"


@pytest.mark.parametrize("case", [CASES[0], CASES[3]], ids=lambda c: c[0])
def test_raster_f32_matches_oracle_and_tile_order(case):
    say("raster f32 " + case[0])
    got, ref, (q, k, v, do, off) = _run(case, "f32", 161)
    for a, b, nm in zip(got, ref, ("O", "LSE", "dQ", "dK", "dV")):
        assert_close(to_host(a), b, "f32", case[0] + " " + nm)
    name, grid, tile, B, H, D, windows, kind, border = case
    layer = Layer(grid, tile, windows, off, q, k, v, "f32", dout=do, border=border)
    t = layer.forward() + layer.backward()
    torch.cuda.synchronize()
    for a, b in zip(got, t):
        assert torch.equal(a, b)


def test_raster_fp8_matches_quantized_oracle():
    """The quantized forward codes Q, K, V per tile from raster rows: against
    the quantized method's oracle within its gates, and against the
    tile-order path to rounding (the smoothing mean of K sums the rows in
    the layout's order, so the LSE correction and rarely a K code differ in
    the last bit)."""
    from oracle import quant
    grid, tile, B, H, D = (8, 16, 24), (2, 8, 8), 2, 2, 128
    windows = [(3, 3, 3), (1, 3, 5)]
    say("raster fp8")
    q, k, v = tensors(B, H, int(np.prod(grid)), D, "bf16", 162)
    r = Raster(grid, tile, windows, None, q, k, v, "bf16")
    o, lse = r.forward(precision="fp8")
    layer = Layer(grid, tile, windows, None, q, k, v, "bf16")
    to, tl = layer.forward(precision="fp8")
    torch.cuda.synchronize()
    assert_fp8(to_host(o), to_host(lse), quant.fwd(q, k, v, grid, tile, windows, bound=True), "raster fp8")
    assert_close(to_host(o), to_host(to), "bf16", "raster fp8 O vs tile order")
    assert float((lse - tl).abs().max()) <= 1e-5


def test_raster_window_shifts_equal_tile_order():
    grid, tile, B, H, D = (8, 16, 24), (2, 8, 8), 2, 3, 128
    windows = [(3, 3, 3), (1, 3, 5), (3, 1, 1)]
    say("raster window shifts")
    q, k = tile_signal(B, H, grid, tile, D, "bf16", 163)
    geom = sta.Geometry(grid, tile)
    qd, kd = to_dev(q, "bf16"), to_dev(k, "bf16")
    for per_batch in (False, True):
        a = sta.window_shifts(qd, kd, geom, windows, (1, 1, 1), per_batch=per_batch, layout="raster")
        b = sta.window_shifts(sta.tile_reorder(qd, geom), sta.tile_reorder(kd, geom), geom, windows, (1, 1, 1),
                              per_batch=per_batch)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_raster_720p_full_size():
    """The 720P training shape (24 heads, window 3x3x5, D 128): raster
    forward and backward equal the tile-order path bit for bit on whole
    tensors, and sampled rows match the oracle."""
    grid, tile, B, H, D = (30, 48, 80), (6, 8, 8), 1, 24, 128
    windows = [(3, 3, 5)] * H
    N = int(np.prod(grid))
    say("raster 720p full size")
    q, k, v, do = tensors(B, H, N, D, "bf16", 164, with_dout=True)
    r = Raster(grid, tile, windows, None, q, k, v, "bf16", dout=do)
    got = r.forward() + r.backward()
    layer = Layer(grid, tile, windows, None, q, k, v, "bf16", dout=do)
    t = layer.forward() + layer.backward()
    torch.cuda.synchronize()
    for a, b, nm in zip(got, t, ("O", "LSE", "dQ", "dK", "dV")):
        assert torch.equal(a, b), "720p " + nm
    g = np.random.default_rng(165)
    rows = np.sort(g.choice(H * N, 48, replace=False)).astype(np.int64)
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, rows=rows)
    pick = torch.from_numpy(rows).cuda()
    assert_close(to_host(got[0].reshape(-1, D)[pick]), ro, "bf16", "720p O")
    assert_lse(to_host(got[1].reshape(-1)[pick]), rl, "bf16")
