"""GPU: token permutation (bit-exact) and block-sparse index (exact lists)
against the oracle."""
import numpy as np
import pytest
import torch

import sliding_tile_attention_amd as sta
from oracle import oracle
from tests.gpu_util import say
from tests.inputs import CONFIGS, WORKLOADS, offsets_for, windows_for

pytestmark = pytest.mark.gpu


REORDER_CASES = [
    # grid, tile, outer, row_bytes
    ((4, 8, 8), (2, 4, 4), 2, 128),        # tiny workload, fp32 D=32 rows
    ((8, 24, 40), (4, 8, 8), 24, 256),     # mid workload, bf16 D=128
    ((30, 48, 80), (6, 8, 8), 24, 256),    # 720P workload, bf16 D=128
    ((30, 48, 80), (6, 8, 8), 24, 4),      # its LSE
    ((6, 10, 9), (3, 5, 3), 3, 6),         # odd row size: byte path
    ((4, 6, 10), (2, 3, 5), 2, 12),        # 4-byte path
    ((3, 4, 5), (1, 1, 1), 2, 16),         # unit tiles: identity
    ((2, 8, 8), (2, 8, 8), 5, 32),         # one tile: identity
    ((6, 4, 16), (2, 4, 4), 1, 3072),      # [B,N,H,D] style: row = H*D*2
]


@pytest.mark.parametrize("case", REORDER_CASES, ids=lambda c: "%s-%s-%d-%d" % c)
def test_reorder_bit_exact_and_round_trip(case):
    grid, tile, outer, row_bytes = case
    say("reorder %s" % (case,))
    N = int(np.prod(grid))
    geom = sta.Geometry(grid, tile)
    g = torch.Generator(device="cpu").manual_seed(7)
    src_h = torch.randint(0, 256, (outer, N, row_bytes), dtype=torch.uint8, generator=g)
    src = src_h.cuda()
    dst = torch.empty_like(src)
    sta.sta_tile_reorder(src, dst, outer, row_bytes, geom, False)
    back = torch.empty_like(src)
    sta.sta_tile_reorder(dst, back, outer, row_bytes, geom, True)
    torch.cuda.synchronize()
    perm = oracle.perm(grid, tile)
    expect = np.empty_like(src_h.numpy())
    expect[:, perm, :] = src_h.numpy()
    assert np.array_equal(dst.cpu().numpy(), expect)
    assert torch.equal(back.cpu(), src_h)


def _check_index(grid, tile, windows, offsets, border="shift"):
    geom = sta.Geometry(grid, tile)
    off = None if offsets is None else torch.from_numpy(np.ascontiguousarray(offsets, np.int32)).cuda()
    idx = sta.StaIndex(geom, windows, off, border=border)
    torch.cuda.synchronize()
    ref = oracle.index(grid, tile, windows, offsets, max_kv=idx.max_kv, max_q=idx.max_q, border=border)
    got = [x.cpu().numpy() for x in (idx.kv_idx, idx.kv_cnt, idx.q_idx, idx.q_cnt)]
    for name, a, b in zip(("kv_idx", "kv_cnt", "q_idx", "q_cnt"), got, ref):
        assert np.array_equal(a, b), name


@pytest.mark.parametrize("cfg", WORKLOADS)
def test_index_workloads(cfg):
    c = CONFIGS[cfg]
    say("index workload %s" % cfg)
    _check_index(c["grid"], c["tile"], windows_for(cfg), offsets_for(cfg))


@pytest.mark.parametrize("seed", range(20))
def test_index_random_geometries(seed):
    g = np.random.default_rng(1000 + seed)
    n = g.integers(1, 9, size=3)
    tile = tuple(int(x) for x in g.integers(1, 4, size=3))
    grid = tuple(int(a * b) for a, b in zip(n, tile))
    H = int(g.integers(1, 5))
    windows = g.integers(1, 10, size=(H, 3))
    offsets = g.integers(-4, 5, size=(int(np.prod(n)), 3)).astype(np.int32) if seed % 2 else None
    say("index random seed %d grid %s tile %s H %d" % (seed, grid, tile, H))
    _check_index(grid, tile, windows, offsets)


def test_index_forward_only():
    """Without transposed buffers only the forward lists are written."""
    c = CONFIGS["mid-7680"]
    geom = sta.Geometry(c["grid"], c["tile"])
    say("index forward only")
    idx = sta.StaIndex(geom, windows_for("mid-7680"), None, transposed=False)
    torch.cuda.synchronize()
    ref = oracle.index(c["grid"], c["tile"], windows_for("mid-7680"), None, max_kv=idx.max_kv)
    assert np.array_equal(idx.kv_idx.cpu().numpy(), ref[0])
    assert np.array_equal(idx.kv_cnt.cpu().numpy(), ref[1])


@pytest.mark.parametrize("seed", range(12))
def test_index_options_random_geometries(seed):
    """Truncated windows and per-head shifts (the 3D-DSA index options):
    every list bit-exact against the oracle."""
    g = np.random.default_rng(2000 + seed)
    n = g.integers(1, 9, size=3)
    tile = tuple(int(x) for x in g.integers(1, 4, size=3))
    grid = tuple(int(a * b) for a, b in zip(n, tile))
    H = int(g.integers(1, 5))
    T = int(np.prod(n))
    windows = g.integers(1, 10, size=(H, 3))
    border = "truncate" if seed % 3 else "shift"
    kind = seed % 4
    offsets = (None if kind == 0 else
               g.integers(-4, 5, size=(T, 3)).astype(np.int32) if kind == 1 else
               g.integers(-4, 5, size=(H, T, 3)).astype(np.int32))
    say("index options seed %d grid %s tile %s H %d border %s offsets %s" %
        (seed, grid, tile, H, border, None if offsets is None else offsets.shape))
    _check_index(grid, tile, windows, offsets, border)


def test_index_options_720p_shape():
    """Per-head windows, per-head shifts and truncation at the 720P tile grid."""
    c = CONFIGS["720p-shifted-perhead"]
    H = 24
    g = np.random.default_rng(77)
    offsets = g.integers([-1, -2, -2], [1, 2, 2], endpoint=True, size=(H, 300, 3)).astype(np.int32)
    say("index options 720p")
    _check_index(c["grid"], c["tile"], windows_for("720p-shifted-perhead"), offsets, "truncate")


def test_tile_reorder_wrapper_writes_out():
    """The tensor-level wrapper: [..., N, C] rows permuted into a caller's out
    tensor (returned), bit-exact against the oracle's permutation, and back."""
    grid, tile = (8, 24, 40), (4, 8, 8)
    say("tile_reorder wrapper %s %s" % (grid, tile))
    geom = sta.Geometry(grid, tile)
    N = int(np.prod(grid))
    g = torch.Generator(device="cpu").manual_seed(11)
    x_h = torch.randint(-2 ** 15, 2 ** 15, (2, 3, N, 64), dtype=torch.int16, generator=g).view(torch.bfloat16)
    x = x_h.cuda()
    out = torch.empty_like(x)
    got = sta.tile_reorder(x, geom, out=out)
    assert got is out
    back = sta.tile_reorder(out, geom, inverse=True)
    torch.cuda.synchronize()
    expect = np.empty_like(x_h.view(torch.int16).numpy())
    expect[:, :, oracle.perm(grid, tile), :] = x_h.view(torch.int16).numpy()
    assert np.array_equal(out.cpu().view(torch.int16).numpy(), expect)
    assert torch.equal(back.cpu().view(torch.int16), x_h.view(torch.int16))
