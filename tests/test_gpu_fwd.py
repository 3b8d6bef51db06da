"""GPU forward parity: libsta (reorder -> index -> sta_fwd -> inverse reorder)
against the CPU oracle on identical seeded inputs."""
import numpy as np
import pytest
import torch

from oracle import oracle
from tests.gpu_util import Layer, assert_close, assert_lse, sample_rows, say, to_host
from tests.inputs import CONFIGS, offsets_for, tensors, windows_for, workload

pytestmark = pytest.mark.gpu


SMALL = [
    # name, grid, tile, B, H, D, windows, offsets?
    ("L32-offsets-D64", (4, 8, 12), (2, 4, 4), 2, 3, 64, [(3, 3, 3), (1, 1, 1), (3, 1, 5)], True),
    ("L32-offsets-D128", (4, 8, 12), (2, 4, 4), 1, 3, 128, [(3, 3, 3), (1, 3, 3), (5, 5, 5)], True),
    ("L48-ragged-D128", (6, 8, 8), (3, 4, 4), 1, 2, 128, [(3, 3, 3), (1, 1, 3)], False),
    ("L48-ragged-D64", (6, 8, 16), (3, 4, 4), 2, 2, 64, [(1, 3, 3), (3, 3, 3)], True),
    ("L128-D128", (4, 16, 24), (2, 8, 8), 1, 2, 128, [(3, 3, 3), (1, 1, 1)], False),
    ("L384-D128", (12, 16, 24), (6, 8, 8), 1, 2, 128, [(3, 3, 3), (1, 3, 3)], True),
    ("L384-D64", (12, 16, 16), (6, 8, 8), 1, 2, 64, [(1, 1, 1), (3, 3, 3)], False),
    ("L256-D128-wide", (8, 16, 40), (4, 8, 8), 1, 1, 128, [(3, 3, 5)], False),
    ("L16-D64", (2, 4, 8), (1, 4, 4), 1, 2, 64, [(1, 1, 1), (3, 3, 3)], False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_fwd_bf16_small_full(case):
    name, grid, tile, B, H, D, windows, use_off = case
    say("fwd bf16 " + name)
    n = [a // b for a, b in zip(grid, tile)]
    T = int(np.prod(n))
    off = np.random.default_rng(5).integers([-1, -2, -2], [1, 2, 2], endpoint=True, size=(T, 3)).astype(
        np.int32) if use_off else None
    N = int(np.prod(grid))
    q, k, v = tensors(B, H, N, D, "bf16", 77)
    layer = Layer(grid, tile, windows, off, q, k, v, "bf16")
    o, lse = layer.forward()
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, off)
    assert_close(to_host(o), ro, "bf16", name + " O")
    assert_lse(to_host(lse), rl, "bf16")


def test_fwd_f32_tiny_workload():
    """Tiny fp32 workload: full tensor against the oracle (also = dense)."""
    w = workload("tiny-fp32")
    say("fwd f32 tiny-fp32 workload")
    layer = Layer(w["grid"], w["tile"], w["windows"], None, w["q"], w["k"], w["v"], "f32")
    o, lse = layer.forward()
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(w["q"], w["k"], w["v"], w["grid"], w["tile"], w["windows"])
    assert_close(to_host(o), ro, "f32", "O")
    assert_close(to_host(lse), rl, "f32", "LSE")


def test_fwd_f32_offsets_d128():
    grid, tile = (4, 8, 12), (2, 4, 4)
    windows = [(3, 1, 3), (1, 3, 5)]
    off = np.random.default_rng(9).integers(-2, 3, size=(12, 3)).astype(np.int32)
    q, k, v = tensors(1, 2, 384, 128, "f32", 12)
    say("fwd f32 offsets D128")
    layer = Layer(grid, tile, windows, off, q, k, v, "f32")
    o, lse = layer.forward(scale=0.05)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, off, scale=0.05)
    assert_close(to_host(o), ro, "f32", "O")
    assert_close(to_host(lse), rl, "f32", "LSE")


def test_fwd_mid_workload():
    """Mid workload (7680 tokens, 24 heads): two heads in full, every head sampled."""
    w = workload("mid-7680")
    say("fwd bf16 mid-7680 workload")
    layer = Layer(w["grid"], w["tile"], w["windows"], None, w["q"], w["k"], w["v"], "bf16")
    o, lse = layer.forward()
    torch.cuda.synchronize()
    o, lse = to_host(o), to_host(lse)
    B, H, N, D = w["q"].shape
    full = np.arange(2 * N, dtype=np.int64)   # heads 0 and 1 of batch 0
    samp = sample_rows(B, H, N, 256, w["grid"], w["tile"], 2, 8, seed=2)
    rows = np.unique(np.concatenate([full, samp]))
    ro, rl = oracle.fwd(w["q"], w["k"], w["v"], w["grid"], w["tile"], w["windows"], rows=rows)
    assert_close(o.reshape(-1, D)[rows], ro, "bf16", "O")
    assert_lse(lse.reshape(-1)[rows], rl, "bf16")


@pytest.mark.parametrize("cfg", ["720p", "720p-shifted-perhead"])
def test_fwd_720p_sampled(cfg):
    """Full 115200-token shape, every head, in the launch configuration the
    benchmark times; sampled rows (corner tiles + seeded tiles) vs oracle."""
    w = workload(cfg)
    say("fwd bf16 workload %s (full size, sampled check)" % cfg)
    layer = Layer(w["grid"], w["tile"], w["windows"], w["offsets"], w["q"], w["k"], w["v"], "bf16")
    o, lse = layer.forward()
    torch.cuda.synchronize()
    B, H, N, D = w["q"].shape
    rows = sample_rows(B, H, N, 384, w["grid"], w["tile"], 4, 4, seed=w["seed"])   # 8 corner + 4 seeded tiles
    ro, rl = oracle.fwd(w["q"], w["k"], w["v"], w["grid"], w["tile"], w["windows"], w["offsets"], rows=rows)
    o = o.reshape(-1, D)[torch.from_numpy(rows).cuda()]
    assert_close(to_host(o), ro, "bf16", "O")
    assert_lse(to_host(lse.reshape(-1)[torch.from_numpy(rows).cuda()]), rl, "bf16")
    assert torch.isfinite(layer.o).all()


def test_fwd_workspace_reuse_and_streams():
    """The bf16 forward takes its work plan from the stream's cached
    workspace: interleaved calls of two shapes (the buffer is reused and
    grows), and a call on a second stream, must give bit-identical results
    to the first call of each shape (the kernels are deterministic), and
    that first call matches the oracle."""
    say("fwd bf16 workspace reuse / streams")
    shapes = [((4, 8, 12), (2, 4, 4), 1, 2, 128, [(3, 3, 3), (1, 3, 3)]),
              ((6, 8, 8), (3, 4, 4), 2, 1, 128, [(3, 3, 3)])]
    layers, firsts = [], []
    for i, (grid, tile, B, H, D, windows) in enumerate(shapes):
        q, k, v = tensors(B, H, int(np.prod(grid)), D, "bf16", 300 + i)
        layer = Layer(grid, tile, windows, None, q, k, v, "bf16")
        o, lse = layer.forward()
        torch.cuda.synchronize()
        ro, rl = oracle.fwd(q, k, v, grid, tile, windows)
        assert_close(to_host(o), ro, "bf16", "first call O")
        layers.append(layer)
        firsts.append((o.clone(), lse.clone()))
    for rep in range(3):
        for layer, (o0, l0) in zip(layers, firsts):
            o, lse = layer.forward()
            assert torch.equal(o, o0) and torch.equal(lse, l0), "repeat %d differs" % rep
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        outs = [layer.forward() for layer in layers]
    side.synchronize()
    for (o, lse), (o0, l0) in zip(outs, firsts):
        assert torch.equal(o, o0) and torch.equal(lse, l0), "second stream differs"


OPTION_CASES = [
    # name, grid, tile, B, H, D, windows, border, offsets kind (None / "shared" / "head")
    ("trunc-L32-D128", (4, 8, 12), (2, 4, 4), 1, 3, 128, [(3, 3, 3), (1, 3, 3), (5, 5, 5)], "truncate", None),
    ("trunc-headoff-L48-D64", (6, 8, 16), (3, 4, 4), 2, 2, 64, [(1, 3, 3), (3, 3, 5)], "truncate", "head"),
    ("shift-headoff-L128-D128", (4, 16, 24), (2, 8, 8), 1, 2, 128, [(3, 3, 3), (1, 1, 3)], "shift", "head"),
    ("trunc-shared-L384-D128", (12, 16, 24), (6, 8, 8), 1, 2, 128, [(3, 3, 3), (1, 3, 3)], "truncate", "shared"),
]


def option_offsets(kind, H, T, seed):
    g = np.random.default_rng(seed)
    if kind is None:
        return None
    shape = (T, 3) if kind == "shared" else (H, T, 3)
    return g.integers([-1, -2, -2], [1, 2, 2], endpoint=True, size=shape).astype(np.int32)


@pytest.mark.parametrize("case", OPTION_CASES, ids=lambda c: c[0])
def test_fwd_bf16_window_options(case):
    """Truncated windows (lists of unequal length) and per-head shifts."""
    name, grid, tile, B, H, D, windows, border, kind = case
    say("fwd bf16 options " + name)
    T = int(np.prod([a // b for a, b in zip(grid, tile)]))
    off = option_offsets(kind, H, T, 9)
    N = int(np.prod(grid))
    q, k, v = tensors(B, H, N, D, "bf16", 91)
    layer = Layer(grid, tile, windows, off, q, k, v, "bf16", border=border)
    o, lse = layer.forward()
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, off, border=border)
    assert_close(to_host(o), ro, "bf16", name + " O")
    assert_lse(to_host(lse), rl, "bf16")
