"""GPU backward parity: libsta (reorder -> index -> sta_fwd -> sta_bwd ->
inverse reorder) against the CPU oracle on identical seeded inputs."""
import numpy as np
import pytest
import torch

from oracle import oracle
from tests.gpu_util import Layer, assert_close, say, to_host
from tests.inputs import tensors, workload

pytestmark = pytest.mark.gpu


SMALL = [
    # name, grid, tile, B, H, D, windows, offsets?
    ("L32-offsets-D128", (4, 8, 12), (2, 4, 4), 1, 3, 128, [(3, 3, 3), (1, 3, 3), (5, 5, 5)], True),
    ("L32-offsets-D64", (4, 8, 12), (2, 4, 4), 2, 2, 64, [(3, 1, 3), (1, 1, 1)], True),
    ("L48-ragged-D128", (6, 8, 8), (3, 4, 4), 1, 2, 128, [(3, 3, 3), (1, 1, 3)], False),
    ("L128-D128", (4, 16, 24), (2, 8, 8), 1, 2, 128, [(3, 3, 3), (1, 1, 1)], False),
    ("L384-D128", (12, 16, 24), (6, 8, 8), 1, 1, 128, [(3, 3, 3)], True),
    ("L256-D64", (8, 16, 24), (4, 8, 8), 1, 2, 64, [(1, 3, 3), (3, 3, 3)], False),
    ("L16-D128", (2, 4, 8), (1, 4, 4), 1, 2, 128, [(1, 1, 1), (3, 3, 3)], False),
]


def _offsets(grid, tile, use, seed=5):
    if not use:
        return None
    T = int(np.prod([a // b for a, b in zip(grid, tile)]))
    return np.random.default_rng(seed).integers([-1, -2, -2], [1, 2, 2], endpoint=True, size=(T, 3)).astype(np.int32)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0])
def test_bwd_bf16_small_full(case):
    name, grid, tile, B, H, D, windows, use_off = case
    say("bwd bf16 " + name)
    off = _offsets(grid, tile, use_off)
    N = int(np.prod(grid))
    q, k, v, do = tensors(B, H, N, D, "bf16", 91, with_dout=True)
    layer = Layer(grid, tile, windows, off, q, k, v, "bf16", dout=do)
    layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, off)
    assert_close(to_host(dq), rq, "bf16", name + " dQ")
    assert_close(to_host(dk), rk, "bf16", name + " dK")
    assert_close(to_host(dv), rv, "bf16", name + " dV")


def test_bwd_bf16_deterministic():
    """No atomics and a fixed reduction order: repeated backward calls, and a
    call on a second stream, give bit-identical dQ, dK and dV (here on a
    720P-shaped slab two tiles deep, 4 heads with shifted windows, about 1400
    workgroups per kernel)."""
    grid, tile, windows = (12, 48, 80), (6, 8, 8), [(3, 3, 5), (1, 3, 3)]
    say("bwd bf16 determinism " + str(grid))
    off = _offsets(grid, tile, True, seed=17)
    q, k, v, do = tensors(1, 4, int(np.prod(grid)), 128, "bf16", 93, with_dout=True)
    layer = Layer(grid, tile, windows * 2, off, q, k, v, "bf16", dout=do)
    layer.forward()
    first = [t.clone() for t in layer.backward()]
    for rep in range(3):
        for a, b, nm in zip(layer.backward(), first, ("dQ", "dK", "dV")):
            assert torch.equal(a, b), "repeat %d: %s differs" % (rep, nm)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        again = [t.clone() for t in layer.backward()]
    side.synchronize()
    for a, b, nm in zip(again, first, ("dQ", "dK", "dV")):
        assert torch.equal(a, b), "second stream: %s differs" % nm
    for t in first:
        assert torch.isfinite(t.float()).all()


def test_bwd_f32_tiny():
    """fp32 path (tiny workload geometry, whole-grid window) vs the oracle."""
    w = workload("tiny-fp32", with_dout=True)
    say("bwd f32 tiny-fp32 workload")
    layer = Layer(w["grid"], w["tile"], w["windows"], None, w["q"], w["k"], w["v"], "f32", dout=w["dout"])
    layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd(w["q"], w["k"], w["v"], w["dout"], w["grid"], w["tile"], w["windows"])
    for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_close(to_host(got), ref, "f32", nm)


def test_bwd_f32_offsets_d128():
    grid, tile = (4, 8, 12), (2, 4, 4)
    windows = [(3, 1, 3), (1, 3, 5)]
    off = np.random.default_rng(9).integers(-2, 3, size=(12, 3)).astype(np.int32)
    q, k, v, do = tensors(1, 2, 384, 128, "f32", 13, with_dout=True)
    say("bwd f32 offsets D128")
    layer = Layer(grid, tile, windows, off, q, k, v, "f32", dout=do)
    layer.forward(scale=0.05)
    dq, dk, dv = layer.backward(scale=0.05)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, off, scale=0.05)
    for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_close(to_host(got), ref, "f32", nm)


def test_bwd_720p_training_sampled():
    """Training workload at full size (115200 tokens, 24 heads, window 3x3x5):
    the whole forward + backward runs on the GPU in the benchmark's launch
    configuration; sampled dQ rows and sampled dK/dV rows (from the least and
    the most attended key tiles) are checked against the oracle, and two
    exact identities are checked on the whole tensors."""
    w = workload("720p-train")
    say("bwd bf16 720p-train workload (full size)")
    layer = Layer(w["grid"], w["tile"], w["windows"], None, w["q"], w["k"], w["v"], "bf16", dout=w["dout"])
    layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    B, H, N, D = w["q"].shape
    L = 384
    inv = np.argsort(oracle.perm(w["grid"], w["tile"]))          # tile-order slot -> raster token
    g = np.random.default_rng(55)
    # dQ: 3 heads x (2 corner tiles + 1 random tile) x 4 rows
    qrows = []
    for h in (0, 11, 23):
        for t in (0, 299, int(g.integers(0, 300))):
            qrows += [h * N + int(inv[t * L + s]) for s in g.choice(L, 4, replace=False)]
    # dK/dV: head 3, key tile 0 (12 query tiles attend it) and tile (2,2,4)=144 (140 attend it)
    krows = []
    for t in (0, 144):
        krows += [3 * N + int(inv[t * L + s]) for s in g.choice(L, 3, replace=False)]
    qrows, krows = np.array(qrows, np.int64), np.array(krows, np.int64)
    say("oracle: %d dQ rows, %d dK/dV rows" % (len(qrows), len(krows)))
    rq, rk, rv = oracle.bwd(w["q"], w["k"], w["v"], w["dout"], w["grid"], w["tile"], w["windows"],
                            qrows=qrows, krows=krows)
    pick = lambda t, rows: to_host(t.reshape(-1, D)[torch.from_numpy(rows).cuda()])
    assert_close(pick(dq, qrows), rq, "bf16", "dQ")
    assert_close(pick(dk, krows), rk, "bf16", "dK")
    assert_close(pick(dv, krows), rv, "bf16", "dV")
    # Identities (rows of P sum to 1, rows of dS to 0): per (b, h)
    #   sum_j dV_j = sum_i dO_i   and   sum_j dK_j = 0.
    # With bf16 storage the residual is of order 2^-9 * |dV_j| * sqrt(N) per
    # component, tiny next to |sum_i dO_i| ~ sqrt(N); gates leave a wide margin.
    sdv = dv.float().sum(2)
    sdo = torch.from_numpy(w["dout"]).cuda().sum(2)
    rel = (torch.linalg.norm(sdv - sdo) / torch.linalg.norm(sdo)).item()
    assert rel < 1e-3, "sum dV vs sum dO: rel %.2e" % rel
    sdk = dk.float().sum(2)
    scale_k = torch.sqrt((dk.float() ** 2).sum(2) * N).clamp_min(1e-30)   # |sum| if all rows aligned
    assert (sdk.abs() / scale_k).max().item() < 1e-2
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()


@pytest.mark.parametrize("case", __import__("tests.test_gpu_fwd", fromlist=["OPTION_CASES"]).OPTION_CASES,
                         ids=lambda c: c[0])
def test_bwd_bf16_window_options(case):
    """Backward with truncated windows (transposed lists of unequal length)
    and per-head shifts."""
    from tests.test_gpu_fwd import option_offsets
    name, grid, tile, B, H, D, windows, border, kind = case
    say("bwd bf16 options " + name)
    T = int(np.prod([a // b for a, b in zip(grid, tile)]))
    off = option_offsets(kind, H, T, 9)
    N = int(np.prod(grid))
    q, k, v, do = tensors(B, H, N, D, "bf16", 93, with_dout=True)
    layer = Layer(grid, tile, windows, off, q, k, v, "bf16", dout=do, border=border)
    layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, off, border=border)
    assert_close(to_host(dq), rq, "bf16", name + " dQ")
    assert_close(to_host(dk), rk, "bf16", name + " dK")
    assert_close(to_host(dv), rv, "bf16", name + " dV")


def test_f32_window_options():
    """fp32 path with truncated windows and per-head shifts (forward and backward)."""
    grid, tile, windows = (4, 8, 12), (2, 4, 4), [(3, 3, 3), (1, 3, 5)]
    B, H, D = 1, 2, 64
    T = int(np.prod([a // b for a, b in zip(grid, tile)]))
    off = np.random.default_rng(12).integers(-2, 2, endpoint=True, size=(H, T, 3)).astype(np.int32)
    N = int(np.prod(grid))
    q, k, v, do = tensors(B, H, N, D, "f32", 95, with_dout=True)
    say("f32 window options")
    layer = Layer(grid, tile, windows, off, q, k, v, "f32", dout=do, border="truncate")
    o, _ = layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    ro, _ = oracle.fwd(q, k, v, grid, tile, windows, off, border="truncate")
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, off, border="truncate")
    for name, got, ref in (("O", o, ro), ("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        assert_close(to_host(got), ref, "f32", name)
