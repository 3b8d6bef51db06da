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


def _identities(dq, dk, dv, dout, what):
    """Whole-tensor identities (rows of P sum to 1, rows of dS to 0): per
    (b, h), sum_j dV_j = sum_i dO_i and sum_j dK_j = 0.  With bf16 storage the
    residual is of order 2^-9 |dV_j| sqrt(N) per component, tiny next to
    |sum_i dO_i| ~ sqrt(N); the gates leave a wide margin."""
    N = dv.shape[2]
    sdv = dv.float().sum(2)
    sdo = torch.from_numpy(dout).cuda().sum(2)
    rel = (torch.linalg.norm(sdv - sdo) / torch.linalg.norm(sdo)).item()
    assert rel < 1e-3, "%s: sum dV vs sum dO: rel %.2e" % (what, rel)
    sdk = dk.float().sum(2)
    scale_k = torch.sqrt((dk.float() ** 2).sum(2) * N).clamp_min(1e-30)   # |sum| if all rows aligned
    worst = (sdk.abs() / scale_k).max().item()
    assert worst < 1e-2, "%s: sum dK: %.2e" % (what, worst)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()


def _tile_rows(inv, h, N, L, t, slots):
    """Flat row ids (head h, batch 0) of tile-order slots of tile t."""
    return [h * N + int(inv[t * L + x]) for x in slots]


def _check_rows(w, dq, dk, dv, qrows, krows, what, offsets=None):
    """dQ on qrows, dK and dV on krows, against the oracle."""
    B, H, N, D = w["q"].shape
    qrows, krows = np.array(qrows, np.int64), np.array(krows, np.int64)
    say("%s: oracle on %d dQ rows, %d dK/dV rows" % (what, len(qrows), len(krows)))
    rq, rk, rv = oracle.bwd(w["q"], w["k"], w["v"], w["dout"], w["grid"], w["tile"], w["windows"], offsets,
                            qrows=qrows, krows=krows)
    pick = lambda t, rows: to_host(t.reshape(-1, D)[torch.from_numpy(rows).cuda()])
    assert_close(pick(dq, qrows), rq, "bf16", what + " dQ")
    assert_close(pick(dk, krows), rk, "bf16", what + " dK")
    assert_close(pick(dv, krows), rv, "bf16", what + " dV")


def _run(w, offsets=None):
    layer = Layer(w["grid"], w["tile"], w["windows"], offsets, w["q"], w["k"], w["v"], "bf16", dout=w["dout"])
    layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    return dq, dk, dv


def _train_720p():
    w = workload("720p-train")
    say("bwd bf16 720p-train workload (full size)")
    dq, dk, dv = _run(w)
    inv = np.argsort(oracle.perm(w["grid"], w["tile"]))          # tile-order slot -> raster token
    return w, dq, dk, dv, inv


def test_bwd_720p_training_sampled():
    """Training workload at full size (115200 tokens, 24 heads, window 3x3x5)
    in the benchmark's launch configuration.  dQ: rows of the 8 corner tiles
    and one seeded tile in every head.  dK/dV: the whole key tiles 0 (12
    query tiles attend it) and (2,2,4) = 144 (140 attend it) in heads 3 and
    17.  Plus the whole-tensor identities."""
    w, dq, dk, dv, inv = _train_720p()
    B, H, N, D = w["q"].shape
    L = 384
    g = np.random.default_rng(55)
    corners = [0, 9, 50, 59, 240, 249, 290, 299]                 # tile grid 5 x 6 x 10
    qrows = []
    for h in range(H):
        for t in corners + [int(g.integers(0, 300))]:
            qrows += _tile_rows(inv, h, N, L, t, g.choice(L, 2, replace=False))
    krows = []
    for h in (3, 17):
        for t in (0, 144):
            krows += _tile_rows(inv, h, N, L, t, range(L))
    _check_rows(w, dq, dk, dv, qrows, krows, "720p-train")
    _identities(dq, dk, dv, w["dout"], "720p-train")


def test_bwd_720p_training_seeded_key_tiles():
    """The same training backward: dK/dV on four more whole key tiles, seeded
    (with the two of the test above, six key tiles in each of heads 3 and
    17), and dQ on the rows of one seeded tile per head."""
    w, dq, dk, dv, inv = _train_720p()
    B, H, N, D = w["q"].shape
    L = 384
    g = np.random.default_rng(58)
    ktiles = [int(t) for t in g.choice([t for t in range(300) if t not in (0, 144)], 4, replace=False)]
    qrows, krows = [], []
    for h in range(H):
        qrows += _tile_rows(inv, h, N, L, int(g.integers(0, 300)), g.choice(L, 2, replace=False))
    for h in (3, 17):
        for t in ktiles:
            krows += _tile_rows(inv, h, N, L, t, range(L))
    _check_rows(w, dq, dk, dv, qrows, krows, "720p-train seeded key tiles %s" % ktiles)


def test_bwd_mid_7680():
    """The mid workload (7680 tokens, 24 heads, D 128, tile (4,8,8), window
    3x3x3 on a 2x3x5 tile grid): heads 0 and 1 in full, and in every head
    dQ rows of two seeded tiles and dK/dV rows of one seeded key tile.  Plus
    the whole-tensor identities."""
    w = workload("mid-7680", with_dout=True)
    say("bwd bf16 mid-7680 workload")
    dq, dk, dv = _run(w)
    B, H, N, D = w["q"].shape
    sl = lambda x: x[:, :2]
    rq, rk, rv = oracle.bwd(sl(w["q"]), sl(w["k"]), sl(w["v"]), sl(w["dout"]), w["grid"], w["tile"],
                            w["windows"][:2])
    for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_close(to_host(got[:, :2]), ref, "bf16", "mid-7680 heads 0-1 " + nm)
    L = 256
    inv = np.argsort(oracle.perm(w["grid"], w["tile"]))
    g = np.random.default_rng(56)
    qrows, krows = [], []
    for h in range(H):
        for t in g.choice(30, 2, replace=False):
            qrows += _tile_rows(inv, h, N, L, int(t), g.choice(L, 4, replace=False))
        krows += _tile_rows(inv, h, N, L, int(g.integers(0, 30)), g.choice(L, 8, replace=False))
    _check_rows(w, dq, dk, dv, qrows, krows, "mid-7680")
    _identities(dq, dk, dv, w["dout"], "mid-7680")


def test_bwd_720p_shifted_perhead():
    """The shifted, per-head-window workload at full size (115200 tokens, 24
    heads with windows 3x3x3, 3x3x5 or 5x5x5 tiles, a seeded shift per query
    tile) through the backward: dQ rows of corner and seeded tiles in three
    heads of every window class; dK/dV on whole key tiles: the least and the
    most attended under the shifts for a 3x3x3 head (6 and 85 query tiles),
    the least attended for a 3x3x5 head (9) and a 5x5x5 head (41).  (The
    oracle forms the statistics of every query row attending a key tile:
    the most attended tiles of the wider windows, 141 and 211 query tiles,
    would take it minutes; the training test covers a 140-attendee tile.)
    Plus the whole-tensor identities."""
    w = workload("720p-shifted-perhead", with_dout=True)
    say("bwd bf16 720p-shifted-perhead workload (full size)")
    off = w["offsets"]
    dq, dk, dv = _run(w, off)
    B, H, N, D = w["q"].shape
    L = 384
    inv = np.argsort(oracle.perm(w["grid"], w["tile"]))
    _, _, _, q_cnt = oracle.index(w["grid"], w["tile"], w["windows"], off)
    classes = {}
    for h in range(H):
        classes.setdefault(tuple(int(x) for x in w["windows"][h]), []).append(h)
    assert sorted(classes) == [(3, 3, 3), (3, 3, 5), (5, 5, 5)]
    g = np.random.default_rng(57)
    qrows = []
    for cls, heads in sorted(classes.items()):
        for h in heads[:3]:
            for t in (0, 59, 240, 299, int(g.integers(0, 300))):
                qrows += _tile_rows(inv, h, N, L, t, g.choice(L, 2, replace=False))
    krows = []
    for cls, which in (((3, 3, 3), ("min", "max")), ((3, 3, 5), ("min",)), ((5, 5, 5), ("min",))):
        h = classes[cls][0]
        for kind in which:
            t = int(np.argmin(q_cnt[h]) if kind == "min" else np.argmax(q_cnt[h]))
            say("  head %d %s: key tile %d attended by %d query tiles" % (h, cls, t, q_cnt[h][t]))
            krows += _tile_rows(inv, h, N, L, t, range(L))
    _check_rows(w, dq, dk, dv, qrows, krows, "720p-shifted-perhead", off)
    _identities(dq, dk, dv, w["dout"], "720p-shifted-perhead")


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


def test_bwd_stages_called_separately():
    """The backward stages as separate calls (Delta, then dK/dV and dQ in
    either order, and dK/dV alone after a Delta call) give the same bits as
    one call of all stages: dK/dV reads Delta from delta_ws through its
    per-row pre-pass (-lse log2 e, -Delta), and each call takes and returns
    its own workspace."""
    import sliding_tile_attention_amd as sta
    from tests.gpu_util import to_dev

    grid, tile, D = (12, 16, 24), (6, 8, 8), 128
    windows = [(3, 3, 3), (1, 3, 3), (3, 3, 5)]
    say("bwd stages called separately " + str(grid))
    geom = sta.Geometry(grid, tile)
    idx = sta.StaIndex(geom, windows)
    N = geom.tokens
    q, k, v, do = (to_dev(x, "bf16") for x in tensors(1, len(windows), N, D, "bf16", 97, with_dout=True))
    o, lse = sta.forward(q, k, v, geom, idx)
    stream = torch.cuda.current_stream()

    def run(stages):
        dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
        delta = torch.full_like(lse, float("nan"))
        for p in stages:
            sta.sta_bwd_ex(q, k, v, o, lse, do, dq, dk, dv, delta, 1, len(windows), D, sta.STA_BF16, D ** -0.5,
                           geom, idx, p, 0, stream, sta.STA_LAYOUT_TILE)
        torch.cuda.synchronize()
        return dq, dk, dv

    ref = run([sta.STA_BWD_ALL])
    for stages in ([sta.STA_BWD_DELTA, sta.STA_BWD_DKDV, sta.STA_BWD_DQ],
                   [sta.STA_BWD_DELTA, sta.STA_BWD_DQ, sta.STA_BWD_DKDV],
                   [sta.STA_BWD_DELTA | sta.STA_BWD_DQ, sta.STA_BWD_DKDV]):
        got = run(stages)
        for a, b, nm in zip(got, ref, ("dQ", "dK", "dV")):
            assert torch.equal(a, b), "%s differs for stages %s" % (nm, stages)
    assert all(torch.isfinite(t.float()).all() for t in ref)
