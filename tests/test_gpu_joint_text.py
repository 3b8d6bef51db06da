"""GPU parity of joint text + video attention (token-type-aware masking,
MOD-DiT README, "Token-Type-Aware Masking"): n_text text tokens follow the
video tokens; libsta (reorder with text rows in place -> index -> forward /
backward) against the CPU oracle on identical seeded inputs."""
import numpy as np
import pytest
import torch

import sliding_tile_attention_amd as sta
from oracle import oracle
from tests.gpu_util import Layer, assert_close, assert_lse, say, to_dev, to_host
from tests.inputs import TEXT_TOKENS_720P, tensors, workload

pytestmark = pytest.mark.gpu

CASES = [
    # name, grid, tile, B, H, D, windows, n_text, border, offsets kind (None / "shared" / "head")
    ("L32-D128-t1", (4, 8, 12), (2, 4, 4), 1, 2, 128, [(3, 3, 3), (1, 3, 3)], 1, "shift", None),
    ("L48-D64-t77", (6, 8, 16), (3, 4, 4), 2, 2, 64, [(1, 3, 3), (3, 3, 5)], 77, "shift", "shared"),
    ("L128-D128-t128", (4, 16, 24), (2, 8, 8), 1, 2, 128, [(3, 3, 3), (1, 1, 1)], 128, "shift", None),
    ("L384-D128-t256", (12, 16, 24), (6, 8, 8), 1, 2, 128, [(3, 3, 3), (1, 3, 3)], 256, "shift", None),
    ("L384-D128-t500-trunc-head", (12, 16, 24), (6, 8, 8), 1, 2, 128, [(3, 3, 5), (1, 3, 3)], 500, "truncate",
     "head"),
    ("L16-D64-t40", (2, 4, 8), (1, 4, 4), 1, 2, 64, [(1, 1, 1), (3, 3, 3)], 40, "shift", None),
    ("L256-D64-t300", (8, 16, 24), (4, 8, 8), 1, 1, 64, [(1, 3, 3)], 300, "shift", None),
]


def _offsets(kind, H, T, seed=9):
    if kind is None:
        return None
    shape = (T, 3) if kind == "shared" else (H, T, 3)
    return np.random.default_rng(seed).integers([-1, -2, -2], [1, 2, 2], endpoint=True,
                                                size=shape).astype(np.int32)


def _setup(case, dtype, seed):
    name, grid, tile, B, H, D, windows, nt, border, kind = case
    T = int(np.prod([a // b for a, b in zip(grid, tile)]))
    off = _offsets(kind, H, T)
    S = int(np.prod(grid)) + nt
    q, k, v, do = tensors(B, H, S, D, dtype, seed, with_dout=True)
    layer = Layer(grid, tile, windows, off, q, k, v, dtype, dout=do, border=border, n_text=nt)
    return layer, off, (q, k, v, do)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_joint_bf16_forward_backward(case):
    name, grid, tile, B, H, D, windows, nt, border, kind = case
    say("joint bf16 " + name)
    layer, off, (q, k, v, do) = _setup(case, "bf16", 130)
    o, lse = layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, off, border=border, n_text=nt)
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, off, border=border, n_text=nt)
    assert_close(to_host(o), ro, "bf16", name + " O")
    assert_lse(to_host(lse), rl, "bf16")
    for got, ref, nm in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_close(to_host(got), ref, "bf16", name + " " + nm)


@pytest.mark.parametrize("case", [CASES[1], CASES[5]], ids=lambda c: c[0])
def test_joint_f32_forward_backward(case):
    name, grid, tile, B, H, D, windows, nt, border, kind = case
    say("joint f32 " + name)
    layer, off, (q, k, v, do) = _setup(case, "f32", 131)
    o, lse = layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, off, border=border, n_text=nt)
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, off, border=border, n_text=nt)
    for got, ref, nm in ((o, ro, "O"), (lse, rl, "LSE"), (dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_close(to_host(got), ref, "f32", name + " " + nm)


def test_joint_reorder_keeps_text_rows():
    """Reorder with text rows: the video rows are permuted exactly as the
    oracle's permutation says, the text rows are copied in place, and the
    inverse restores the input bit for bit."""
    grid, tile, nt = (4, 8, 12), (2, 4, 4), 37
    N = int(np.prod(grid))
    say("joint reorder")
    x = torch.randint(-2 ** 31, 2 ** 31 - 1, (3, N + nt, 5), dtype=torch.int32)
    geom = sta.Geometry(grid, tile)
    y = sta.tile_reorder(x.cuda(), geom, n_text=nt)
    z = sta.tile_reorder(y, geom, inverse=True, n_text=nt)
    torch.cuda.synchronize()
    p = oracle.perm(grid, tile)                    # raster token -> tile-order slot
    want = np.empty((3, N + nt, 5), np.int32)
    want[:, p] = x.numpy()[:, :N]
    want[:, N:] = x.numpy()[:, N:]
    assert np.array_equal(y.cpu().numpy(), want)
    assert torch.equal(z.cpu(), x)


def test_joint_zero_text_matches_plain_calls():
    """n_text = 0 through the options calls is bit-identical to the plain calls."""
    grid, tile, windows = (4, 8, 12), (2, 4, 4), [(3, 3, 3), (1, 3, 5)]
    B, H, D = 1, 2, 128
    say("joint n_text=0")
    q, k, v, do = (to_dev(x, "bf16") for x in tensors(B, H, int(np.prod(grid)), D, "bf16", 132, with_dout=True))
    geom = sta.Geometry(grid, tile)
    idx = sta.StaIndex(geom, windows)
    o0, l0 = torch.empty_like(q), torch.empty((B, H, q.shape[2]), dtype=torch.float32, device="cuda")
    sta.sta_fwd(q, k, v, o0, l0, B, H, D, sta.STA_BF16, D ** -0.5, geom, idx)
    o1, l1 = sta.forward(q, k, v, geom, idx, n_text=0)
    g0 = [torch.empty_like(q) for _ in range(3)]
    sta.sta_bwd(q, k, v, o0, l0, do, *g0, torch.empty_like(l0), B, H, D, sta.STA_BF16, D ** -0.5, geom, idx)
    g1 = sta.backward(q, k, v, o1, l1, do, geom, idx, n_text=0)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    for a, b in zip(g0, g1):
        assert torch.equal(a, b)


def test_joint_720p_sampled():
    """Full 115200-token grid with 1164 text tokens (about 1% of the joint
    sequence), 24 heads, window 3x3x5: forward and backward run whole on the
    GPU; sampled video rows (corner and random tiles) and text rows (the
    longest walks, over every key) of O, LSE and dQ, and dK/dV rows of the
    least attended key tile, are checked against the oracle.  Text keys (which
    every query attends: the oracle would need every row's statistics) are
    checked exactly by the small cases and here by the whole-tensor
    identities sum_j dV_j = sum_i dO_i and sum_j dK_j = 0, which include
    them."""
    nt = TEXT_TOKENS_720P
    w = workload("720p-train", n_text=nt)
    say("joint bf16 720p + %d text (full size)" % nt)
    layer = Layer(w["grid"], w["tile"], w["windows"], None, w["q"], w["k"], w["v"], "bf16", dout=w["dout"],
                  n_text=nt)
    o, lse = layer.forward()
    dq, dk, dv = layer.backward()
    torch.cuda.synchronize()
    B, H, S, D = w["q"].shape
    N, L = S - nt, 384
    inv = np.argsort(oracle.perm(w["grid"], w["tile"]))          # tile-order slot -> raster token
    g = np.random.default_rng(57)
    qrows = []
    for h in (0, 13, 23):
        for t in (0, 299, int(g.integers(0, 300))):
            qrows += [h * S + int(inv[t * L + s]) for s in g.choice(L, 3, replace=False)]
        qrows += [h * S + N + int(s) for s in (0, nt - 1, *g.choice(nt, 3, replace=False))]
    krows = [5 * S + int(inv[s]) for s in g.choice(L, 3, replace=False)]        # key tile 0
    qrows, krows = np.array(qrows, np.int64), np.array(krows, np.int64)
    say("oracle: %d query rows, %d key rows" % (len(qrows), len(krows)))
    ro, rl = oracle.fwd(w["q"], w["k"], w["v"], w["grid"], w["tile"], w["windows"], rows=qrows, n_text=nt)
    rq, rk, rv = oracle.bwd(w["q"], w["k"], w["v"], w["dout"], w["grid"], w["tile"], w["windows"],
                            qrows=qrows, krows=krows, n_text=nt)
    pick = lambda t, rows: to_host(t.reshape(-1, D)[torch.from_numpy(rows).cuda()])
    assert_close(pick(o, qrows), ro, "bf16", "O")
    assert_lse(to_host(lse.reshape(-1)[torch.from_numpy(qrows).cuda()]), rl, "bf16")
    assert_close(pick(dq, qrows), rq, "bf16", "dQ")
    assert_close(pick(dk, krows), rk, "bf16", "dK")
    assert_close(pick(dv, krows), rv, "bf16", "dV")
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t).all()
    # Rows of P sum to 1 and rows of dS to 0 over every key, text included
    # (gates as in the video-only training check).
    sdv, sdo = dv.float().sum(2), torch.from_numpy(w["dout"]).cuda().sum(2)
    rel = (torch.linalg.norm(sdv - sdo) / torch.linalg.norm(sdo)).item()
    assert rel < 1e-3, "sum dV vs sum dO: rel %.2e" % rel
    sdk = dk.float().sum(2)
    scale_k = torch.sqrt((dk.float() ** 2).sum(2) * S).clamp_min(1e-30)
    assert (sdk.abs() / scale_k).max().item() < 1e-2
