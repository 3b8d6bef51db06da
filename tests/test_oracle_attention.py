"""Pins of the oracle's forward and backward (CPU only).

The pages give no numeric example of STA.  What they fix is the operator:
softmax attention restricted to the local window ("Fast Video Generation
with Sliding Tile Attention", abstract), which must reduce to 3D full
attention when the window covers the whole grid.  The pins are therefore:
library attention (torch SDPA / autograd, float64) under an independently
built mask, closed forms, finite differences, and exact identities.
"""
import numpy as np
import pytest
import torch

from oracle import oracle, dense_ref
from tests.inputs import CONFIGS, tensors, windows_for


def _small_case(seed, grid=(4, 4, 6), tile=(2, 2, 2), H=3, D=16, offsets=True):
    g = np.random.default_rng(seed)
    n = oracle.tiles_per_axis(grid, tile)
    T = int(np.prod(n))
    windows = g.integers(1, 4, size=(H, 3)).astype(np.int32)
    off = g.integers(-2, 3, size=(T, 3)).astype(np.int32) if offsets else None
    N = int(np.prod(grid))
    q, k, v, do = tensors(2, H, N, D, "f32", seed, with_dout=True)
    return grid, tile, windows, off, q, k, v, do


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("offsets", [False, True])
def test_forward_backward_match_torch_dense(seed, offsets):
    grid, tile, windows, off, q, k, v, do = _small_case(seed, offsets=offsets)
    o_ref, lse_ref, dq_ref, dk_ref, dv_ref = dense_ref.attention(q, k, v, grid, tile, windows, off, dout=do)
    o, lse = oracle.fwd(q, k, v, grid, tile, windows, off)
    dq, dk, dv = oracle.bwd(q, k, v, do, grid, tile, windows, off)
    for a, b in ((o, o_ref), (lse, lse_ref), (dq, dq_ref), (dk, dk_ref), (dv, dv_ref)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)


def test_whole_grid_window_is_full_attention():
    """Tiny fp32 workload: window (3,3,3) over a 2x2x2 tile grid = 3D full attention."""
    c = CONFIGS["tiny-fp32"]
    N = int(np.prod(c["grid"]))
    q, k, v, do = tensors(c["B"], c["H"], N, c["D"], "f32", 1235, with_dout=True)
    o, lse = oracle.fwd(q, k, v, c["grid"], c["tile"], windows_for("tiny-fp32"))
    dq, dk, dv = oracle.bwd(q, k, v, do, c["grid"], c["tile"], windows_for("tiny-fp32"))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    to.backward(torch.tensor(do, dtype=torch.float64))
    tl = torch.logsumexp(torch.matmul(tq, tk.transpose(-1, -2)) / np.sqrt(c["D"]), dim=-1)
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, tl.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_unit_window_is_per_tile_attention():
    """Window (1,1,1): each tile attends only to itself (block-diagonal)."""
    grid, tile = (4, 4, 4), (2, 2, 2)
    N, L = 64, 8
    q, k, v = tensors(1, 1, N, 8, "f32", 5)
    o, lse = oracle.fwd(q, k, v, grid, tile, [(1, 1, 1)])
    p = oracle.perm(grid, tile)
    inv = np.argsort(p)          # tile-order slot -> raster token
    for t in range(N // L):
        toks = inv[t * L:(t + 1) * L]
        tq, tk, tv = (torch.tensor(x[0, 0, toks], dtype=torch.float64) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None])[0]
        np.testing.assert_allclose(o[0, 0, toks], ref.numpy(), rtol=1e-11, atol=1e-12)


def test_constant_values_and_zero_queries():
    grid, tile = (6, 4, 10), (2, 2, 2)
    n = oracle.tiles_per_axis(grid, tile)
    N, L, D = int(np.prod(grid)), 8, 8
    w = [(3, 1, 3), (1, 3, 5)]
    q, k, v = tensors(1, 2, N, D, "f32", 11)
    o, _ = oracle.fwd(q, k, v, grid, tile, w, scale=0.7)
    np.testing.assert_allclose(oracle.fwd(q, k, np.ones_like(v), grid, tile, w)[0], 1.0, rtol=0, atol=1e-13)
    # q = 0: uniform weights -> mean of v over the window, LSE = ln(count * L)
    oz, lz = oracle.fwd(np.zeros_like(q), k, v, grid, tile, w)
    kv_idx, kv_cnt, _, _ = oracle.index(grid, tile, w)
    p = oracle.perm(grid, tile)
    tile_of = p // L
    for h in range(2):
        cnt = int(np.prod(np.minimum(w[h], n)))
        np.testing.assert_allclose(lz[0, h], np.log(cnt * L), rtol=1e-14)
        for i in range(0, N, 7):
            keys = np.isin(tile_of, kv_idx[h, tile_of[i], :cnt])
            np.testing.assert_allclose(oz[0, h, i], v[0, h, keys].astype(np.float64).mean(0), rtol=1e-12, atol=1e-13)
    assert np.all(np.isfinite(o))


def test_lse_bounds():
    """max_j s_ij <= LSE_i <= max_j s_ij + ln(#allowed keys)."""
    grid, tile, windows, off, q, k, v, _ = _small_case(4)
    _, lse = oracle.fwd(q, k, v, grid, tile, windows, off)
    B, H, N, D = q.shape
    for h in range(H):
        m = dense_ref.token_mask(grid, tile, tuple(windows[h]), off)
        for b in range(B):
            s = (q[b, h].astype(np.float64) @ k[b, h].astype(np.float64).T) / np.sqrt(D)
            s = np.where(m, s, -np.inf)
            mx = s.max(1)
            assert np.all(lse[b, h] >= mx - 1e-12)
            assert np.all(lse[b, h] <= mx + np.log(m.sum(1)) + 1e-12)


def test_backward_matches_finite_differences():
    """d/dx of f = sum(O * dO) by central differences of the oracle's own
    forward, for sampled entries of q, k and v."""
    grid, tile, windows, off, q, k, v, do = _small_case(6, grid=(2, 4, 4), tile=(1, 2, 2), H=2, D=8)
    dq, dk, dv = oracle.bwd(q, k, v, do, grid, tile, windows, off)
    g = np.random.default_rng(0)

    def f(qq, kk, vv):
        o, _ = oracle.fwd(qq, kk, vv, grid, tile, windows, off)
        return float(np.sum(o * do.astype(np.float64)))

    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(25):
            idx = tuple(int(g.integers(0, s)) for s in q.shape)
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            x0 = args[name][idx]
            plus, minus = np.float32(x0 + 1e-2), np.float32(x0 - 1e-2)
            args[name][idx] = plus
            fp = f(args["q"], args["k"], args["v"])
            args[name][idx] = minus
            fm = f(args["q"], args["k"], args["v"])
            num = (fp - fm) / (float(plus) - float(minus))
            assert abs(num - grad[idx]) <= 2e-5 * (1 + abs(grad[idx])), (name, idx, num, grad[idx])


def test_gradient_identities():
    """Rows of P sum to 1 and rows of dS sum to 0, hence per (b,h):
    sum_j dV_j = sum_i dO_i and sum_j dK_j = 0."""
    grid, tile, windows, off, q, k, v, do = _small_case(8, H=2, D=16)
    _, dk, dv = oracle.bwd(q, k, v, do, grid, tile, windows, off)
    np.testing.assert_allclose(dv.sum(2), do.astype(np.float64).sum(2), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dk.sum(2), 0.0, atol=1e-11)


def test_sampled_rows_equal_full_rows():
    grid, tile, windows, off, q, k, v, do = _small_case(9)
    B, H, N, D = q.shape
    o, lse = oracle.fwd(q, k, v, grid, tile, windows, off)
    dq, dk, dv = oracle.bwd(q, k, v, do, grid, tile, windows, off)
    rows = np.array([0, 5, N + 3, 2 * N * H - 1, H * N + 17])
    o2, l2 = oracle.fwd(q, k, v, grid, tile, windows, off, rows=rows)
    dq2, dk2, dv2 = oracle.bwd(q, k, v, do, grid, tile, windows, off, qrows=rows, krows=rows[::-1])
    flat = lambda x: x.reshape(-1, D)
    np.testing.assert_array_equal(o2, flat(o)[rows])
    np.testing.assert_array_equal(l2, lse.reshape(-1)[rows])
    np.testing.assert_array_equal(dq2, flat(dq)[rows])
    np.testing.assert_array_equal(dk2, flat(dk)[rows[::-1]])
    np.testing.assert_array_equal(dv2, flat(dv)[rows[::-1]])
