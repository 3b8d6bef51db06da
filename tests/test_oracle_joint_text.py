"""Pins of the oracle's joint text + video attention (CPU only).

Token-type-aware masking (MOD-DiT README mirror, "Token-Type-Aware
Masking"): text tokens are appended after the video tokens; every pair with
a text token on either side is attended, video-video pairs keep the sliding
tile window.  The pins: dense masked attention (torch SDPA + autograd,
float64) under an independently built mask; text rows against unmasked
library attention; video rows against the log-sum-exp merge of the
video-only oracle and unmasked attention over the text keys; a whole-grid
window against full attention; zero text tokens against the video-only
problem; and a permutation of the text tokens.
"""
import numpy as np
import pytest
import torch

from oracle import dense_ref, oracle
from tests.inputs import tensors


def _case(seed, n_text, grid=(4, 4, 6), tile=(2, 2, 2), H=2, D=8, B=1):
    g = np.random.default_rng(seed)
    N = int(np.prod(grid)) + n_text
    q, k, v, do = tensors(B, H, N, D, "f32", seed, with_dout=True)
    T = int(np.prod(oracle.tiles_per_axis(grid, tile)))
    off = g.integers(-1, 1, endpoint=True, size=(H, T, 3)).astype(np.int32)
    return grid, tile, q, k, v, do, off


def _t(x, grad=False):
    return torch.tensor(x, dtype=torch.float64, requires_grad=grad)


@pytest.mark.parametrize("border", ["shift", "truncate"])
@pytest.mark.parametrize("n_text", [1, 7])
def test_joint_matches_torch_dense(border, n_text):
    grid, tile, q, k, v, do, off = _case(40 + n_text, n_text)
    windows = [(1, 3, 3), (3, 1, 1)]
    o, lse = oracle.fwd(q, k, v, grid, tile, windows, off, border=border, n_text=n_text)
    dq, dk, dv = oracle.bwd(q, k, v, do, grid, tile, windows, off, border=border, n_text=n_text)
    ref = dense_ref.attention(q, k, v, grid, tile, windows, off, dout=do, border=border, n_text=n_text)
    for got, want in zip((o, lse, dq, dk, dv), ref):
        assert np.max(np.abs(got - want)) < 1e-10


def test_text_rows_are_unmasked_attention():
    n_text = 5
    grid, tile, q, k, v, do, _ = _case(51, n_text)
    nv = int(np.prod(grid))
    o, lse = oracle.fwd(q, k, v, grid, tile, [(1, 1, 1), (1, 1, 3)], n_text=n_text)
    tq, tk, tv = _t(q[:, :, nv:]), _t(k), _t(v)
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    wl = torch.logsumexp(torch.matmul(tq, tk.transpose(-1, -2)) / np.sqrt(q.shape[-1]), dim=-1)
    np.testing.assert_allclose(o[:, :, nv:], want.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, nv:], wl.numpy(), rtol=1e-12, atol=1e-12)


def test_video_rows_merge_window_and_text_keys():
    """A video row attends its window plus every text key; softmax over a
    union of disjoint key sets is the log-sum-exp weighted merge of the
    two partial attentions."""
    n_text = 6
    grid, tile, q, k, v, do, off = _case(52, n_text)
    nv = int(np.prod(grid))
    windows = [(1, 1, 3), (3, 3, 1)]
    o, lse = oracle.fwd(q, k, v, grid, tile, windows, off, n_text=n_text)
    ov, lv = oracle.fwd(q[:, :, :nv], k[:, :, :nv], v[:, :, :nv], grid, tile, windows, off)
    tq, tk, tv = _t(q[:, :, :nv]), _t(k[:, :, nv:]), _t(v[:, :, nv:])
    ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).numpy()
    lt = torch.logsumexp(torch.matmul(tq, tk.transpose(-1, -2)) / np.sqrt(q.shape[-1]), dim=-1).numpy()
    lm = np.logaddexp(lv, lt)
    om = np.exp(lv - lm)[..., None] * ov + np.exp(lt - lm)[..., None] * ot
    np.testing.assert_allclose(lse[:, :, :nv], lm, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o[:, :, :nv], om, rtol=1e-10, atol=1e-12)


def test_whole_grid_window_with_text_is_full_attention():
    n_text = 4
    grid, tile, q, k, v, do, _ = _case(53, n_text)
    windows = [(3, 3, 5), (3, 3, 5)]     # covers the 2x2x3 tile grid from every tile
    o, lse = oracle.fwd(q, k, v, grid, tile, windows, n_text=n_text)
    dq, dk, dv = oracle.bwd(q, k, v, do, grid, tile, windows, n_text=n_text)
    tq, tk, tv = _t(q, True), _t(k, True), _t(v, True)
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    to.backward(_t(do))
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-11, atol=1e-12)
    for got, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_zero_text_tokens_equal_video_only():
    grid, tile, q, k, v, do, off = _case(54, 0)
    windows = [(1, 3, 1), (3, 1, 3)]
    a = oracle.fwd(q, k, v, grid, tile, windows, off) + oracle.bwd(q, k, v, do, grid, tile, windows, off)
    b = (oracle.fwd(q, k, v, grid, tile, windows, off, n_text=0)
         + oracle.bwd(q, k, v, do, grid, tile, windows, off, n_text=0))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_text_permutation_equivariance():
    """Reordering the text tokens reorders the text rows of every output and
    leaves the video rows unchanged (up to summation order)."""
    n_text = 5
    grid, tile, q, k, v, do, off = _case(55, n_text)
    nv = int(np.prod(grid))
    windows = [(3, 1, 3), (1, 3, 1)]
    perm = np.concatenate([np.arange(nv), nv + np.random.default_rng(9).permutation(n_text)])
    a = oracle.fwd(q, k, v, grid, tile, windows, off, n_text=n_text) + \
        oracle.bwd(q, k, v, do, grid, tile, windows, off, n_text=n_text)
    pq, pk, pv, pd = (np.ascontiguousarray(x[:, :, perm]) for x in (q, k, v, do))
    b = oracle.fwd(pq, pk, pv, grid, tile, windows, off, n_text=n_text) + \
        oracle.bwd(pq, pk, pv, pd, grid, tile, windows, off, n_text=n_text)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x[:, :, perm], y, rtol=1e-12, atol=1e-13)
