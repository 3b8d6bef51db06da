"""Brute-force dense reference for tiny problems (torch CPU, float64).

TEST INFRASTRUCTURE, NOT PRODUCT CODE; used only to pin the C oracle.

It shares no code with ``sta_oracle.c`` and reaches the same result by a
different route:

* the window of a query tile is found by ENUMERATION, not by a clamp
  formula: among every placement [s, s+c) of a c-tile window that fits the
  axis, take the one whose start is closest to the centred start
  q + o - floor(w/2) (the projection of a point onto an interval is
  unique, so there is exactly one); under the truncating border rule, the
  centre is the grid tile nearest to q + o and the window is the set of
  tiles within -floor(w/2) .. w-1-floor(w/2) of it;
* the token mask is an explicit N x N boolean matrix built from token
  coordinates;
* attention itself is a library routine (``torch.nn.functional.
  scaled_dot_product_attention`` with that mask), gradients come from
  torch autograd, and LSE from ``torch.logsumexp`` over the masked scores.

Source of the operator: "Fast Video Generation with Sliding Tile Attention"
(abstract: attention restricted to local 3D windows instead of 3D full
attention); window shifts as the stand-in for the deformable windows of
"MegaSlide-DiT ..." (abstract, 3D-DSA).
"""
import itertools

import numpy as np
import torch


def window_by_enumeration(n, w, q, o=0):
    """Start and count of the allowed tile range on one axis."""
    c = min(w, n)
    centred = q + o - w // 2
    best = None
    for s in range(0, n - c + 1):
        key = abs(s - centred)
        if best is None or key < best[0]:
            best = (key, s)
    return best[1], c


def window_truncated_by_enumeration(n, w, q, o=0):
    """Start and count under the truncating border rule, by enumeration:
    the centre is the grid tile nearest to q + o, and the window is every
    tile k of the axis with -floor(w/2) <= k - centre <= w - 1 - floor(w/2)."""
    centre = min(range(n), key=lambda c: abs(c - (q + o)))
    members = [k for k in range(n) if -(w // 2) <= k - centre <= w - 1 - w // 2]
    return members[0], len(members)


def token_mask(grid, tile, window, offsets=None, border="shift"):
    """[N, N] bool: mask[i, j] is True when key token j may be attended by
    query token i.  offsets: None or [T, 3] (one shift per query tile)."""
    T_, H_, W_ = grid
    nt = [-(-g // t) for g, t in zip(grid, tile)]                                  # border tiles may be cut
    coords = np.array(list(itertools.product(range(T_), range(H_), range(W_))))  # raster order
    tc = coords // np.array(tile)                                                  # tile coords
    tid = (tc[:, 0] * nt[1] + tc[:, 1]) * nt[2] + tc[:, 2]
    N = len(coords)
    lo = np.zeros((N, 3), np.int64)
    hi = np.zeros((N, 3), np.int64)
    for i in range(N):
        o = (0, 0, 0) if offsets is None else offsets[tid[i]]
        for d in range(3):
            rule = window_truncated_by_enumeration if border == "truncate" else window_by_enumeration
            s, c = rule(nt[d], window[d], int(tc[i, d]), int(o[d]))
            lo[i, d], hi[i, d] = s, s + c
    m = np.ones((N, N), bool)
    for d in range(3):
        m &= (tc[None, :, d] >= lo[:, None, d]) & (tc[None, :, d] < hi[:, None, d])
    return m


def joint_mask(video_mask, n_text):
    """Token-type-aware mask of a joint sequence: video tokens (in the order
    of video_mask) followed by n_text text tokens; text rows and text
    columns are fully allowed."""
    nv = video_mask.shape[0]
    m = np.ones((nv + n_text, nv + n_text), bool)
    m[:nv, :nv] = video_mask
    return m


def attention(q, k, v, grid, tile, windows, offsets=None, scale=None, dout=None, border="shift", n_text=0):
    """q,k,v: float arrays [B,H,N,D] in raster order (N = grid tokens +
    n_text, text tokens last).  offsets: None, [T, 3] (shared by heads) or
    [H, T, 3] (one set per head).  Returns float64 numpy (o, lse) and, with
    dout given, also (dq, dk, dv)."""
    q = torch.tensor(np.asarray(q), dtype=torch.float64)
    k = torch.tensor(np.asarray(k), dtype=torch.float64)
    v = torch.tensor(np.asarray(v), dtype=torch.float64)
    B, H, N, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    per_head = offsets is not None and np.asarray(offsets).ndim == 3
    masks = torch.stack([torch.from_numpy(joint_mask(token_mask(grid, tile, windows[h],
                                                                np.asarray(offsets)[h] if per_head else offsets,
                                                                border), n_text))
                         for h in range(H)])
    want_grad = dout is not None
    for t in (q, k, v):
        t.requires_grad_(want_grad)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=masks[None], scale=scale)
    scores = torch.matmul(q, k.transpose(-1, -2)) * scale
    lse = torch.logsumexp(scores.masked_fill(~masks[None], float("-inf")), dim=-1)
    if not want_grad:
        return o.detach().numpy(), lse.detach().numpy()
    o.backward(torch.tensor(np.asarray(dout), dtype=torch.float64))
    return (o.detach().numpy(), lse.detach().numpy(),
            q.grad.numpy(), k.grad.numpy(), v.grad.numpy())
