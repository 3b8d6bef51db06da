"""sliding_tile_attention_amd.attention: the forward and backward calls as one
differentiable operation.  Its output and the gradients autograd returns are
bit-identical to forward() and backward() called directly, and match the
oracle."""
import numpy as np
import pytest
import torch

import sliding_tile_attention_amd as sta
from oracle import oracle
from tests.gpu_util import assert_close, say
from tests.inputs import tensors

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,n_text,shifts", [("bf16", 0, False), ("bf16", 40, True), ("f32", 7, True)])
def test_attention_autograd_matches_calls_and_oracle(dtype, n_text, shifts):
    grid, tile, B, H, D = (4, 8, 12), (2, 4, 4), 1, 2, 64
    windows = [(3, 3, 3), (1, 3, 5)]
    say("autograd %s text %d shifts %s" % (dtype, n_text, shifts))
    geom = sta.Geometry(grid, tile)
    T = geom.num_tiles
    off = np.random.default_rng(9).integers(-1, 2, size=(T, 3)).astype(np.int32) if shifts else None
    idx = sta.StaIndex(geom, windows, None if off is None else torch.from_numpy(off).cuda())
    N = geom.tokens + n_text
    q, k, v, do = tensors(B, H, N, D, dtype, 4100, with_dout=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda x: sta.tile_reorder(torch.from_numpy(x).to("cuda", tdt), geom, n_text=n_text)
    qt, kt, vt, dot = dev(q), dev(k), dev(v), dev(do)
    leaves = [x.clone().requires_grad_(True) for x in (qt, kt, vt)]
    o = sta.attention(*leaves, geom, idx, n_text=n_text)
    o.backward(dot)
    torch.cuda.synchronize()
    o2, lse2 = sta.forward(qt, kt, vt, geom, idx, n_text=n_text)
    dq2, dk2, dv2 = sta.backward(qt, kt, vt, o2, lse2, dot, geom, idx, n_text=n_text)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for leaf, ref in zip(leaves, (dq2, dk2, dv2)):
        assert torch.equal(leaf.grad, ref)
    host = lambda t: sta.tile_reorder(t.detach(), geom, inverse=True, n_text=n_text).float().cpu().numpy()
    ro, _ = oracle.fwd(q, k, v, grid, tile, windows, off, n_text=n_text)
    rq, rk, rv = oracle.bwd(q, k, v, do, grid, tile, windows, off, n_text=n_text)
    assert_close(host(o), ro, dtype, "O")
    for leaf, ref, nm in zip(leaves, (rq, rk, rv), ("dQ", "dK", "dV")):
        assert_close(host(leaf.grad), ref, dtype, nm)
