"""GPU parity of the quantized forward (INT8 QK^T, FP8 PV): libsta against
the oracle of the quantized method (oracle/quant.py) on identical seeded
inputs.  The oracle decides every code from exact values; the kernel forms
the logits in fp32, so the comparison allows, element by element, exactly
what a code rounded to its neighbour can change (the oracle's bound), plus
the bf16 rounding of the output and fp32 accumulation (tests/gpu_util.py,
assert_fp8).  Also the accuracy of the method against exact attention at
full size.  The scheme reads the pages' quantized-attention dependency
(MOD-DiT README, "Project Structure" and "Acknowledgements")."""
import numpy as np
import pytest
import torch

from oracle import oracle, quant
from tests.gpu_util import Layer, assert_fp8, errors, say, to_host
from tests.inputs import tensors, workload

pytestmark = pytest.mark.gpu

CASES = [
    # name, grid, tile, B, H, D, windows, offsets kind, border, n_text
    ("L384-D128", (12, 16, 24), (6, 8, 8), 1, 2, 128, [(3, 3, 3), (1, 3, 3)], None, "shift", 0),
    ("L128-D128-offsets", (4, 16, 24), (2, 8, 8), 2, 2, 128, [(3, 3, 3), (1, 1, 3)], "shared", "shift", 0),
    ("L32-D64-partial-blocks", (4, 8, 12), (2, 4, 4), 1, 3, 64, [(3, 3, 3), (1, 3, 3), (5, 5, 5)], "head",
     "truncate", 0),
    ("L384-D128-text-cut", (12, 13, 16), (6, 8, 8), 1, 2, 128, [(3, 3, 3), (1, 1, 3)], None, "shift", 77),
    ("L48-D64-text", (6, 8, 16), (3, 4, 4), 1, 2, 64, [(1, 3, 3), (3, 3, 5)], "head", "shift", 100),
    # cut tiles of 384, 240, 192 and 120 tokens (partial 64-key blocks) under truncated, per-head shifted windows
    ("L384-D128-cut-truncate-head", (12, 13, 20), (6, 8, 8), 1, 2, 128, [(3, 3, 5), (1, 3, 3)], "head",
     "truncate", 0),
]


def _offsets(kind, H, T, seed=13):
    if kind is None:
        return None
    shape = (T, 3) if kind == "shared" else (H, T, 3)
    return np.random.default_rng(seed).integers([-1, -2, -2], [1, 2, 2], endpoint=True,
                                                size=shape).astype(np.int32)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_fp8_forward_matches_quantized_oracle(case):
    name, grid, tile, B, H, D, windows, kind, border, nt = case
    say("fp8 fwd " + name)
    T = int(np.prod(oracle.tiles_per_axis(grid, tile)))
    off = _offsets(kind, H, T)
    S = int(np.prod(grid)) + nt
    q, k, v = tensors(B, H, S, D, "bf16", 190)
    layer = Layer(grid, tile, windows, off, q, k, v, "bf16", border=border, n_text=nt)
    o, lse = layer.forward(precision="fp8")
    torch.cuda.synchronize()
    ref = quant.fwd(q, k, v, grid, tile, windows, off, border=border, n_text=nt, bound=True)
    assert_fp8(to_host(o), to_host(lse), ref, name)


def test_fp8_zero_query_rows_and_constant_keys_on_partial_blocks():
    """Scale factors of zero: query rows of zeros (row scale 0) and a head
    whose keys are all equal (every smoothed key 0, every K block scale 0),
    on tiles of 32 keys, so every 64-key block is partial and has masked
    keys.  Such rows attend uniformly over their window; the outputs are
    finite and match the oracle."""
    grid, tile, H, D = (4, 8, 12), (2, 4, 4), 2, 64
    windows = [(3, 3, 3), (1, 3, 3)]
    N = int(np.prod(grid))
    say("fp8 fwd zero rows / constant keys")
    q, k, v = tensors(1, H, N, D, "bf16", 194)
    q[0, :, [0, 37, 200, 383], :] = 0.0
    k[0, 1] = k[0, 1, 7].copy()
    layer = Layer(grid, tile, windows, None, q, k, v, "bf16")
    o, lse = layer.forward(precision="fp8")
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    ref = quant.fwd(q, k, v, grid, tile, windows, bound=True)
    assert_fp8(to_host(o), to_host(lse), ref, "zero rows / constant keys")


def test_fp8_forward_deterministic_and_repeatable():
    """Two calls (and a call after a call of another shape) give identical
    bits: the statistics pass reduces in a fixed order, no atomics."""
    grid, tile, windows = (12, 16, 24), (6, 8, 8), [(3, 3, 3)]
    q, k, v = tensors(1, 1, int(np.prod(grid)), 128, "bf16", 191)
    layer = Layer(grid, tile, windows, None, q, k, v, "bf16")
    o1, l1 = (x.clone() for x in layer.forward(precision="fp8"))
    other = Layer((4, 8, 12), (2, 4, 4), [(3, 3, 3)], None, *tensors(1, 1, 384, 128, "bf16", 192), "bf16")
    other.forward(precision="fp8")
    o2, l2 = layer.forward(precision="fp8")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_720p_sampled_and_method_accuracy():
    """The 720p forward (115200 tokens, 24 heads, window 3x3x5) in the FP8
    path: sampled rows against the quantized method's oracle (its bound),
    and against exact attention, whose error is the method's own (relative
    L2 below 8e-2: e4m3 P and V each carry a rounding of relative RMS about
    2^-4/sqrt(3))."""
    w = workload("720p")
    say("fp8 fwd 720p (full size)")
    layer = Layer(w["grid"], w["tile"], w["windows"], None, w["q"], w["k"], w["v"], "bf16")
    o, lse = layer.forward(precision="fp8")
    torch.cuda.synchronize()
    B, H, N, D = w["q"].shape
    inv = np.argsort(oracle.perm(w["grid"], w["tile"]))
    g = np.random.default_rng(193)
    rows = []
    for h in (0, 11, 23):
        for t in (0, 299, 144, int(g.integers(0, 300))):
            rows += [h * N + int(inv[t * 384 + s]) for s in g.choice(384, 4, replace=False)]
    rows = np.array(rows, np.int64)
    say("quantized oracle on %d rows" % len(rows))
    ref = quant.fwd(w["q"], w["k"], w["v"], w["grid"], w["tile"], w["windows"], rows=rows, bound=True)
    pick = lambda x: to_host(x.reshape(-1, D)[torch.from_numpy(rows).cuda()])
    got = pick(o)
    assert_fp8(got, to_host(lse.reshape(-1)[torch.from_numpy(rows).cuda()]), ref, "720p sampled")
    eo, _ = oracle.fwd(w["q"], w["k"], w["v"], w["grid"], w["tile"], w["windows"], rows=rows)
    max_abs, rel = errors(got, eo)
    say("fp8 vs exact attention: max-abs %.3e rel-L2 %.3e" % (max_abs, rel))
    assert rel < 8e-2
    assert torch.isfinite(layer.o).all()
