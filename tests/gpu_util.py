"""Helpers for the GPU parity tests: device copies of the seeded inputs, the
layer-level path through libsta (raster -> tile order -> kernels -> raster),
and the numeric gates."""
import sys

import numpy as np
import torch

import sliding_tile_attention_amd as sta

# Gates for bf16 outputs and gradients: max-abs error and relative L2 error.
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
# fp32 path: both sides compute in >= fp32 from the same fp32 inputs.
F32_MAX_ABS = 1e-4
# LSE of the bf16 path: the kernel sums the probabilities after rounding
# them to bf16 (the same values the PV product uses).  A sum of positive
# terms each carrying relative error <= 2^-9 has relative error <= 2^-9, so
# |dLSE| <= ln(1 + 2^-9) = 1.95e-3; 2.5e-3 leaves room for fp32 rounding.
BF16_LSE_MAX_ABS = 2.5e-3


def say(msg):
    """A progress line on the process's own stderr (not captured by pytest),
    so that a long oracle check shows what it is doing while it runs."""
    sys.__stderr__.write("[gpu] " + msg + "\n")
    sys.__stderr__.flush()


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def to_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    max_abs = float(np.max(np.abs(got - ref))) if got.size else 0.0
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)) if got.size else 0.0
    return max_abs, rel_l2


def assert_lse(got, ref, dtype, what="LSE"):
    err = float(np.max(np.abs(np.asarray(got, np.float64) - ref))) if np.size(ref) else 0.0
    gate = BF16_LSE_MAX_ABS if dtype == "bf16" else F32_MAX_ABS
    assert err <= gate, "%s: max-abs %.3e (gate %.1e)" % (what, err, gate)
    return err


def assert_close(got, ref, dtype, what=""):
    max_abs, rel_l2 = errors(got, ref)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    if dtype == "bf16":
        assert max_abs <= BF16_MAX_ABS and rel_l2 <= BF16_REL_L2, \
            "%s: max-abs %.3e (gate %.0e), rel-L2 %.3e (gate %.0e)" % (what, max_abs, BF16_MAX_ABS, rel_l2,
                                                                       BF16_REL_L2)
    else:
        assert max_abs <= F32_MAX_ABS, "%s: max-abs %.3e (gate %.0e)" % (what, max_abs, F32_MAX_ABS)
    return max_abs, rel_l2


def assert_fp8(got_o, got_lse, ref, what=""):
    """The quantized forward against its oracle, run with bound=True
    (oracle/quant.py): element by element,
        |O - O_ref| <= bound + 2^-8 |O_ref| + 1e-4 a + 1e-7,
        |LSE - LSE_ref| <= bound + 1e-5 (1 + |LSE_ref|),
    where the bounds cover the codes of P that a fp32 evaluation of the
    logits may round the other way, 2^-8 |O| the bf16 rounding of the output
    (2^-9) with room, and a = sum_j p_j |w_j| / l the scale of the fp32
    accumulation error (about sqrt(n) 2^-24 of it over n <= 5e4 keys, 1.3e-5).
    Returns (rows whose bound is nonzero, max |dO|)."""
    ro, rl, ob, lb, oa = (np.asarray(x, np.float64) for x in ref)
    o = np.asarray(got_o, np.float64).reshape(ro.shape)
    lse = np.asarray(got_lse, np.float64).reshape(rl.shape)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what + ": non-finite output"
    tol = ob + 2.0 ** -8 * np.abs(ro) + 1e-4 * oa + 1e-7
    err = np.abs(o - ro)
    bad = err > tol
    assert not bad.any(), "%s: %d of %d elements of O outside the bound (worst |dO| %.3e against %.3e)" % (
        what, bad.sum(), bad.size, err[bad].max(), tol[bad][np.argmax(err[bad])])
    lerr = np.abs(lse - rl)
    lbad = lerr > lb + 1e-5 * (1 + np.abs(rl))
    assert not lbad.any(), "%s: %d LSE values outside the bound (worst %.3e)" % (what, lbad.sum(), lerr.max())
    flagged = int(np.count_nonzero(lb.reshape(-1) > 0))
    say("%s: max |dO| %.3e, max |dLSE| %.3e, %d rows with codes a fp32 evaluation may move" % (
        what, float(err.max()) if err.size else 0.0, float(lerr.max()) if lerr.size else 0.0, flagged))
    return flagged, float(err.max()) if err.size else 0.0


class Layer:
    """Device state of one attention layer: inputs reordered to tile order,
    the index, and the outputs converted back to raster order.  With n_text
    > 0 the token axis holds the grid's tokens and then n_text text tokens,
    which stay in place."""

    def __init__(self, grid, tile, windows, offsets, q, k, v, dtype, dout=None, transposed=True, border="shift",
                 n_text=0):
        self.geom = sta.Geometry(tuple(grid), tuple(tile))
        self.dtype = dtype
        self.n_text = n_text
        self.B, self.H, self.N, self.D = q.shape
        self.windows = [tuple(int(x) for x in w) for w in windows]
        self.off_dev = None if offsets is None else torch.from_numpy(np.ascontiguousarray(offsets, np.int32)).cuda()
        self.index = sta.StaIndex(self.geom, self.windows, self.off_dev, transposed=transposed, border=border)
        self.q, self.k, self.v = (self._tiled(to_dev(x, dtype)) for x in (q, k, v))
        self.dout = None if dout is None else self._tiled(to_dev(dout, dtype))

    def _tiled(self, x):
        return sta.tile_reorder(x, self.geom, n_text=self.n_text)

    def _raster(self, x):
        return sta.tile_reorder(x, self.geom, inverse=True, n_text=self.n_text)

    def forward(self, scale=None, precision="default"):
        self.o, self.lse = sta.forward(self.q, self.k, self.v, self.geom, self.index, scale, n_text=self.n_text,
                                       precision=precision)
        return self._raster(self.o), self._raster(self.lse.unsqueeze(-1)).squeeze(-1)

    def backward(self, scale=None):
        dq, dk, dv = sta.backward(self.q, self.k, self.v, self.o, self.lse, self.dout, self.geom, self.index,
                                  scale, n_text=self.n_text)
        return tuple(self._raster(x) for x in (dq, dk, dv))


def sample_rows(B, H, N, L, grid, tile, per_head_tiles, rows_per_tile, seed):
    """Flat row ids (b*H + h)*N + raster_i covering the corner tiles and a few
    seeded random tiles of every head."""
    from oracle import oracle   # test infrastructure: only the parity checks use it
    g = np.random.default_rng(seed)
    n = [a // b for a, b in zip(grid, tile)]
    T = int(np.prod(n))
    corners = sorted({(a * n[1] + b) * n[2] + c for a in (0, n[0] - 1) for b in (0, n[1] - 1)
                      for c in (0, n[2] - 1)})
    inv = np.argsort(oracle.perm(grid, tile))   # tile-order slot -> raster token
    rows = []
    for b in range(B):
        for h in range(H):
            tiles = list(corners) + list(g.integers(0, T, size=per_head_tiles))
            for t in tiles:
                slots = g.choice(L, size=min(rows_per_tile, L), replace=False)
                rows.extend(((b * H + h) * N + inv[t * L + slots]).tolist())
    return np.unique(np.asarray(rows, np.int64))
