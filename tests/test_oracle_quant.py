"""Pins of the quantized-attention oracle (oracle/quant.py; CPU only).

The quantized scheme reads the pages' quantized-attention dependency
(MOD-DiT README, "Project Structure" and "Acknowledgements": SageAttention).
Every pin is a check of a module (`check_*(mod)`), so that
tests/test_oracle_quant_mutants.py can run them against altered copies:

* e4m3 rounding against torch's float8_e4m3fn cast (a library routine) and
  hand-worked values; e4m3 commuting with powers of two in the normal range
  (what a kernel's integer running max rests on);
* int8 codes against their closed forms; the scale groups (Q per row, K per
  64-key block of a tile found from token coordinates, V per channel); the
  smoothing (keys offset by a common vector come out centred);
* P's codes, the row sum, O and LSE on rows worked by hand
  (tests/golden/quant_p_rows.txt);
* the attention steps fed with unquantized values reproduce the exact
  oracle (key sets, text keys, smoothing, LSE correction);
* the flip bound: every change a fp32 evaluation of the logits, or rounding
  at another power-of-two scale, makes to the codes is flagged, and the
  resulting change of O and LSE stays within the bound;
* the method's own error against exact attention."""
import os

import numpy as np
import pytest
import torch

from oracle import oracle, quant
from tests.inputs import tensors

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quant_p_rows.txt")


def check_e4m3_torch(mod):
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(20000) * 8, g.uniform(-448, 448, 20000), 2.0 ** g.uniform(-12, -5, 5000),
                        -(2.0 ** g.uniform(-12, 8, 5000))]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(mod.e4m3(x), want.astype(np.float64))


E4M3_HAND = [(1.0, 1.0), (1.0625, 1.0), (1.1875, 1.25), (1.1, 1.125), (17.0, 16.0), (19.0, 20.0), (448.0, 448.0),
             (2 ** -9, 2 ** -9), (2 ** -10, 0.0), (3 * 2 ** -11, 2 ** -9), (0.015625, 0.015625), (-1.0625, -1.0),
             (0.0, 0.0)]


def check_e4m3_hand(mod):
    """Spacing 2^(e-3) in the binade [2^e, 2^(e+1)), 2^-9 below 2^-6; ties to
    the even mantissa (1.0625 -> 1.0, 1.1875 -> 1.25, 17 -> 16, 19 -> 20)."""
    for x, want in E4M3_HAND:
        assert mod.e4m3(np.float32(x)) == want, (x, want)


def check_e4m3_commutes(mod):
    g = np.random.default_rng(1)
    x = 2.0 ** g.uniform(-6, 0, 50000)              # normal range, <= 1
    for k in range(0, 9):                            # 2^k x stays <= 256 < 448
        assert np.array_equal(mod.e4m3(x * 2.0 ** k), mod.e4m3(x) * 2.0 ** k)


def check_int8_closed_forms(mod):
    g = np.random.default_rng(2)
    x = (g.standard_normal((50, 64)) * g.uniform(0.1, 10, (50, 1))).astype(np.float32)
    amax = np.abs(x).max(axis=1, keepdims=True)
    c, s = mod.int8_codes(x, amax)
    assert np.all(np.abs(c).max(axis=1) == 127)
    at = np.abs(x).argmax(axis=1)
    assert np.array_equal(c[np.arange(50), at], np.sign(x[np.arange(50), at]).astype(np.int32) * 127)
    assert np.all(np.abs(x - c * s) <= s * (0.5 + 1e-5))
    z, zs = mod.int8_codes(np.zeros((2, 8), np.float32), np.zeros((2, 1), np.float32))
    assert np.all(z == 0) and np.all(zs == 0)


def _golden():
    rows, want = {}, {}
    for line in open(GOLDEN):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "=":
            want[int(f[1])] = (float(f[2]), float(f[3]))
        else:
            rows.setdefault(int(f[0]), []).append((float(f[1]), float(f[2]), float(f[3])))
    return [(np.array([r[0] for r in rows[i]]), np.array([[r[1]] for r in rows[i]]), np.array([r[2] for r in rows[i]]),
             want[i]) for i in sorted(rows)]


def check_p_rows_golden(mod):
    """P codes, O and LSE of rows worked by hand: the ceil of the row max, the
    2^4 headroom, the e4m3 rounding (normal and subnormal) and the 2^-4 back."""
    for s, w, p_want, (o_want, lse_want) in _golden():
        o, lse0, p, M, x = mod.softmax_row(s, w)
        assert np.array_equal(p, p_want), (p, p_want)
        assert abs(o[0] - o_want) < 1e-11 and abs(lse0 - lse_want) < 1e-9, (o, lse0)


def _coord_blocks(grid, tile):
    """For every raster token of a grid the tile divides: (tile id, 64-key
    block of the tile), from token coordinates (tokens of a tile in raster
    order)."""
    t, h, w = np.unravel_index(np.arange(int(np.prod(grid))), grid)
    n = [g // s for g, s in zip(grid, tile)]
    tid = ((t // tile[0]) * n[1] + h // tile[1]) * n[2] + w // tile[2]
    rank = ((t % tile[0]) * tile[1] + h % tile[1]) * tile[2] + w % tile[2]
    return tid, rank // 64


def check_k_block_scales(mod):
    """K (smoothed) is scaled per block of 64 consecutive keys of a tile: keys
    of one block share a scale, every block's largest code is 127, and a
    block of keys 10^3 times smaller gets a scale more than 10 times smaller
    (the smoothing mean, common to all keys, bounds the ratio; one scale per
    tile would give 1)."""
    grid, tile = (4, 8, 16), (2, 8, 8)                 # 4 tiles of 128 tokens: 2 blocks each
    N = int(np.prod(grid))
    tid, blk = _coord_blocks(grid, tile)
    q, k, v = tensors(1, 1, N, 16, "f32", 150)
    k = (k * np.where(blk == 0, 1e-3, 1.0)[None, None, :, None]).astype(np.float32)
    Q = mod.quantize(q, k, v, grid, tile)
    sk, kc = Q["sk"][0, 0, :, 0], Q["kc"][0, 0]
    for t in range(4):
        for b in range(2):
            sel = (tid == t) & (blk == b)
            assert np.all(sk[sel] == sk[sel][0]), (t, b)
            assert np.abs(kc[sel]).max() == 127, (t, b)
        ratio = sk[(tid == t) & (blk == 1)][0] / sk[(tid == t) & (blk == 0)][0]
        assert ratio > 10, ratio


def check_v_channel_scales(mod):
    """V is scaled per channel over all rows: every channel's largest code is
    448 and its scale is max |v_d| / 448; the codes are e4m3 values."""
    grid, tile = (4, 8, 12), (2, 4, 4)
    q, k, v = tensors(1, 2, int(np.prod(grid)), 32, "f32", 151)
    v = (v * np.logspace(-2, 2, 32)[None, None, None, :]).astype(np.float32)
    Q = mod.quantize(q, k, v, grid, tile)
    assert np.all(np.abs(Q["vc"]).max(axis=2) == 448.0)
    np.testing.assert_allclose(Q["sv"][:, :, 0, :], np.abs(v).max(axis=2) / 448.0, rtol=1e-6)
    assert np.array_equal(mod.e4m3(Q["vc"]), Q["vc"])


def check_q_row_scales(mod):
    """Q is scaled per row: every row's largest code is 127."""
    grid, tile = (4, 8, 12), (2, 4, 4)
    q, k, v = tensors(1, 2, int(np.prod(grid)), 32, "f32", 152)
    q = (q * np.logspace(-2, 2, 32)[None, None, None, :]).astype(np.float32)
    Q = mod.quantize(q, k, v, grid, tile)
    assert np.all(np.abs(Q["qc"]).max(axis=3) == 127)


def check_smoothing(mod):
    """K is smoothed by its mean over the rows: keys offset by a common vector
    (+3) dequantize to centred values (column means within half a step of 0),
    and the mean returned is the offset's."""
    grid, tile = (4, 8, 12), (2, 4, 4)
    q, k, v = tensors(1, 1, int(np.prod(grid)), 16, "f32", 153)
    k = (k + 3.0).astype(np.float32)
    Q = mod.quantize(q, k, v, grid, tile)
    deq = Q["kc"][0, 0] * Q["sk"][0, 0]
    assert np.all(np.abs(deq.mean(axis=0)) <= Q["sk"].max() * 0.5 + 1e-6)
    assert np.all(np.abs(Q["m"] - 3.0) < 0.3)


CASES = [
    # grid, tile, windows, n_text, per-head offsets
    ((4, 8, 12), (2, 4, 4), [(3, 3, 3), (1, 3, 3)], 0, False),
    ((5, 7, 9), (2, 4, 4), [(1, 3, 3), (3, 1, 3)], 23, True),
]


def check_exact_codes(mod, case):
    """Steps 5-7 fed with unquantized values (codes = the smoothed inputs,
    unit scales) and without P rounding reproduce the exact oracle: the key
    sets, the text keys, the smoothing (which leaves O unchanged) and the LSE
    correction scale * <q, m>."""
    grid, tile, windows, nt, per_head = CASES[case]
    H, D = len(windows), 16
    T = int(np.prod(oracle.tiles_per_axis(grid, tile)))
    off = np.random.default_rng(3).integers(-1, 1, endpoint=True, size=(H, T, 3)).astype(np.int32) \
        if per_head else None
    S = int(np.prod(grid)) + nt
    q, k, v = tensors(1, H, S, D, "f32", 160 + case)
    m = k.astype(np.float64).mean(axis=2, keepdims=True).astype(np.float32)
    one = np.ones(q.shape[:3] + (1,), np.float32)
    fake = dict(m=m, qc=q, sq=one, kc=k.astype(np.float64) - m, sk=one, vc=v,
                sv=np.ones((1, H, 1, D), np.float32))
    o, lse = mod.fwd(q, k, v, grid, tile, windows, off, n_text=nt, quant=fake, round_p=False)
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, off, n_text=nt)
    np.testing.assert_allclose(o, ro, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(lse, rl, rtol=1e-9, atol=1e-9)


def check_reconstruct(mod):
    grid, tile, nt = (5, 7, 9), (2, 4, 4), 23
    S = int(np.prod(grid)) + nt
    q, k, v = tensors(1, 2, S, 32, "bf16", 170)
    Q = mod.quantize(q, k, v, grid, tile, nt)
    assert np.all(np.abs(q - Q["qc"] * Q["sq"]) <= Q["sq"] * (0.5 + 1e-5))
    ks = k - Q["m"]
    assert np.all(np.abs(ks - Q["kc"] * Q["sk"]) <= Q["sk"] * (0.5 + 1e-5))
    rel_v = np.abs(v - Q["vc"] * Q["sv"]) / np.maximum(np.abs(v), 1e-30)
    assert np.all(rel_v[np.abs(v) >= Q["sv"] * 2.0 ** -6] <= 2.0 ** -4 + 1e-6)     # e4m3: half a mantissa step
    assert np.all(np.abs(Q["vc"]) <= 448)


def _midpoint_row(g, n):
    """Logits of a row in which many keys sit exactly at, or a hair off, an
    e4m3 midpoint of x = 2^(s - M + 4), plus keys in the subnormal range."""
    x = np.concatenate([2.0 ** g.uniform(-12, 4, n // 2), np.full(1, 15.9)])
    mids = []
    for e in range(-5, 4):                           # midpoints m = (k + 1/2) 2^(e-3) of the binade [2^e, 2^(e+1))
        kk = g.integers(8, 16, 8)
        mids.append((kk + 0.5) * 2.0 ** (e - 3))
    mids = np.concatenate(mids)
    mids = mids * (1.0 + g.choice([-1.0, 0.0, 1.0], mids.size) * 2.0 ** -30)
    x = np.concatenate([x, mids])
    M = 3.0
    return np.log2(x) + M - 4.0                      # max x = 15.9 < 16, so ceil(max s) = M


def check_flip_bound(mod):
    """Every code a fp32-accurate evaluation of 2^(s - M + 4) (relative error
    within 2^-22, inside the oracle's margin) or a rounding at 2^t times the
    row scale (t = -1 .. 4, as a running integer max allows) changes is one
    the bound flags, and O, LSE move by no more than the bound."""
    g = np.random.default_rng(7)
    for trial in range(6):
        s = _midpoint_row(g, 400)
        w = g.standard_normal((s.size, 3)) * 2
        o, lse0, p, M, x = mod.softmax_row(s, w)
        assert M == 3.0
        st = mod.flip_steps(s, M, x)
        l, E = p.sum(), st.sum()
        ob = st @ np.abs(w - o) / (l - E)
        lb = -np.log1p(-E / l)
        variants = [mod.e4m3(x * (1.0 + g.uniform(-1, 1, x.size) * 2.0 ** -22)) * 2.0 ** -4]
        variants += [mod.e4m3(x * 2.0 ** t) * 2.0 ** -t * 2.0 ** -4 for t in (-1, 1, 2, 3, 4)]
        for p2 in variants:
            moved = p2 != p
            assert np.all(st[moved] >= np.abs(p2 - p)[moved] - 1e-18), "unflagged code change"
            o2 = p2 @ w / p2.sum()
            assert np.all(np.abs(o2 - o) <= ob + 1e-12)
            assert abs(np.log(p2.sum()) - np.log(l)) <= lb + 1e-12
        assert np.count_nonzero(st) > 20             # the row does exercise the bound


def check_method_error(mod):
    """Accuracy of the quantized method itself on N(0,1) inputs (random data
    spreads the softmax, the hardest case for P in e4m3): relative L2 of O
    against exact attention below 8e-2 (P and V each carry an e4m3 rounding
    of relative RMS 2^-4/sqrt(3) ~ 3.6%), LSE within 2e-2."""
    grid, tile, windows = (4, 8, 12), (2, 4, 4), [(3, 3, 3), (1, 3, 5)]
    q, k, v = tensors(1, 2, int(np.prod(grid)), 64, "bf16", 180)
    o, lse = mod.fwd(q, k, v, grid, tile, windows)
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows)
    rel = np.linalg.norm(o - ro) / np.linalg.norm(ro)
    assert rel < 8e-2, rel
    assert np.max(np.abs(lse - rl)) < 2e-2
    # and without the P rounding the error is that of the quantized inputs alone
    o2, _ = mod.fwd(q, k, v, grid, tile, windows, round_p=False)
    assert np.linalg.norm(o2 - ro) / np.linalg.norm(ro) < rel


def all_checks():
    """(name, callable(mod)) for every check, parameters bound."""
    out = [("e4m3-torch", check_e4m3_torch), ("e4m3-hand", check_e4m3_hand), ("e4m3-commutes", check_e4m3_commutes),
           ("int8-closed-forms", check_int8_closed_forms), ("p-rows-golden", check_p_rows_golden),
           ("k-block-scales", check_k_block_scales), ("v-channel-scales", check_v_channel_scales),
           ("q-row-scales", check_q_row_scales), ("smoothing", check_smoothing), ("reconstruct", check_reconstruct),
           ("flip-bound", check_flip_bound), ("method-error", check_method_error)]
    out += [("exact-codes-%d" % c, lambda m, c=c: check_exact_codes(m, c)) for c in range(len(CASES))]
    return out


@pytest.mark.parametrize("name,check", all_checks(), ids=[n for n, _ in all_checks()])
def test_quant_oracle_pin(name, check):
    check(quant)


def test_bound_output_shapes_and_zero_when_unrounded():
    grid, tile, windows = (4, 8, 12), (2, 4, 4), [(3, 3, 3)]
    q, k, v = tensors(1, 1, int(np.prod(grid)), 16, "bf16", 181)
    o, lse, ob, lb, oa = quant.fwd(q, k, v, grid, tile, windows, bound=True)
    assert ob.shape == o.shape and lb.shape == lse.shape and oa.shape == o.shape
    assert np.all(ob >= 0) and np.all(lb >= 0) and np.all(oa > 0)
    _, _, ob2, lb2, _ = quant.fwd(q, k, v, grid, tile, windows, bound=True, round_p=False)
    assert np.all(ob2 == 0) and np.all(lb2 == 0)
