"""Pins of the quantized-attention oracle (oracle/quant.py; CPU only).

The e4m3 rounding is pinned to torch's float8_e4m3fn cast (a library
routine) and to hand-worked values; the int8 codes to their closed forms;
the attention steps (window, text keys, smoothing, LSE correction) by
running them on unquantized "codes" against the exact oracle; the property
the GPU kernel's integer running max rests on (e4m3 rounding commutes with
power-of-two scaling in the normal range) directly; and the method's own
error against exact attention is bounded on random inputs (the accuracy
study of the quantized path)."""
import numpy as np
import pytest
import torch

from oracle import oracle, quant
from tests.inputs import tensors


def test_e4m3_matches_torch_cast():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(20000) * 8, g.uniform(-448, 448, 20000), 2.0 ** g.uniform(-12, -5, 5000),
                        -(2.0 ** g.uniform(-12, 8, 5000))]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(quant.e4m3(x), want.astype(np.float64))


@pytest.mark.parametrize("x,want", [(1.0, 1.0), (1.0625, 1.0), (1.1875, 1.25), (1.1, 1.125), (17.0, 16.0),
                                    (19.0, 20.0), (448.0, 448.0), (2 ** -9, 2 ** -9), (2 ** -10, 0.0),
                                    (3 * 2 ** -11, 2 ** -9), (0.015625, 0.015625), (-1.0625, -1.0), (0.0, 0.0)])
def test_e4m3_hand_values(x, want):
    """Spacing 2^(e-3) in the binade [2^e, 2^(e+1)), 2^-9 below 2^-6; ties to
    the even mantissa (1.0625 -> 1.0, 1.1875 -> 1.25, 17 -> 16, 19 -> 20)."""
    assert quant.e4m3(np.float32(x)) == want


def test_e4m3_commutes_with_powers_of_two_in_the_normal_range():
    g = np.random.default_rng(1)
    x = 2.0 ** g.uniform(-6, 0, 50000)              # normal range, <= 1
    for k in range(0, 9):                            # 2^k x stays <= 256 < 448
        assert np.array_equal(quant.e4m3(x * 2.0 ** k), quant.e4m3(x) * 2.0 ** k)


def test_int8_codes_closed_forms():
    g = np.random.default_rng(2)
    x = (g.standard_normal((50, 64)) * g.uniform(0.1, 10, (50, 1))).astype(np.float32)
    amax = np.abs(x).max(axis=1, keepdims=True)
    c, s = quant.int8_codes(x, amax)
    assert np.all(np.abs(c).max(axis=1) == 127)
    at = np.abs(x).argmax(axis=1)
    assert np.array_equal(c[np.arange(50), at], np.sign(x[np.arange(50), at]).astype(np.int32) * 127)
    assert np.all(np.abs(x - c * s) <= s * (0.5 + 1e-5))
    z, zs = quant.int8_codes(np.zeros((2, 8), np.float32), np.zeros((2, 1), np.float32))
    assert np.all(z == 0) and np.all(zs == 0)


CASES = [
    # grid, tile, windows, n_text, per-head offsets
    ((4, 8, 12), (2, 4, 4), [(3, 3, 3), (1, 3, 3)], 0, False),
    ((5, 7, 9), (2, 4, 4), [(1, 3, 3), (3, 1, 3)], 23, True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_attention_steps_on_exact_codes_equal_exact_attention(case):
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
    o, lse = quant.fwd(q, k, v, grid, tile, windows, off, n_text=nt, quant=fake, round_p=False)
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows, off, n_text=nt)
    np.testing.assert_allclose(o, ro, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(lse, rl, rtol=1e-9, atol=1e-9)


def test_quantize_reconstructs_inputs_within_half_a_step():
    grid, tile, nt = (5, 7, 9), (2, 4, 4), 23
    S = int(np.prod(grid)) + nt
    q, k, v = tensors(1, 2, S, 32, "bf16", 170)
    Q = quant.quantize(q, k, v, grid, tile, nt)
    assert np.all(np.abs(q - Q["qc"] * Q["sq"]) <= Q["sq"] * (0.5 + 1e-5))
    ks = k - Q["m"]
    assert np.all(np.abs(ks - Q["kc"] * Q["sk"]) <= Q["sk"] * (0.5 + 1e-5))
    # every 64-key block of a tile holds one code of magnitude 127 (its max)
    rel_v = np.abs(v - Q["vc"] * Q["sv"]) / np.maximum(np.abs(v), 1e-30)
    assert np.all(rel_v[np.abs(v) >= Q["sv"] * 2.0 ** -6] <= 2.0 ** -4 + 1e-6)     # e4m3: half a mantissa step
    assert np.all(np.abs(Q["vc"]) <= 448)


def test_method_error_against_exact_attention():
    """Accuracy of the quantized method itself on N(0,1) inputs (random data
    spreads the softmax, the hardest case for P in e4m3): relative L2 of O
    against exact attention below 8e-2 (P and V each carry an e4m3 rounding
    of relative RMS 2^-4/sqrt(3) ~ 3.6%), LSE within 2e-2."""
    grid, tile, windows = (4, 8, 12), (2, 4, 4), [(3, 3, 3), (1, 3, 5)]
    q, k, v = tensors(1, 2, int(np.prod(grid)), 64, "bf16", 180)
    o, lse = quant.fwd(q, k, v, grid, tile, windows)
    ro, rl = oracle.fwd(q, k, v, grid, tile, windows)
    rel = np.linalg.norm(o - ro) / np.linalg.norm(ro)
    assert rel < 8e-2, rel
    assert np.max(np.abs(lse - rl)) < 2e-2
    # and without the P rounding the error is that of the quantized inputs alone
    o2, _ = quant.fwd(q, k, v, grid, tile, windows, round_p=False)
    assert np.linalg.norm(o2 - ro) / np.linalg.norm(ro) < rel
