"""Oracle of the quantized (INT8 QK^T, FP8 PV) sliding-tile attention forward.

Test infrastructure only: loaded by tests/ and never by the library.  The
pages name quantized attention kernels only as a dependency of one of them
(MOD-DiT README, "Project Structure" and "Acknowledgements": the
SageAttention submodule); the scheme below is this library's own reading of
such a kernel, so every step is spelled out here and followed by the GPU:

  1. K smoothing: m = mean over the rows of K of each (b, h) (fp64, then
     fp32).  Subtracting one vector from every key shifts all scores of a
     query by the same amount, so the softmax is unchanged.
  2. Q: int8 codes per row, amax = max |q|, codes = rint(q * (127 / amax))
     in fp32, scale amax / 127.
  3. K - m: int8 codes per block of 64 consecutive rows of a tile in tile
     order (text pseudo-tiles of L rows likewise), same formulas.
  4. V: e4m3 codes per channel d over all rows of (b, h): amax_d = max |v_d|,
     codes = e4m3(v * (448 / amax_d)) in fp32, scale amax_d / 448.
  5. Base-2 scores s_ij = (sum_d qc_id kc_jd) * sq_i * sk_j * scale * log2(e)
     over the allowed keys j (the STA window, plus text keys), exact: the
     integer sums and the fp32 scales multiplied in fp64 (scale is the fp32
     value the library receives).
  6. M_i = ceil(max_j s_ij); p_ij = 2^-4 e4m3(2^(s_ij - M_i + 4)), the power
     of two taken exactly: P is rounded at 16 times the row-max scale, so
     that every probability down to 2^-10 of the row's largest stays in
     e4m3's normal range (3 mantissa bits; the subnormal range below 2^-6
     holds fewer).
  7. l_i = sum_j p_ij;  o_i = (sum_j p_ij vc_j) * sv / l_i;
     LSE_i = ln 2 * (M_i + log2 l_i) + scale * <q_i, m>  (the natural-log LSE
     of the unsmoothed scores).

A kernel evaluates step 5 in floating point, so where 2^(s - M + 4) lies
within its rounding error of a midpoint between two e4m3 values it may take
the other one; and a kernel may round at a power-of-two multiple of the row
scale (a running integer max), which commutes with e4m3 rounding in the
normal range only.  `fwd(..., bound=True)` lists, per row, every key whose
code such arithmetic can move (one e4m3 step, or one subnormal step below
2^-5) and bounds the resulting change of O and LSE: with E_i the sum of
those steps (in p units), |dO_id| <= sum_j step_j |w_jd - o_id| / (l_i - E_i)
and |dLSE_i| <= -ln(1 - E_i / l_i), w_j the dequantized value rows.

e4m3 is the OCP FP8 E4M3 format (1 sign bit, 4 exponent bits with bias 7, 3
mantissa bits, largest finite 448, subnormal spacing 2^-9), rounded to
nearest with ties to even.
"""
import numpy as np

from oracle import oracle

E4M3_MAX = 448.0
KEY_BLOCK = 64          # keys per K scale block
P_SHIFT = 4             # P is rounded at 2^P_SHIFT times the row-max scale


def e4m3(x):
    """Round to the nearest e4m3 value, ties to even (|x| <= 448)."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    if np.any(a >= 464.0):
        raise ValueError("value beyond the e4m3 range")
    # spacing of the binade of a: 2^(e - 3), with the subnormal spacing 2^-9
    # for a < 2^-6
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    step = 2.0 ** (e - 3)
    r = np.round(a / step) * step            # numpy rounds halves to even
    return np.where(x < 0, -r, r)


def e4m3_step(x):
    """Spacing of the e4m3 values around |x| (<= 448): 2^(e - 3) in the
    binade [2^e, 2^(e+1)), 2^-9 below 2^-6."""
    a = np.abs(np.asarray(x, np.float64))
    return 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3)


def e4m3_near_midpoint(x, rel):
    """True where |x| lies within rel * |x| of a midpoint between two
    adjacent e4m3 values (where rounding can go either way)."""
    a = np.abs(np.asarray(x, np.float64))
    h = e4m3_step(a)
    frac = a / h - np.floor(a / h)
    return np.abs(frac - 0.5) * h <= rel * a


def p_codes(s):
    """Step 6 for one row of exact base-2 logits s (float64): returns
    (p, M, x) with M = ceil(max s), x = 2^(s - M + P_SHIFT) and
    p = 2^-P_SHIFT e4m3(x)."""
    s = np.asarray(s, np.float64)
    M = float(np.ceil(s.max()))
    x = np.exp2(s - M + P_SHIFT)
    return e4m3(x) * 2.0 ** -P_SHIFT, M, x


def flip_steps(s, M, x):
    """Per key of a row: the largest change (p units) of its probability that
    a kernel evaluating step 5 in fp32 can make; zero where the code is
    decided.  The margin covers the fp32 roundings of the logit factor (four
    roundings), of the fused exponent argument and of a hardware 2^x (within
    4 ulp), doubled: 2 (ln 2 (4 |s| + |s - M| + 8) 2^-24 + 2^-21)."""
    s = np.asarray(s, np.float64)
    rel = 2.0 * (np.log(2.0) * (4.0 * np.abs(s) + np.abs(s - M) + 8.0) * 2.0 ** -24 + 2.0 ** -21)
    step = np.where(e4m3_near_midpoint(x, rel), e4m3_step(x), 0.0)
    # below 2^-5 a kernel rounding at up to twice the row scale, or at a
    # finer one, differs by less than one subnormal step of twice the scale
    step = np.where(x < 2.0 ** -5, 2.0 ** -8, step)
    return step * 2.0 ** -P_SHIFT


def int8_codes(x, amax):
    """int8 codes of fp32 x under the fp32 group maxima amax (broadcast):
    rint(x * (127 / amax)) in fp32; zero groups give zero codes."""
    x = np.asarray(x, np.float32)
    amax = np.asarray(amax, np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(127.0) / np.where(amax > 0, amax, np.float32(1.0)), np.float32(0.0))
    return np.clip(np.rint((x * inv).astype(np.float32)), -127, 127).astype(np.int32), (amax / np.float32(127.0))


def softmax_row(s, w, round_p=True):
    """Steps 6-7 for one row: exact base-2 logits s [n] and dequantized value
    rows w [n, D] (float64).  Returns (o [D], ln 2 (M + log2 l), p, M, x);
    round_p=False takes p = 2^(s - M) unrounded (x is then None)."""
    if round_p:
        p, M, x = p_codes(s)
    else:
        M, x = float(np.ceil(np.max(s))), None
        p = np.exp2(np.asarray(s, np.float64) - M)
    l = p.sum()
    return (p @ np.asarray(w, np.float64)) / l, np.log(2.0) * (M + np.log2(l)), p, M, x


def _tile_layout(grid, tile, n_text):
    """Per raster token (and text token): tile id and rank in the tile's rows
    (compact tile order); text tokens form pseudo-tiles of L rows."""
    N = int(np.prod(grid))
    L = int(np.prod([min(a, b) for a, b in zip(grid, tile)]))
    p = oracle.perm(grid, tile)
    t, h, w = np.unravel_index(np.arange(N), grid)
    n = oracle.tiles_per_axis(grid, tile)
    tid = ((t // tile[0]) * n[1] + h // tile[1]) * n[2] + w // tile[2]
    T = int(np.prod(n))
    start = np.full(T, np.iinfo(np.int64).max)
    np.minimum.at(start, tid, p)
    rank = p - start[tid]
    j = np.arange(n_text)
    return (np.concatenate([tid, T + j // L]), np.concatenate([rank, j % L]), T, L)


def quantize(q, k, v, grid, tile, n_text=0):
    """Steps 1-4 for [B,H,S,D] float arrays in raster order (text rows last).
    Returns a dict of codes and scales."""
    q, k, v = (np.asarray(x, np.float32) for x in (q, k, v))
    tid, rank, T, L = _tile_layout(grid, tile, n_text)
    m = k.astype(np.float64).mean(axis=2, keepdims=True).astype(np.float32)       # [B,H,1,D]
    ks = (k - m).astype(np.float32)
    qc, sq = int8_codes(q, np.abs(q).max(axis=3, keepdims=True))
    # K blocks: key j belongs to block (tid[j], rank[j] // 64)
    blk = tid * ((L + KEY_BLOCK - 1) // KEY_BLOCK) + rank // KEY_BLOCK
    nblk = int(blk.max()) + 1
    amax_k = np.zeros(k.shape[:2] + (nblk,), np.float32)
    for b in range(k.shape[0]):
        for hh in range(k.shape[1]):
            np.maximum.at(amax_k[b, hh], blk, np.abs(ks[b, hh]).max(axis=1))
    kc, sk_blk = int8_codes(ks, amax_k[:, :, blk, None])
    amax_v = np.abs(v).max(axis=2, keepdims=True)                                    # [B,H,1,D]
    with np.errstate(divide="ignore"):
        inv_v = np.where(amax_v > 0, np.float32(E4M3_MAX) / np.where(amax_v > 0, amax_v, 1), 0).astype(np.float32)
    vc = e4m3((v * inv_v).astype(np.float32))
    sv = (amax_v / np.float32(E4M3_MAX)).astype(np.float32)
    return dict(m=m, qc=qc, sq=sq, kc=kc, sk=sk_blk, vc=vc, sv=sv)


def _allowed_keys(grid, tile, windows, offsets, border, n_text, h):
    """Callable row -> allowed key indices (raster order, text last)."""
    N = int(np.prod(grid))
    kv_idx, kv_cnt, _, _ = oracle.index(grid, tile, windows, offsets, border=border)
    tid, _, T, _ = _tile_layout(grid, tile, 0)
    members = [np.flatnonzero(tid == t) for t in range(T)]
    text = np.arange(N, N + n_text)
    allk = np.arange(N + n_text)

    def keys(i):
        if i >= N:
            return allk
        lst = kv_idx[h, tid[i], : kv_cnt[h, tid[i]]]
        return np.concatenate([members[t] for t in lst] + [text])
    return keys


def fwd(q, k, v, grid, tile, windows, offsets=None, scale=None, rows=None, border="shift", n_text=0, quant=None,
        round_p=True, bound=False):
    """Steps 5-7 on the quantized tensors.  Returns (o, lse) in float64: for
    rows=None shaped [B,H,S,D] and [B,H,S], else [n_rows, D], [n_rows] for the
    flat row ids (b*H + h)*S + i.  `quant` replaces step 1-4's output (a dict
    as quantize returns); round_p=False skips the e4m3 rounding of P.
    bound=True also returns (o_bound, lse_bound, o_abs): the bounds on |dO|
    and |dLSE| of the header (codes a fp32 evaluation can move), and
    sum_j p_ij |w_jd| / l_i (the scale of accumulation rounding)."""
    B, H, S, D = np.shape(q)
    scale = float(np.float32(1.0 / np.sqrt(D) if scale is None else scale))
    windows = np.asarray(windows, np.int64).reshape(-1, 3)
    r = np.arange(B * H * S) if rows is None else np.asarray(rows, np.int64)
    keyfns = {}
    slabs = {}

    def slab(b, hh):
        """Steps 1-4 of one (b, h) (each slab is quantized on its own)."""
        if quant is not None:
            return {n: a[b:b + 1, hh:hh + 1] if np.shape(a)[1] == H else a for n, a in quant.items()}
        if (b, hh) not in slabs:
            slabs[(b, hh)] = quantize(q[b:b + 1, hh:hh + 1], k[b:b + 1, hh:hh + 1], v[b:b + 1, hh:hh + 1], grid,
                                      tile, n_text)
        return slabs[(b, hh)]
    o = np.zeros((len(r), D))
    lse = np.zeros(len(r))
    ob, lb, oa = np.zeros((len(r), D)), np.zeros(len(r)), np.zeros((len(r), D))
    c = scale * np.log2(np.e)
    for n_, row in enumerate(r):
        b, hh, i = row // (H * S), (row // S) % H, row % S
        if hh not in keyfns:
            off = offsets
            if offsets is not None and np.ndim(offsets) == 3:
                off = np.asarray(offsets)[hh]
            keyfns[hh] = _allowed_keys(grid, tile, windows[hh:hh + 1], off, border, n_text, 0)
        j = keyfns[hh](i)
        Q = slab(b, hh)
        acc = Q["kc"][0, 0, j].astype(np.float64) @ Q["qc"][0, 0, i].astype(np.float64)
        s = acc * float(Q["sq"][0, 0, i, 0]) * Q["sk"][0, 0, j, 0].astype(np.float64) * c
        w = Q["vc"][0, 0, j].astype(np.float64) * Q["sv"][0, 0, 0].astype(np.float64)
        o[n_], lse0, p, M, x = softmax_row(s, w, round_p)
        lse[n_] = lse0 + scale * float(np.asarray(q[b, hh, i], np.float64) @ Q["m"][0, 0, 0].astype(np.float64))
        if bound:
            l = p.sum()
            st = flip_steps(s, M, x) if round_p else np.zeros_like(p)
            E = st.sum()
            ob[n_] = (st @ np.abs(w - o[n_])) / (l - E) if E < l else np.inf
            lb[n_] = -np.log1p(-E / l) if E < l else np.inf
            oa[n_] = (p @ np.abs(w)) / l
    if rows is None:
        o, lse = o.reshape(B, H, S, D), lse.reshape(B, H, S)
        ob, lb, oa = ob.reshape(B, H, S, D), lb.reshape(B, H, S), oa.reshape(B, H, S, D)
    return (o, lse, ob, lb, oa) if bound else (o, lse)
