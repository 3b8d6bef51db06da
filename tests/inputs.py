"""Seeded synthetic inputs and the five workload shapes.

This module holds no attention arithmetic: only geometry, random draws and
the bf16 rounding of those draws.  The oracle, the HIP path, the smoke check
and the benchmark all take their inputs from here, so both sides of every
comparison see identical values.

Workloads stand in for the pages' 5-second 720P video generation ("Fast
Video Generation with Sliding Tile Attention", abstract): a (30,48,80) latent
token grid, 24 heads of width 128.  Values are i.i.d. N(0,1), drawn with
numpy's PCG64: tensors from seed [seed, stream, b, h] per (batch, head)
slab, streams 0=Q 1=K 2=V 3=dO; window offsets (stream 4) and the per-head
window choice (stream 5) from seed [seed, stream], with each workload's own
seed (1235 .. 1239).  bf16 workloads round the draws to bf16
(round-to-nearest-even).

Joint text + video workloads append n_text text tokens after the video
tokens of every (batch, head) slab, drawn in the same slab draw (N + n_text
rows).  The MOD-DiT README ("Token-Type-Aware Masking") puts text at about
1% of a joint sequence: TEXT_TOKENS_720P = 1164 is 1% of 115200 + 1164.
"""
import concurrent.futures
import os

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_DO, STREAM_OFF, STREAM_WIN, STREAM_TILE = range(7)

TEXT_TOKENS_720P = 1164

# Window sizes (in tiles) that the per-head variant draws from.
HEAD_WINDOW_CHOICES = ((3, 3, 3), (3, 3, 5), (5, 5, 5))

# The workloads, by name: the tiny fp32 forward on a 4x8x8 grid, the
# 7680-token forward, the 720P-shaped forward, the same with per-head
# windows and per-query-tile shifts, and the 720P training step.
CONFIGS = {
    "tiny-fp32": dict(seed=1235, B=1, H=2, D=64, dtype="f32", grid=(4, 8, 8), tile=(2, 4, 4),
                      window=(3, 3, 3), offsets=False, per_head=False, backward=False),
    "mid-7680": dict(seed=1236, B=1, H=24, D=128, dtype="bf16", grid=(8, 24, 40), tile=(4, 8, 8),
                     window=(3, 3, 3), offsets=False, per_head=False, backward=False),
    "720p": dict(seed=1237, B=1, H=24, D=128, dtype="bf16", grid=(30, 48, 80), tile=(6, 8, 8),
                 window=(3, 3, 5), offsets=False, per_head=False, backward=False),
    "720p-shifted-perhead": dict(seed=1238, B=1, H=24, D=128, dtype="bf16", grid=(30, 48, 80),
                                 tile=(6, 8, 8), window=None, offsets=True, per_head=True, backward=False),
    "720p-train": dict(seed=1239, B=1, H=24, D=128, dtype="bf16", grid=(30, 48, 80), tile=(6, 8, 8),
                       window=(3, 3, 5), offsets=False, per_head=False, backward=True),
}
WORKLOADS = tuple(CONFIGS)


def tiles_per_axis(grid, tile):
    return tuple(g // t for g, t in zip(grid, tile))


def num_tiles(grid, tile):
    return int(np.prod(tiles_per_axis(grid, tile)))


def rng(seed, stream):
    return np.random.default_rng([int(seed), int(stream)])


def round_bf16(x):
    """float32 array -> float32 array holding the bf16 round-to-nearest-even
    of each value (exactly representable in bf16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert np.all(np.isfinite(x[: min(x.size, 1 << 16)].reshape(-1)))
    u = x.view(np.uint32)
    # finite inputs stay below 0xFF800000, so the sum cannot wrap in 32 bits
    r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


def normal(shape, seed, stream, dtype):
    """[B,H,N,D] i.i.d. N(0,1); slab (b,h) is drawn from PCG64 seeded with
    [seed, stream, b, h], so the slabs can be generated in parallel."""
    B, H = shape[0], shape[1]
    out = np.empty(shape, np.float32)

    def fill(bh):
        b, h = divmod(bh, H)
        g = np.random.default_rng([int(seed), int(stream), b, h])
        x = g.standard_normal(size=shape[2:], dtype=np.float32)
        out[b, h] = round_bf16(x) if dtype == "bf16" else x

    with concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(B * H)))
    return out


def windows_for(cfg, seed=None):
    """[H,3] int32 window sizes (tiles) for a workload (its name, or its dict)."""
    c = CONFIGS[cfg] if isinstance(cfg, str) else cfg
    if not c["per_head"]:
        return np.tile(np.asarray(c["window"], np.int32), (c["H"], 1))
    seed = c["seed"] if seed is None else seed
    pick = rng(seed, STREAM_WIN).integers(0, len(HEAD_WINDOW_CHOICES), size=c["H"])
    return np.asarray([HEAD_WINDOW_CHOICES[i] for i in pick], np.int32)


def offsets_for(cfg, seed=None, lo=(-1, -2, -2), hi=(1, 2, 2)):
    """[T,3] int32 per-query-tile window shifts (tiles), or None."""
    c = CONFIGS[cfg] if isinstance(cfg, str) else cfg
    if not c["offsets"]:
        return None
    seed = c["seed"] if seed is None else seed
    T = num_tiles(c["grid"], c["tile"])
    return rng(seed, STREAM_OFF).integers(lo, hi, endpoint=True, size=(T, 3)).astype(np.int32)


def tensors(B, H, N, D, dtype, seed, with_dout=False):
    """(q, k, v[, dout]) float32 numpy arrays [B,H,N,D] in raster token order."""
    shape = (B, H, N, D)
    out = [normal(shape, seed, s, dtype) for s in (STREAM_Q, STREAM_K, STREAM_V)]
    if with_dout:
        out.append(normal(shape, seed, STREAM_DO, dtype))
    return tuple(out)


def tile_signal(B, H, grid, tile, D, dtype, seed, amp=1.0, disp=None, n_text=0, unit=False):
    """(q, k) float32 [B,H,N+n_text,D] in raster order with a component per
    tile on top of the N(0,1) draws of `tensors`: every video token of tile
    t of slab (b,h) gets amp * u[b,h,t] added to q; k gets amp * u[b,h,t-d]
    (d = disp[h], or disp[b][h] for a [B,H,3] array: the content of a tile
    moved by d tiles) where t - d lies in the tile grid, else amp * v[b,h,t]
    (v independent of u; the same for every tile when disp is None).  u, v
    are i.i.d. N(0,1) from seed [seed, STREAM_TILE]; text rows keep only
    the draws.  unit=True divides the video rows by sqrt(1 + amp^2), back
    to unit variance.  Rounded to bf16 last when dtype is "bf16"."""
    N = int(np.prod(grid))
    n = tuple(-(-a // b) for a, b in zip(grid, tile))
    T = int(np.prod(n))
    q, k, _ = tensors(B, H, N + n_text, D, "f32", seed)
    g = rng(seed, STREAM_TILE)
    u = g.standard_normal((B, H, T, D)).astype(np.float32)
    v = g.standard_normal((B, H, T, D)).astype(np.float32)
    t, h, w = np.unravel_index(np.arange(N), grid)
    tc = np.stack([t // tile[0], h // tile[1], w // tile[2]], 1)
    tid = (tc[:, 0] * n[1] + tc[:, 1]) * n[2] + tc[:, 2]
    dd = None if disp is None else np.asarray(disp, np.int64)
    for b in range(B):
        for hh in range(H):
            q[b, hh, :N] += amp * u[b, hh, tid]
            ks = v[b, hh, tid]
            if dd is not None:
                d = dd[hh] if dd.ndim == 2 else dd[b, hh]
                src = tc - d
                inside = np.all((src >= 0) & (src < np.array(n)), axis=1)
                sid = (src[:, 0] * n[1] + src[:, 1]) * n[2] + src[:, 2]
                ks = np.where(inside[:, None], u[b, hh, np.where(inside, sid, 0)], ks)
            k[b, hh, :N] += amp * ks
    if unit:
        q[:, :, :N] /= np.float32(np.sqrt(1.0 + amp * amp))
        k[:, :, :N] /= np.float32(np.sqrt(1.0 + amp * amp))
    if dtype == "bf16":
        q, k = round_bf16(q), round_bf16(k)
    return q, k


def workload(cfg, heads=None, with_dout=None, n_text=0, grid=None):
    """Everything one workload needs: dict with geometry, windows, offsets and
    q, k, v (and dout for the training workload).  ``heads`` keeps only the
    first few heads (their values equal those heads of the full draw).
    dout is drawn for the training workload, or when with_dout is True.
    With n_text > 0 the tensors hold N + n_text rows per slab (text last).
    ``grid`` replaces the workload's token grid (same tile, windows and
    seeds), e.g. the 720p latent grid (30,45,80) that the tile does not
    divide."""
    c = dict(CONFIGS[cfg])
    if heads is not None:
        c["H"] = heads
    if grid is not None:
        c["grid"] = tuple(int(x) for x in grid)
    seed = c["seed"]
    N = int(np.prod(c["grid"]))
    w = windows_for(cfg)[: c["H"]]
    off = offsets_for(cfg)
    want = c["backward"] if with_dout is None else with_dout
    ts = tensors(c["B"], c["H"], N + n_text, c["D"], c["dtype"], seed, with_dout=want)
    c.update(N=N, n_text=n_text, windows=w, offsets=off, q=ts[0], k=ts[1], v=ts[2], dout=ts[3] if want else None,
             scale=1.0 / np.sqrt(c["D"]), seed=seed)
    return c


def counted_flops(kv_counts, B, L, D):
    """Forward FLOP counted on unmasked tile pairs only: 4*B*L^2*D per pair
    (QK^T and PV, 2 flop per multiply-add).  kv_counts: per (head, q-tile)."""
    return 4.0 * B * float(np.sum(kv_counts)) * L * L * D
