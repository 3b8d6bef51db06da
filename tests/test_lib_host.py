"""Host-side tests of libsta (no GPU needed): the library loads, exports every
entry point the header declares, sizes indices like the oracle, and rejects
malformed calls before anything is launched."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import sliding_tile_attention_amd as sta
from oracle import oracle
from tests.inputs import CONFIGS, WORKLOADS, offsets_for, windows_for

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libsta.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sta_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(sta.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", sta.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(sta_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(sta.lib, name)


def test_measurement_probes_load_and_reject_bad_sizes():
    """The benchmark's probe library (exponential rate, matrix-core rate, LDS
    read rate, copy calibration, block copies into LDS) loads beside libsta and rejects sizes before
    launching anything."""
    path = os.path.join(os.path.dirname(sta.LIB_PATH), "libsta_probe.so")
    lib = ctypes.CDLL(path)
    lib.sta_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.sta_probe_exp.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.sta_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.sta_probe_lds.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert lib.sta_probe_copy(None, None, 0, None) == 1
    assert lib.sta_probe_copy(None, None, 24, None) == 1       # not a multiple of 16
    assert lib.sta_probe_exp(None, 0, 16, None) == 1
    assert lib.sta_probe_mfma(None, 0, 16, None) == 1
    assert lib.sta_probe_mfma(None, 4, -1, None) == 1
    assert lib.sta_probe_lds(None, 0, 16, None) == 1
    lib.sta_probe_block_copy.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p]
    assert lib.sta_probe_block_copy(None, 8192, 4, 16, None, None) == 1         # below one 16 KB block
    assert lib.sta_probe_block_copy(None, 16384 + 16, 4, 16, None, None) == 1   # not whole blocks
    assert lib.sta_probe_block_copy(None, 16384 << 31, 4, 16, None, None) == 1  # too many blocks
    assert lib.sta_probe_block_copy(None, 16384, 0, 16, None, None) == 1
    assert lib.sta_probe_block_copy(None, 16384, 4, 0, None, None) == 1


def test_status_strings_and_version():
    for code, name in ((0, "STA_OK"), (1, "STA_ERR_INVALID"), (2, "STA_ERR_UNSUPPORTED"), (3, "STA_ERR_HIP")):
        assert sta.lib.sta_status_str(code).decode() == name
    assert sta.lib.sta_version() >= 10000


@pytest.mark.parametrize("cfg", WORKLOADS)
def test_index_dims_match_oracle(cfg):
    c = CONFIGS[cfg]
    geom = sta.Geometry(c["grid"], c["tile"])
    w = windows_for(cfg)
    off = offsets_for(cfg)
    max_kv, max_q = sta.sta_index_dims(geom, w, off is not None)
    kv_idx, kv_cnt, q_idx, q_cnt = oracle.index(c["grid"], c["tile"], w, off)
    assert max_kv == kv_cnt.max()
    if off is None:
        assert max_q == q_cnt.max()          # exact without shifts
    else:
        assert max_q == geom.num_tiles and max_q >= q_cnt.max()


def test_index_dims_random_geometries():
    g = np.random.default_rng(3)
    for _ in range(50):
        n = g.integers(1, 9, size=3)
        tile = g.integers(1, 3, size=3)
        grid = tuple(int(a * b) for a, b in zip(n, tile))
        w = g.integers(1, 10, size=(int(g.integers(1, 4)), 3))
        _, kv_cnt, _, q_cnt = oracle.index(grid, tuple(int(x) for x in tile), w)
        assert sta.sta_index_dims(sta.Geometry(grid, tuple(int(x) for x in tile)), w, False) == \
            (kv_cnt.max(), q_cnt.max())


def test_index_dims_ragged_geometries():
    """Grids the tile does not divide (and tiles longer than the grid):
    capacities as the oracle's lists, whose tile grid is ceil(grid/tile)."""
    g = np.random.default_rng(8)
    for _ in range(50):
        grid = tuple(int(x) for x in g.integers(1, 13, size=3))
        tile = tuple(int(x) for x in g.integers(1, 6, size=3))
        w = g.integers(1, 8, size=(int(g.integers(1, 4)), 3))
        _, kv_cnt, _, q_cnt = oracle.index(grid, tile, w)
        geom = sta.Geometry(grid, tile)
        assert geom.num_tiles == kv_cnt.shape[1]
        assert sta.sta_index_dims(geom, w, False) == (kv_cnt.max(), q_cnt.max())


# ---- argument checks: every call below must fail on the host -----------

GEOM = sta.Geometry((4, 8, 8), (2, 4, 4))


def _fake(n=1 << 16, align=0):
    """A host buffer whose address stands in for a device pointer; the calls
    below are rejected before anything could touch it."""
    t = torch.empty(n + 64, dtype=torch.uint8)
    off = (-t.data_ptr()) % 16 + align
    return t[off:]


def _expect(status, fn, *args):
    with pytest.raises(sta.StaError) as e:
        fn(*args)
    assert e.value.status == status
    assert sta.lib.sta_last_error().decode()


class _FakeIndex:
    def __init__(self, H=2, T=8, max_kv=8, max_q=8, transposed=True):
        self.num_heads, self.num_tiles, self.max_kv, self.max_q = H, T, max_kv, max_q
        self.buf = _fake()
        self.transposed = transposed

    def c(self):
        p = self.buf.data_ptr()
        return sta.sta_index(self.num_heads, self.num_tiles, self.max_kv, self.max_q, p, p,
                             p if self.transposed else None, p if self.transposed else None)


def test_reorder_rejects_bad_arguments():
    a, b = _fake(), _fake()
    _expect(sta.STA_ERR_INVALID, sta.sta_tile_reorder, a, b, 1, 4, sta.Geometry((5, 0, 8), (2, 4, 4)), 0, 0)
    _expect(sta.STA_ERR_INVALID, sta.sta_tile_reorder, a, b, 1, 4, sta.Geometry((4, 8, 8), (0, 4, 4)), 0, 0)
    _expect(sta.STA_ERR_INVALID, sta.sta_tile_reorder, None, b, 1, 4, GEOM, 0, 0)
    _expect(sta.STA_ERR_INVALID, sta.sta_tile_reorder, a, b, 0, 4, GEOM, 0, 0)
    _expect(sta.STA_ERR_INVALID, sta.sta_tile_reorder, a, b, 1, 0, GEOM, 0, 0)
    _expect(sta.STA_ERR_INVALID, sta.sta_tile_reorder, a, a[16:], 1, 4, GEOM, 0, 0)   # overlap


def test_build_index_rejects_bad_arguments():
    w = [(3, 3, 3)] * 2
    _expect(sta.STA_ERR_INVALID, sta.sta_build_index, GEOM, [(0, 3, 3), (3, 3, 3)], None, _FakeIndex(), 0)
    _expect(sta.STA_ERR_INVALID, sta.sta_build_index, GEOM, w, None, _FakeIndex(H=3), 0)
    _expect(sta.STA_ERR_INVALID, sta.sta_build_index, GEOM, w, None, _FakeIndex(T=9), 0)
    _expect(sta.STA_ERR_INVALID, sta.sta_build_index, GEOM, w, None, _FakeIndex(max_kv=7), 0)
    _expect(sta.STA_ERR_INVALID, sta.sta_build_index, GEOM, w, None, _FakeIndex(max_q=7), 0)
    # a grid the tile does not divide has ceil(grid/tile) tiles per axis: 12 here
    _expect(sta.STA_ERR_INVALID, sta.sta_build_index, sta.Geometry((4, 8, 9), (2, 4, 4)), w, None,
            _FakeIndex(), 0)
    # with shifts the transposed capacity must be the tile count
    _expect(sta.STA_ERR_INVALID, sta.sta_build_index, sta.Geometry((6, 8, 8), (2, 4, 4)), w, _fake(),
            _FakeIndex(T=12, max_kv=12, max_q=11), 0)


def _fwd_args(**kw):
    a = dict(q=_fake(), k=_fake(), v=_fake(), o=_fake(), lse=_fake(), B=1, H=2, D=64, dtype=sta.STA_BF16,
             scale=0.125, geom=GEOM, index=_FakeIndex(), stream=0)
    a.update(kw)
    return a


def test_fwd_rejects_bad_arguments():
    f = lambda **kw: sta.sta_fwd(**_fwd_args(**kw))
    bad = [
        (sta.STA_ERR_INVALID, dict(q=None)),
        (sta.STA_ERR_INVALID, dict(lse=None)),
        (sta.STA_ERR_INVALID, dict(B=0)),
        (sta.STA_ERR_INVALID, dict(H=3)),                       # index built for 2 heads
        (sta.STA_ERR_INVALID, dict(scale=0.0)),
        (sta.STA_ERR_INVALID, dict(scale=float("nan"))),
        (sta.STA_ERR_INVALID, dict(dtype=7)),
        (sta.STA_ERR_INVALID, dict(k=_fake(align=2))),           # misaligned
        (sta.STA_ERR_INVALID, dict(index=_FakeIndex(T=9))),
        (sta.STA_ERR_INVALID, dict(geom=sta.Geometry((4, 8, 9), (2, 4, 4)))),   # 12 tiles, index has 8
        (sta.STA_ERR_INVALID, dict(geom=sta.Geometry((4, -8, 8), (2, 4, 4)))),
        (sta.STA_ERR_UNSUPPORTED, dict(D=96)),
        (sta.STA_ERR_UNSUPPORTED, dict(geom=sta.Geometry((2, 3, 3), (2, 3, 1)),
                                       index=_FakeIndex(T=3, max_kv=3, max_q=3))),  # L=6, bf16
    ]
    for status, kw in bad:
        with pytest.raises(sta.StaError) as e:
            f(**kw)
        assert e.value.status == status, (kw, e.value)


def test_bwd_rejects_bad_arguments():
    def f(**kw):
        a = _fwd_args()
        a.update(dout=_fake(), dq=_fake(), dk=_fake(), dv=_fake(), delta_ws=_fake())
        a.update(kw)
        sta.sta_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
                    a["delta_ws"], a["B"], a["H"], a["D"], a["dtype"], a["scale"], a["geom"], a["index"],
                    a["stream"])
    for status, kw in [(sta.STA_ERR_INVALID, dict(index=_FakeIndex(transposed=False))),
                       (sta.STA_ERR_INVALID, dict(dout=None)),
                       (sta.STA_ERR_INVALID, dict(delta_ws=None)),
                       (sta.STA_ERR_INVALID, dict(dq=_fake(align=4))),
                       (sta.STA_ERR_UNSUPPORTED, dict(D=32))]:
        with pytest.raises(sta.StaError) as e:
            f(**kw)
        assert e.value.status == status, (kw, e.value)


def test_index_dims_rejects_bad_arguments():
    _expect(sta.STA_ERR_INVALID, sta.sta_index_dims, GEOM, [(1, 1, 0)], False)
    _expect(sta.STA_ERR_INVALID, sta.sta_index_dims, sta.Geometry((3, 8, 8), (2, 4, -4)), [(1, 1, 1)], False)
    g = sta.lib.sta_index_dims(ctypes.byref(GEOM.c()), 0, None, 0, None, None)
    assert g == sta.STA_ERR_INVALID
    # extents near the int32 limit are refused as too large, not wrapped
    big = 2 ** 31 - 1
    for grid, tile in (((big, 2, 2), (1, 1, 1)), ((big, big, big), (7, 7, 7)), ((big, 1, 1), (big, 1, 1))):
        _expect(sta.STA_ERR_UNSUPPORTED, sta.sta_index_dims, sta.Geometry(grid, tile), [(1, 1, 1)], False)
    # status codes outside the enum still get a name
    assert sta.lib.sta_status_str(-1).decode() == sta.lib.sta_status_str(99).decode() == "STA_ERR_UNKNOWN"


def test_index_dims_ex_match_oracle_with_options():
    """Truncated windows without shifts: the capacities are exact (the
    central tile of every axis has the full window and the most attendees)."""
    g = np.random.default_rng(4)
    for _ in range(40):
        n = g.integers(1, 9, size=3)
        tile = tuple(int(x) for x in g.integers(1, 3, size=3))
        grid = tuple(int(a * b) for a, b in zip(n, tile))
        w = g.integers(1, 10, size=(int(g.integers(1, 4)), 3))
        _, kv_cnt, _, q_cnt = oracle.index(grid, tile, w, border="truncate")
        geom = sta.Geometry(grid, tile)
        assert sta.sta_index_dims_ex(geom, w, False, "truncate") == (kv_cnt.max(), q_cnt.max())
        assert sta.sta_index_dims_ex(geom, w, False, "shift") == sta.sta_index_dims(geom, w, False)
        T = int(np.prod(n))
        assert sta.sta_index_dims_ex(geom, w, True, "truncate", True)[1] == T


def test_index_options_reject_bad_values():
    w = (sta.sta_dim3 * 1)(sta.sta_dim3(3, 3, 3))
    kv, q = ctypes.c_int32(), ctypes.c_int32()
    for border, per_head in ((2, 0), (-1, 0), (0, 2)):
        opts = sta.sta_index_opts(border, per_head)
        st = sta.lib.sta_index_dims_ex(ctypes.byref(GEOM.c()), 1, w, 0, ctypes.byref(opts), ctypes.byref(kv),
                                       ctypes.byref(q))
        assert st == sta.STA_ERR_INVALID and sta.lib.sta_last_error().decode()
        st = sta.lib.sta_build_index_ex(ctypes.byref(GEOM.c()), 1, w, None, ctypes.byref(opts),
                                        ctypes.byref(_FakeIndex(H=1).c()), None)
        assert st == sta.STA_ERR_INVALID
    with pytest.raises(ValueError):
        sta.sta_index_dims_ex(GEOM, [(3, 3, 3)], False, "wrap")


def test_attn_options_reject_bad_text_counts():
    """Joint text + video options: a negative text count is malformed and a
    sequence beyond 2^30 rows unsupported, for every call that takes them."""
    a = _fwd_args()
    fwd = lambda nt: sta.sta_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["D"], a["dtype"],
                                   a["scale"], a["geom"], a["index"], nt, 0)
    bwd = lambda nt: sta.sta_bwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], _fake(), _fake(), _fake(), _fake(),
                                    _fake(), a["B"], a["H"], a["D"], a["dtype"], a["scale"], a["geom"], a["index"],
                                    sta.STA_BWD_ALL, nt, 0)
    reorder = lambda nt: sta.sta_tile_reorder_ex(_fake(), _fake(), 1, 4, GEOM, 0, nt, 0)
    for call in (fwd, bwd, reorder):
        _expect(sta.STA_ERR_INVALID, call, -1)
        _expect(sta.STA_ERR_UNSUPPORTED, call, 2 ** 30)
    # other argument checks still apply with text tokens
    _expect(sta.STA_ERR_INVALID, lambda: sta.sta_fwd_ex(None, a["k"], a["v"], a["o"], a["lse"], 1, 2, 64,
                                                        sta.STA_BF16, 0.125, GEOM, a["index"], 5, 0))


def test_attn_options_null_equals_zero_text():
    """A NULL options pointer is accepted like n_text = 0 (argument checks
    only: a malformed call fails the same way with either)."""
    a = _fwd_args(B=0)
    args = (a["q"], a["k"], a["v"], a["o"], a["lse"], 0, 2, 64, sta.STA_BF16, 0.125)
    g, x = ctypes.byref(GEOM.c()), ctypes.byref(a["index"].c())
    st_null = sta.lib.sta_fwd_ex(*[sta._ptr(t) if isinstance(t, torch.Tensor) else t for t in args], g, x, None,
                                 None)
    st_zero = sta.lib.sta_fwd_ex(*[sta._ptr(t) if isinstance(t, torch.Tensor) else t for t in args], g, x,
                                 ctypes.byref(sta.sta_attn_opts(0)), None)
    assert st_null == st_zero == sta.STA_ERR_INVALID


def test_precision_option_checks():
    """The quantized forward takes bf16 tensors only, the backward runs in
    the tensors' dtype, and unknown precision values are malformed."""
    a = _fwd_args()

    def fwd(prec, dtype=sta.STA_BF16):
        opts = sta.sta_attn_opts(0, prec)
        st = sta.lib.sta_fwd_ex(*[sta._ptr(a[n]) for n in ("q", "k", "v", "o", "lse")], 1, 2, 64, dtype, 0.125,
                                ctypes.byref(GEOM.c()), ctypes.byref(a["index"].c()), ctypes.byref(opts), None)
        return st

    def bwd(prec):
        opts = sta.sta_attn_opts(0, prec)
        ptrs = [sta._ptr(_fake()) for _ in range(10)]
        return sta.lib.sta_bwd_ex(*ptrs, 1, 2, 64, sta.STA_BF16, 0.125, ctypes.byref(GEOM.c()),
                                  ctypes.byref(a["index"].c()), sta.STA_BWD_ALL, ctypes.byref(opts), None)
    assert fwd(7) == sta.STA_ERR_INVALID
    assert fwd(sta.STA_PREC_FP8, sta.STA_F32) == sta.STA_ERR_UNSUPPORTED
    assert bwd(sta.STA_PREC_FP8) == sta.STA_ERR_UNSUPPORTED
    assert bwd(5) == sta.STA_ERR_INVALID


def test_index_for_batch_items_checks():
    """An attention call takes an index of H list sets (shared by the batch)
    or B*H (one per batch item); any other count is malformed."""
    a = _fwd_args(B=2, H=2, index=_FakeIndex(H=3))
    with pytest.raises(sta.StaError) as e:
        sta.sta_fwd(**a)
    assert e.value.status == sta.STA_ERR_INVALID and "list sets" in str(e.value)
    a = _fwd_args(B=2, H=2, index=_FakeIndex(H=4, T=9))          # B*H sets, wrong tile count: still checked
    with pytest.raises(sta.StaError) as e:
        sta.sta_fwd(**a)
    assert e.value.status == sta.STA_ERR_INVALID and "tiles" in str(e.value)


def test_window_shifts_rejects_bad_arguments():
    def f(**kw):
        a = dict(q=_fake(), k=_fake(), B=1, H=2, D=64, dtype=sta.STA_BF16, scale=0.125, geom=GEOM,
                 windows=[(1, 1, 1), (3, 3, 3)], radius=(1, 1, 1), offsets=_fake(), border="shift",
                 per_batch=False, n_text=0)
        a.update(kw)
        sta.sta_window_shifts(a["q"], a["k"], a["B"], a["H"], a["D"], a["dtype"], a["scale"], a["geom"],
                              a["windows"], a["radius"], a["offsets"], a["border"], a["per_batch"], a["n_text"], 0)
    bad = [
        (sta.STA_ERR_INVALID, dict(q=None)),
        (sta.STA_ERR_INVALID, dict(offsets=None)),
        (sta.STA_ERR_INVALID, dict(k=_fake(align=4))),
        (sta.STA_ERR_INVALID, dict(B=0)),
        (sta.STA_ERR_INVALID, dict(scale=-1.0)),
        (sta.STA_ERR_INVALID, dict(scale=float("inf"))),
        (sta.STA_ERR_INVALID, dict(dtype=3)),
        (sta.STA_ERR_INVALID, dict(radius=(0, -1, 0))),
        (sta.STA_ERR_INVALID, dict(windows=[(1, 1, 1), (3, 0, 3)])),
        (sta.STA_ERR_INVALID, dict(border="sideways")),
        (sta.STA_ERR_INVALID, dict(n_text=-2)),
        (sta.STA_ERR_INVALID, dict(geom=sta.Geometry((4, 0, 8), (2, 4, 4)))),
        (sta.STA_ERR_UNSUPPORTED, dict(D=96)),
        (sta.STA_ERR_UNSUPPORTED, dict(radius=(8, 8, 8))),                       # 4913 candidates
        (sta.STA_ERR_UNSUPPORTED, dict(geom=sta.Geometry((64, 64, 64), (2, 2, 2)),
                                       windows=[(21, 21, 21)] * 2, radius=(0, 0, 0))),  # region 9261 tiles
    ]
    for status, kw in bad:
        with pytest.raises(sta.StaError) as e:
            f(**kw)
        assert e.value.status == status, (kw, e.value)
    # per_batch must be 0 or 1
    opts = sta.sta_shift_opts(0, 2, 0)
    w, _ = sta._windows([(1, 1, 1)] * 2)
    st = sta.lib.sta_window_shifts(sta._ptr(_fake()), sta._ptr(_fake()), 1, 2, 64, sta.STA_BF16, 0.125,
                                   ctypes.byref(GEOM.c()), w, ctypes.byref(sta.sta_dim3(1, 1, 1)),
                                   ctypes.byref(opts), sta._ptr(_fake()), None)
    assert st == sta.STA_ERR_INVALID


def test_window_shifts_noalloc_checks_before_launching():
    """The allocation-free producer takes the same argument checks, and
    rejects tile means beyond its 16 MiB scratch before anything runs: the
    720P shape (24 heads of 300 tiles, D = 128) fits for up to 2 batch items
    with per-item shifts, not for 3; without per-item shifts the means are
    pooled and any batch fits."""
    geom = sta.Geometry((30, 48, 80), (6, 8, 8))

    def call(B, per_batch, **kw):
        a = dict(q=_fake(), D=128, windows=[(3, 3, 5)] * 24)
        a.update(kw)
        sta.sta_window_shifts(a["q"], _fake(), B, 24, a["D"], sta.STA_BF16, 0.088, geom, a["windows"],
                              (1, 1, 1), _fake(), "shift", per_batch, 0, 0, noalloc=True)
    for kw, status in ((dict(q=None), sta.STA_ERR_INVALID), (dict(D=96), sta.STA_ERR_UNSUPPORTED),
                       (dict(windows=[(3, 0, 5)] * 24), sta.STA_ERR_INVALID)):
        with pytest.raises(sta.StaError) as e:
            call(1, False, **kw)
        assert e.value.status == status, kw
    with pytest.raises(sta.StaError) as e:
        call(3, True)
    assert e.value.status == sta.STA_ERR_UNSUPPORTED and "scratch" in str(e.value)
    assert 2 * 2 * 24 * 300 * 128 * 4 <= 16 << 20 < 2 * 3 * 24 * 300 * 128 * 4


def test_layout_option_checks():
    """Raster layout: unknown values are malformed; grids the tile does not
    divide, text rows, and bf16 tiles whose rows the 32-row copy pattern
    cannot gather are unsupported.  Checked before anything is launched."""
    def fwd(layout, geom=GEOM, n_text=0, dtype=sta.STA_BF16, index=None):
        a = _fwd_args()
        opts = sta.sta_attn_opts(n_text, 0, layout)
        idx = index or a["index"]
        return sta.lib.sta_fwd_ex(*[sta._ptr(a[n]) for n in ("q", "k", "v", "o", "lse")], 1, 2, 64, dtype, 0.125,
                                  ctypes.byref(geom.c()), ctypes.byref(idx.c()), ctypes.byref(opts), None)

    def bwd(layout, geom=GEOM, n_text=0):
        a = _fwd_args()
        opts = sta.sta_attn_opts(n_text, 0, layout)
        ptrs = [sta._ptr(_fake()) for _ in range(10)]
        return sta.lib.sta_bwd_ex(*ptrs, 1, 2, 64, sta.STA_BF16, 0.125, ctypes.byref(geom.c()),
                                  ctypes.byref(a["index"].c()), sta.STA_BWD_ALL, ctypes.byref(opts), None)
    for call in (fwd, bwd):
        assert call(2) == sta.STA_ERR_INVALID
        assert call(-1) == sta.STA_ERR_INVALID
        # (5,8,8) with (2,4,4) tiles: 3x2x2 = 12 tiles, the last t-tile cut
        assert call(sta.STA_LAYOUT_RASTER, geom=sta.Geometry((5, 8, 8), (2, 4, 4))) == sta.STA_ERR_UNSUPPORTED
        assert call(sta.STA_LAYOUT_RASTER, n_text=3) == sta.STA_ERR_UNSUPPORTED
    # tw = 32 does not divide the 16-row copies of the bf16 kernels
    wide = sta.Geometry((4, 4, 64), (2, 2, 32))
    assert fwd(sta.STA_LAYOUT_RASTER, geom=wide, index=_FakeIndex(T=8)) == sta.STA_ERR_UNSUPPORTED
    # th*tw = 24 is not a power of two
    odd = sta.Geometry((4, 12, 8), (2, 6, 4))
    assert fwd(sta.STA_LAYOUT_RASTER, geom=odd, index=_FakeIndex(T=8)) == sta.STA_ERR_UNSUPPORTED
    # the window-shift producer takes the same layout values
    w, _ = sta._windows([(1, 1, 1)] * 2)
    for layout, want in ((3, sta.STA_ERR_INVALID),):
        opts = sta.sta_shift_opts(0, 0, 0, layout)
        st = sta.lib.sta_window_shifts(sta._ptr(_fake()), sta._ptr(_fake()), 1, 2, 64, sta.STA_BF16, 0.125,
                                       ctypes.byref(GEOM.c()), w, ctypes.byref(sta.sta_dim3(1, 1, 1)),
                                       ctypes.byref(opts), sta._ptr(_fake()), None)
        assert st == want
