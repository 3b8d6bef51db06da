"""ctypes front end of the plain C oracle (``sta_oracle.c``).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the tests, the smoke check and
the benchmark's CPU-baseline leg import this module.  It never touches the
HIP library and the HIP library never touches it.

All tensors here are numpy arrays in RASTER token order (t slowest, w
fastest), shaped [B, H, N, D]; floating inputs are float32 and outputs are
float64.  Row ids passed to ``fwd``/``bwd`` are flat ``(b*H + h)*N + i``
with ``i`` a raster token index.

Joint text + video sequences: ``n_text`` text tokens follow the grid's
video tokens in every [B, H, N, D] tensor (N = grid tokens + n_text); text
queries attend every key and every query attends the text keys.

Window options (the 3D-DSA variants): ``border="truncate"`` selects the
truncating border rule instead of the inward shift, and ``offsets`` may be
[T, 3] (one shift per query tile, shared by heads) or [H, T, 3] (one per
head and query tile).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sta_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force=False, src=_SRC, lib=_LIB):
    """Compile the oracle with gcc (plain -O2, no fast-math: sums keep the
    order the C source writes them in)."""
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(src):
        tmp = lib + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-shared", "-fPIC",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, lib)
    return lib


def load(path=None):
    """Load an oracle build (default: the one next to this file, built on
    demand).  A non-default path lets tests load deliberately altered builds."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    lib = ctypes.CDLL(build() if path is None else path)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.oracle_perm.argtypes = [i32p, i32p, i64p]
    lib.oracle_perm.restype = ctypes.c_int
    lib.oracle_index.argtypes = [i32p, i32p, ctypes.c_int, i32p, i32p, ctypes.c_int,
                                 ctypes.c_int, i32p, i32p, ctypes.c_int, i32p, i32p]
    lib.oracle_index.restype = ctypes.c_int
    lib.oracle_fwd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p, i32p, i32p, i32p, ctypes.c_int,
                               ctypes.c_int, ctypes.c_double, f32p, f32p, f32p, ctypes.c_int64, i64p, f64p, f64p]
    lib.oracle_fwd.restype = ctypes.c_int
    lib.oracle_bwd.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p, i32p, i32p, i32p, ctypes.c_int,
                               ctypes.c_int, ctypes.c_double, f32p, f32p, f32p, f32p,
                               ctypes.c_int64, i64p, f64p, ctypes.c_int64, i64p, f64p, f64p]
    lib.oracle_bwd.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


_active = None  # an alternative build selected with use(); None = default


def use(path):
    """Route the functions below to another build (None restores the default)."""
    global _active
    _active = None if path is None else load(path)


def _load():
    return _active if _active is not None else load()


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _i32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def tiles_per_axis(grid, tile):
    """Tiles per axis, ceil(grid / tile): a tile cut by the grid border holds
    only the tokens inside the grid."""
    return tuple(-(-g // t) for g, t in zip(grid, tile))


_TRUNCATE, _HEAD_OFFS = 1, 2


def _window_opts(offsets, H, T, border):
    """(offsets as a contiguous int32 array or None, flags)."""
    if border not in ("shift", "truncate"):
        raise ValueError("border must be 'shift' or 'truncate'")
    flags = _TRUNCATE if border == "truncate" else 0
    if offsets is None:
        return None, flags
    off = _i32(offsets)
    if off.ndim == 3:
        if off.shape != (H, T, 3):
            raise ValueError("per-head offsets must be [H, T, 3]")
        return off, flags | _HEAD_OFFS
    return off.reshape(T, 3), flags


def perm(grid, tile):
    """perm[r] = tile-contiguous position of raster token r."""
    lib = _load()
    n = int(np.prod(grid))
    out = np.empty(n, dtype=np.int64)
    if not lib.oracle_perm(_ptr(_i32(grid), ctypes.c_int32), _ptr(_i32(tile), ctypes.c_int32),
                           _ptr(out, ctypes.c_int64)):
        raise ValueError("grid and tile extents must be positive")
    return out


def index(grid, tile, windows, offsets=None, max_kv=None, max_q=None, border="shift"):
    """Block-sparse lists: (kv_idx [H,T,max_kv], kv_cnt [H,T], q_idx [H,T,max_q], q_cnt [H,T])."""
    lib = _load()
    windows = _i32(windows).reshape(-1, 3)
    H = windows.shape[0]
    T = int(np.prod(tiles_per_axis(grid, tile)))
    max_kv = T if max_kv is None else max_kv
    max_q = T if max_q is None else max_q
    kv_idx = np.empty((H, T, max_kv), np.int32)
    kv_cnt = np.empty((H, T), np.int32)
    q_idx = np.empty((H, T, max_q), np.int32)
    q_cnt = np.empty((H, T), np.int32)
    off, flags = _window_opts(offsets, H, T, border)
    ok = lib.oracle_index(_ptr(_i32(grid), ctypes.c_int32), _ptr(_i32(tile), ctypes.c_int32), H,
                          _ptr(windows, ctypes.c_int32), _ptr(off, ctypes.c_int32), flags,
                          max_kv, _ptr(kv_idx, ctypes.c_int32), _ptr(kv_cnt, ctypes.c_int32),
                          max_q, _ptr(q_idx, ctypes.c_int32), _ptr(q_cnt, ctypes.c_int32))
    if not ok:
        raise ValueError("invalid geometry or list capacity too small")
    return kv_idx, kv_cnt, q_idx, q_cnt


def _rows(rows, total):
    if rows is None:
        return np.arange(total, dtype=np.int64)
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def fwd(q, k, v, grid, tile, windows, offsets=None, scale=None, rows=None, border="shift", n_text=0):
    """Forward rows: returns (o [n_rows, D], lse [n_rows]) in float64.
    With rows=None every row is computed and o is reshaped to [B,H,N,D]."""
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N, D = q.shape
    assert k.shape == q.shape and v.shape == q.shape and N == int(np.prod(grid)) + n_text
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    windows = _i32(windows).reshape(H, 3)
    T = int(np.prod(tiles_per_axis(grid, tile)))
    off, flags = _window_opts(offsets, H, T, border)
    r = _rows(rows, B * H * N)
    o = np.empty((len(r), D), np.float64)
    lse = np.empty(len(r), np.float64)
    ok = lib.oracle_fwd(B, H, D, _ptr(_i32(grid), ctypes.c_int32), _ptr(_i32(tile), ctypes.c_int32),
                        _ptr(windows, ctypes.c_int32), _ptr(off, ctypes.c_int32), flags, int(n_text), scale,
                        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
                        len(r), _ptr(r, ctypes.c_int64), _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double))
    if not ok:
        raise ValueError("oracle_fwd rejected its arguments")
    if rows is None:
        return o.reshape(B, H, N, D), lse.reshape(B, H, N)
    return o, lse


def bwd(q, k, v, dout, grid, tile, windows, offsets=None, scale=None, qrows=None, krows=None, border="shift",
        n_text=0):
    """Backward rows: returns (dq [n_q, D], dk [n_k, D], dv [n_k, D]) in float64.
    With qrows=None and krows=None everything is computed, shaped [B,H,N,D]."""
    lib = _load()
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, H, N, D = q.shape
    assert N == int(np.prod(grid)) + n_text
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    windows = _i32(windows).reshape(H, 3)
    T = int(np.prod(tiles_per_axis(grid, tile)))
    off, flags = _window_opts(offsets, H, T, border)
    full = qrows is None and krows is None
    qr = _rows(qrows, B * H * N) if (qrows is not None or full) else np.zeros(0, np.int64)
    kr = _rows(krows, B * H * N) if (krows is not None or full) else np.zeros(0, np.int64)
    dq = np.empty((len(qr), D), np.float64)
    dk = np.empty((len(kr), D), np.float64)
    dv = np.empty((len(kr), D), np.float64)
    ok = lib.oracle_bwd(B, H, D, _ptr(_i32(grid), ctypes.c_int32), _ptr(_i32(tile), ctypes.c_int32),
                        _ptr(windows, ctypes.c_int32), _ptr(off, ctypes.c_int32), flags, int(n_text), scale,
                        _ptr(q, ctypes.c_float), _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float),
                        _ptr(dout, ctypes.c_float),
                        len(qr), _ptr(qr, ctypes.c_int64), _ptr(dq, ctypes.c_double),
                        len(kr), _ptr(kr, ctypes.c_int64), _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double))
    if not ok:
        raise ValueError("oracle_bwd rejected its arguments")
    if full:
        shp = (B, H, N, D)
        return dq.reshape(shp), dk.reshape(shp), dv.reshape(shp)
    return dq, dk, dv
