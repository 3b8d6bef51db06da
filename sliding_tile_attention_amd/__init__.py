"""Python binding of libsta (sliding-tile attention for MI355X / gfx950).

Thin ctypes layer over the C ABI in ``include/libsta.h``: the functions
named ``sta_*`` take torch tensors (device memory) and marshal their data
pointers, sizes and the current HIP stream; every step of the computation
runs in the HIP kernels of ``libsta.so``.  There is no CPU fallback: if the
library is missing, importing this package raises.

Operator: "Fast Video Generation with Sliding Tile Attention" (abstract) --
attention restricted to a window of tiles around each query tile of the
(T,H,W) video token grid; optional per-query-tile window shifts stand in for
the deformable windows (3D-DSA) of "MegaSlide-DiT" (abstract).  Joint text +
video sequences (``n_text`` text tokens after the video tokens) follow the
token-type-aware masking of the MOD-DiT README ("Token-Type-Aware Masking").
"""
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsta.so")

STA_OK, STA_ERR_INVALID, STA_ERR_UNSUPPORTED, STA_ERR_HIP = 0, 1, 2, 3
STA_BF16, STA_F32 = 0, 1
STA_BWD_DELTA, STA_BWD_DKDV, STA_BWD_DQ, STA_BWD_ALL = 1, 2, 4, 7
STA_BORDER_SHIFT, STA_BORDER_TRUNCATE = 0, 1
STA_PREC_DEFAULT, STA_PREC_FP8 = 0, 1
_PRECISIONS = {"default": STA_PREC_DEFAULT, "fp8": STA_PREC_FP8}
STA_LAYOUT_TILE, STA_LAYOUT_RASTER = 0, 1
_LAYOUTS = {"tile": STA_LAYOUT_TILE, "raster": STA_LAYOUT_RASTER}
EXPORTS = ("sta_status_str", "sta_last_error", "sta_version", "sta_index_dims", "sta_index_dims_ex",
           "sta_tile_reorder", "sta_tile_reorder_ex", "sta_build_index", "sta_build_index_ex", "sta_fwd",
           "sta_fwd_ex", "sta_bwd", "sta_bwd_parts", "sta_bwd_ex", "sta_window_shifts", "sta_window_shifts_noalloc")


class StaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (_STATUS_NAMES.get(status, status), message))
        self.status = status


_STATUS_NAMES = {0: "STA_OK", 1: "STA_ERR_INVALID", 2: "STA_ERR_UNSUPPORTED", 3: "STA_ERR_HIP"}


class sta_dim3(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32)]


class sta_geom(ctypes.Structure):
    _fields_ = [("grid", sta_dim3), ("tile", sta_dim3)]


class sta_index_opts(ctypes.Structure):
    _fields_ = [("border", ctypes.c_int32), ("per_head_offsets", ctypes.c_int32)]


class sta_attn_opts(ctypes.Structure):
    _fields_ = [("n_text", ctypes.c_int32), ("precision", ctypes.c_int32), ("layout", ctypes.c_int32)]


class sta_shift_opts(ctypes.Structure):
    _fields_ = [("border", ctypes.c_int32), ("per_batch", ctypes.c_int32), ("n_text", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class sta_index(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("num_tiles", ctypes.c_int32),
                ("max_kv", ctypes.c_int32), ("max_q", ctypes.c_int32),
                ("kv_idx", ctypes.c_void_p), ("kv_cnt", ctypes.c_void_p),
                ("q_idx", ctypes.c_void_p), ("q_cnt", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libsta.so is not built (expected at %s); run "
                          "`python sliding_tile_attention_amd/build.py`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    G, X, OP = ctypes.POINTER(sta_geom), ctypes.POINTER(sta_index), ctypes.POINTER(sta_index_opts)
    AO = ctypes.POINTER(sta_attn_opts)
    SO = ctypes.POINTER(sta_shift_opts)
    W = ctypes.POINTER(sta_dim3)
    sig = {
        "sta_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "sta_last_error": (ctypes.c_char_p, []),
        "sta_version": (I32, []),
        "sta_index_dims": (ctypes.c_int, [G, I32, W, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "sta_index_dims_ex": (ctypes.c_int, [G, I32, W, I32, OP, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "sta_tile_reorder": (ctypes.c_int, [P, P, I64, I64, G, I32, P]),
        "sta_tile_reorder_ex": (ctypes.c_int, [P, P, I64, I64, G, I32, AO, P]),
        "sta_build_index": (ctypes.c_int, [G, I32, W, P, X, P]),
        "sta_build_index_ex": (ctypes.c_int, [G, I32, W, P, OP, X, P]),
        "sta_fwd": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, ctypes.c_int, F32, G, X, P]),
        "sta_fwd_ex": (ctypes.c_int, [P, P, P, P, P, I32, I32, I32, ctypes.c_int, F32, G, X, AO, P]),
        "sta_bwd": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P, I32, I32, I32, ctypes.c_int, F32, G, X, P]),
        "sta_bwd_parts": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P, I32, I32, I32, ctypes.c_int, F32, G, X,
                                         I32, P]),
        "sta_bwd_ex": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P, I32, I32, I32, ctypes.c_int, F32, G, X,
                                      I32, AO, P]),
        "sta_window_shifts": (ctypes.c_int, [P, P, I32, I32, I32, ctypes.c_int, F32, G, W, W, SO, P, P]),
        "sta_window_shifts_noalloc": (ctypes.c_int, [P, P, I32, I32, I32, ctypes.c_int, F32, G, W, W, SO, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


lib = _load()


def _check(status):
    if status != STA_OK:
        raise StaError(status, lib.sta_last_error().decode())


@dataclass(frozen=True)
class Geometry:
    """Token grid (T,H,W) and tile (tt,th,tw) extents."""
    grid: tuple
    tile: tuple

    def c(self):
        return sta_geom(sta_dim3(*self.grid), sta_dim3(*self.tile))

    @property
    def tiles(self):
        """Tiles per axis; a tile cut by the grid border counts as one."""
        return tuple(-(-g // t) for g, t in zip(self.grid, self.tile))

    @property
    def num_tiles(self):
        a, b, c = self.tiles
        return a * b * c

    @property
    def tokens(self):
        a, b, c = self.grid
        return a * b * c

    @property
    def tile_tokens(self):
        a, b, c = self.tile
        return a * b * c


def _windows(windows):
    ws = [tuple(int(x) for x in w) for w in windows]
    arr = (sta_dim3 * len(ws))(*[sta_dim3(*w) for w in ws])
    return arr, len(ws)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ---------------------------------------------------------------- C ABI --

def _opts(border, per_head_offsets):
    if border not in ("shift", "truncate"):
        raise ValueError("border must be 'shift' or 'truncate'")
    return sta_index_opts(STA_BORDER_TRUNCATE if border == "truncate" else STA_BORDER_SHIFT,
                          int(bool(per_head_offsets)))


def sta_index_dims(geom, windows, has_offsets):
    """(max_kv, max_q) capacities for H = len(windows) heads."""
    w, H = _windows(windows)
    kv, q = ctypes.c_int32(), ctypes.c_int32()
    _check(lib.sta_index_dims(ctypes.byref(geom.c()), H, w, int(bool(has_offsets)),
                              ctypes.byref(kv), ctypes.byref(q)))
    return kv.value, q.value


def sta_index_dims_ex(geom, windows, has_offsets, border="shift", per_head_offsets=False):
    w, H = _windows(windows)
    kv, q = ctypes.c_int32(), ctypes.c_int32()
    opts = _opts(border, per_head_offsets)
    _check(lib.sta_index_dims_ex(ctypes.byref(geom.c()), H, w, int(bool(has_offsets)), ctypes.byref(opts),
                                 ctypes.byref(kv), ctypes.byref(q)))
    return kv.value, q.value


def sta_tile_reorder(src, dst, outer, row_bytes, geom, inverse, stream=None):
    _check(lib.sta_tile_reorder(_ptr(src), _ptr(dst), int(outer), int(row_bytes), ctypes.byref(geom.c()),
                                int(bool(inverse)), _stream(stream)))


def sta_tile_reorder_ex(src, dst, outer, row_bytes, geom, inverse, n_text=0, stream=None):
    opts = sta_attn_opts(int(n_text))
    _check(lib.sta_tile_reorder_ex(_ptr(src), _ptr(dst), int(outer), int(row_bytes), ctypes.byref(geom.c()),
                                   int(bool(inverse)), ctypes.byref(opts), _stream(stream)))


def sta_build_index(geom, windows, offsets, index, stream=None):
    """offsets: None or int32 device tensor [num_tiles, 3]; index: StaIndex."""
    w, H = _windows(windows)
    _check(lib.sta_build_index(ctypes.byref(geom.c()), H, w, _ptr(offsets), ctypes.byref(index.c()),
                               _stream(stream)))


def sta_build_index_ex(geom, windows, offsets, index, border="shift", per_head_offsets=False, stream=None):
    """offsets: None, or int32 device tensor [num_tiles, 3] ([H, num_tiles, 3]
    with per_head_offsets); border: 'shift' or 'truncate'."""
    w, H = _windows(windows)
    opts = _opts(border, per_head_offsets)
    _check(lib.sta_build_index_ex(ctypes.byref(geom.c()), H, w, _ptr(offsets), ctypes.byref(opts),
                                  ctypes.byref(index.c()), _stream(stream)))


def sta_fwd(q, k, v, o, lse, B, H, D, dtype, scale, geom, index, stream=None):
    _check(lib.sta_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, D, dtype, float(scale),
                       ctypes.byref(geom.c()), ctypes.byref(index.c()), _stream(stream)))


def sta_fwd_ex(q, k, v, o, lse, B, H, D, dtype, scale, geom, index, n_text=0, stream=None, precision=STA_PREC_DEFAULT,
               layout=STA_LAYOUT_TILE):
    opts = sta_attn_opts(int(n_text), int(precision), int(layout))
    _check(lib.sta_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, D, dtype, float(scale),
                          ctypes.byref(geom.c()), ctypes.byref(index.c()), ctypes.byref(opts), _stream(stream)))


def sta_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta_ws, B, H, D, dtype, scale, geom, index, stream=None):
    _check(lib.sta_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                       _ptr(dv), _ptr(delta_ws), B, H, D, dtype, float(scale), ctypes.byref(geom.c()),
                       ctypes.byref(index.c()), _stream(stream)))


def sta_bwd_parts(q, k, v, o, lse, dout, dq, dk, dv, delta_ws, B, H, D, dtype, scale, geom, index, parts,
                  stream=None):
    _check(lib.sta_bwd_parts(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(delta_ws), B, H, D, dtype, float(scale), ctypes.byref(geom.c()),
                             ctypes.byref(index.c()), int(parts), _stream(stream)))


def sta_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta_ws, B, H, D, dtype, scale, geom, index, parts,
               n_text=0, stream=None, layout=STA_LAYOUT_TILE):
    opts = sta_attn_opts(int(n_text), STA_PREC_DEFAULT, int(layout))
    _check(lib.sta_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                          _ptr(dv), _ptr(delta_ws), B, H, D, dtype, float(scale), ctypes.byref(geom.c()),
                          ctypes.byref(index.c()), int(parts), ctypes.byref(opts), _stream(stream)))


def sta_window_shifts(q, k, B, H, D, dtype, scale, geom, windows, radius, offsets, border="shift", per_batch=False,
                      n_text=0, stream=None, layout=STA_LAYOUT_TILE, noalloc=False):
    """offsets: int32 device tensor [H, num_tiles, 3] ([B, H, num_tiles, 3]
    with per_batch), written by the call.  noalloc=True calls
    sta_window_shifts_noalloc (static scratch, no allocation)."""
    w, nw = _windows(windows)
    if nw != H:
        raise ValueError("need one window per head")
    r = sta_dim3(*[int(x) for x in radius])
    opts = sta_shift_opts(STA_BORDER_TRUNCATE if border == "truncate" else STA_BORDER_SHIFT if border == "shift"
                          else -1, int(bool(per_batch)), int(n_text), int(layout))
    fn = lib.sta_window_shifts_noalloc if noalloc else lib.sta_window_shifts
    _check(fn(_ptr(q), _ptr(k), B, H, D, dtype, float(scale), ctypes.byref(geom.c()), w, ctypes.byref(r),
              ctypes.byref(opts), _ptr(offsets), _stream(stream)))


# ------------------------------------------------- argument checks --
# The C ABI takes bare pointers and cannot see strides, dtypes or devices, so
# the wrappers below check them before any pointer is passed: a transposed
# view (say q.transpose(1, 2) of a [B, S, H, D] tensor) or a tensor of
# another dtype would otherwise be read as if it were contiguous [B, H, S, D].
# Device checks come last, after every layout check.

def _check_attn(geom, n_text, tensors, lse=None, index=None):
    """tensors: [(name, tensor)] that must be contiguous [B, H, S, D] of one
    shape, dtype (bfloat16 or float32) and device, with S = geom.tokens +
    n_text; lse: a contiguous float32 [B, H, S] tensor on that device; index:
    a StaIndex of H or B*H list sets on that device."""
    name0, ref = tensors[0]
    for name, t in tensors:
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch tensor" % name)
        if t.dim() != 4:
            raise ValueError("%s must be [B, H, S, D], got shape %s" % (name, tuple(t.shape)))
        if t.shape != ref.shape:
            raise ValueError("%s has shape %s, %s has %s" % (name, tuple(t.shape), name0, tuple(ref.shape)))
        if t.dtype != ref.dtype:
            raise TypeError("%s is %s, %s is %s" % (name, t.dtype, name0, ref.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous [B, H, S, D] (a transposed view is not)" % name)
    _dtype_code(ref)
    B, H, S, D = ref.shape
    if S != geom.tokens + n_text:
        raise ValueError("token axis holds %d rows, the geometry %d (+ %d text)" % (S, geom.tokens, n_text))
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [B, H, S] = %s tensor, got %s %s" % (
                (B, H, S), lse.dtype, tuple(lse.shape)))
    if index is not None and index.num_heads not in (H, B * H):
        raise ValueError("index holds %d list sets; H = %d heads (or B*H = %d) expected" % (
            index.num_heads, H, B * H))
    others = ([("lse", lse)] if lse is not None else []) + ([("index", index.kv_idx)] if index is not None else [])
    for name, t in tensors + others:
        if t.device != ref.device:
            raise ValueError("%s is on %s, %s on %s" % (name, t.device, name0, ref.device))
    if ref.device.type != "cuda":
        raise ValueError("libsta computes on a GPU: tensors are on %s" % ref.device)


def _device(d):
    """torch.device of d, a bare "cuda" resolved to the current device."""
    d = torch.device(d)
    if d.type == "cuda" and d.index is None and torch.cuda.is_available():
        d = torch.device("cuda", torch.cuda.current_device())
    return d


def _check_offsets(offsets, geom, H, device):
    """offsets: int32, contiguous, [T, 3], [H, T, 3] or [B, H, T, 3] for the
    geometry's T tiles and the H windows, on the index's device."""
    if not isinstance(offsets, torch.Tensor):
        raise TypeError("offsets must be a torch tensor")
    if offsets.dtype != torch.int32:
        raise TypeError("offsets must be int32, got %s" % offsets.dtype)
    T = geom.num_tiles
    shp = tuple(offsets.shape)
    if not (shp == (T, 3) or shp == (H, T, 3) or (len(shp) == 4 and shp[1:] == (H, T, 3) and shp[0] >= 1)):
        raise ValueError("offsets must be [T, 3], [H, T, 3] or [B, H, T, 3] with T = %d tiles and H = %d windows, "
                         "got %s" % (T, H, shp))
    if not offsets.is_contiguous():
        raise ValueError("offsets must be contiguous")
    if offsets.device != _device(device):
        raise ValueError("offsets are on %s, the index on %s" % (offsets.device, _device(device)))


# ------------------------------------------------- allocation helpers --

class StaIndex:
    """Device buffers of a block-sparse index (allocated with torch).
    offsets: None, an int32 device tensor [num_tiles, 3] shared by the heads,
    [H, num_tiles, 3] (one set per head) or [B, H, num_tiles, 3] (one set per
    batch item and head: the index then holds B*H list sets, list set
    b*H + h serving (b, h)); border: 'shift' or 'truncate'."""

    def __init__(self, geom, windows, offsets=None, device="cuda", transposed=True, stream=None, border="shift"):
        if offsets is not None:
            _check_offsets(offsets, geom, len(windows), device)
        if torch.device(device).type != "cuda":
            raise ValueError("the index is built on a GPU device, not %s" % device)
        self.batch = 1
        if offsets is not None and offsets.dim() == 4:
            self.batch = offsets.shape[0]
            windows = list(windows) * self.batch
            offsets = offsets.reshape(-1, offsets.shape[2], 3).contiguous()
        H, T = len(windows), geom.num_tiles
        per_head = offsets is not None and offsets.dim() == 3
        self.max_kv, max_q = sta_index_dims_ex(geom, windows, offsets is not None, border, per_head)
        self.max_q = max_q if transposed else 0
        i32 = dict(dtype=torch.int32, device=device)
        self.kv_idx = torch.empty((H, T, self.max_kv), **i32)
        self.kv_cnt = torch.empty((H, T), **i32)
        self.q_idx = torch.empty((H, T, self.max_q), **i32) if transposed else None
        self.q_cnt = torch.empty((H, T), **i32) if transposed else None
        self.num_heads, self.num_tiles = H, T
        self.windows = [tuple(w) for w in windows]
        self.border = border
        sta_build_index_ex(geom, windows, offsets, self, border, per_head, stream)

    def c(self):
        return sta_index(self.num_heads, self.num_tiles, self.max_kv, self.max_q,
                         self.kv_idx.data_ptr(), self.kv_cnt.data_ptr(),
                         self.q_idx.data_ptr() if self.q_idx is not None else None,
                         self.q_cnt.data_ptr() if self.q_cnt is not None else None)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return STA_BF16
    if t.dtype == torch.float32:
        return STA_F32
    raise TypeError("libsta supports bfloat16 and float32 tensors, got %s" % t.dtype)


def window_shifts(q, k, geom, windows, radius, scale=None, border="shift", per_batch=False, n_text=0, stream=None,
                  layout="tile", noalloc=False):
    """Window shift of every query tile (and head, and batch item with
    per_batch) chosen on device from q, k [B,H,N+n_text,D] (video rows in
    tile order, or raster order with layout="raster"): int32 [H, num_tiles,
    3] or [B, H, num_tiles, 3], ready for StaIndex(..., offsets=...)."""
    B, H, S, D = q.shape
    _check_attn(geom, n_text, [("q", q), ("k", k)])
    scale = D ** -0.5 if scale is None else scale
    shape = (B, H, geom.num_tiles, 3) if per_batch else (H, geom.num_tiles, 3)
    out = torch.empty(shape, dtype=torch.int32, device=q.device)
    sta_window_shifts(q, k, B, H, D, _dtype_code(q), scale, geom, windows, radius, out, border, per_batch, n_text,
                      stream, _LAYOUTS[layout], noalloc)
    return out


def tile_reorder(x, geom, inverse=False, out=None, stream=None, n_text=0):
    """Permute the token axis of a contiguous [..., N + n_text, C] tensor
    between raster and tile order (the n_text text rows after the grid's
    tokens stay in place); returns a new tensor (or writes `out`)."""
    S = geom.tokens + n_text
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch tensor")
    if x.dim() < 2 or x.shape[-2] != S:
        raise ValueError("x must be [..., %d, C] (%d grid tokens + %d text rows), got shape %s" % (
            S, geom.tokens, n_text, tuple(x.shape)))
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    else:
        if not isinstance(out, torch.Tensor):
            raise TypeError("out must be a torch tensor")
        if out.shape != x.shape or out.dtype != x.dtype:
            raise ValueError("out is %s %s, x is %s %s" % (out.dtype, tuple(out.shape), x.dtype, tuple(x.shape)))
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
        if out.device != x.device:
            raise ValueError("out is on %s, x on %s" % (out.device, x.device))
    if x.device.type != "cuda":
        raise ValueError("libsta computes on a GPU: x is on %s" % x.device)
    if x.numel() == 0:
        return out
    row_bytes = x.shape[-1] * x.element_size()
    outer = x.numel() // (S * x.shape[-1])
    sta_tile_reorder_ex(x, out, outer, row_bytes, geom, inverse, n_text, stream)
    return out


def forward(q, k, v, geom, index, scale=None, stream=None, n_text=0, precision="default", layout="tile"):
    """q, k, v [B,H,N+n_text,D] (video rows in tile order, then the text
    rows) -> (o [B,H,N+n_text,D], lse [B,H,N+n_text] fp32).  precision
    "fp8" runs the quantized products (INT8 QK^T, FP8 PV; bf16 tensors).
    layout "raster": every tensor holds the video rows in raster token order
    (no reorder needed; grids the tile divides, no text rows)."""
    _check_attn(geom, n_text, [("q", q), ("k", k), ("v", v)], index=index)
    B, H, S, D = q.shape
    scale = D ** -0.5 if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    sta_fwd_ex(q, k, v, o, lse, B, H, D, _dtype_code(q), scale, geom, index, n_text, stream, _PRECISIONS[precision],
               _LAYOUTS[layout])
    return o, lse


def backward(q, k, v, o, lse, dout, geom, index, scale=None, stream=None, n_text=0, layout="tile"):
    """Gradients (dq, dk, dv) of forward(); same layout as forward()."""
    _check_attn(geom, n_text, [("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)], lse, index)
    B, H, S, D = q.shape
    scale = D ** -0.5 if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    sta_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, D, _dtype_code(q), scale, geom, index,
               STA_BWD_ALL, n_text, stream, _LAYOUTS[layout])
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    """forward() and backward() as one differentiable operation: the forward
    keeps q, k, v, o and lse for the backward, which runs on the stream that
    autograd runs it on."""

    @staticmethod
    def forward(ctx, q, k, v, geom, index, scale, n_text, layout):
        o, lse = forward(q, k, v, geom, index, scale, n_text=n_text, layout=layout)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (geom, index, scale, n_text, layout)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        geom, index, scale, n_text, layout = ctx.args
        dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), geom, index, scale, n_text=n_text, layout=layout)
        return dq, dk, dv, None, None, None, None, None


def attention(q, k, v, geom, index, scale=None, n_text=0, layout="tile"):
    """Differentiable sliding-tile attention: o = forward(q, k, v, ...)[0],
    with gradients for q, k and v through backward() (training through the
    operator, "MegaSlide-DiT", abstract).  Same tensors, layouts and checks
    as forward(); bf16 or fp32."""
    return _Attention.apply(q, k, v, geom, index, scale, n_text, layout)
