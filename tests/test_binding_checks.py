"""The Python binding checks what the C ABI cannot see (CPU only): strides,
dtypes, shapes and devices of the tensors it passes as bare pointers.  Each
malformed call is rejected before any pointer is passed; host tensors reach
the device check last."""
from types import SimpleNamespace

import pytest
import torch

import sliding_tile_attention_amd as sta

GEOM = sta.Geometry((4, 8, 12), (2, 4, 4))          # 384 tokens, 12 tiles
B, H, S, D = 1, 2, 384, 64


def _index(heads=H):
    return SimpleNamespace(num_heads=heads, kv_idx=torch.empty(0, dtype=torch.int32))


def _qkv(dtype=torch.bfloat16):
    return [torch.zeros(B, H, S, D, dtype=dtype) for _ in range(3)]


def _raises(exc, match, fn, *a, **kw):
    with pytest.raises(exc, match=match):
        fn(*a, **kw)


def test_forward_rejects_a_transposed_view():
    q, k, v = _qkv()
    qt = torch.zeros(B, S, H, D, dtype=torch.bfloat16).transpose(1, 2)        # [B, H, S, D] view, not contiguous
    _raises(ValueError, "contiguous", sta.forward, qt, k, v, GEOM, _index())


def test_forward_rejects_mixed_dtypes_and_shapes():
    q, k, v = _qkv()
    _raises(TypeError, "k is torch.float32", sta.forward, q, k.float(), v, GEOM, _index())
    _raises(ValueError, "shape", sta.forward, q, k[:, :1].contiguous(), v, GEOM, _index())
    _raises(ValueError, r"\[B, H, S, D\]", sta.forward, q[0], k[0], v[0], GEOM, _index())
    _raises(TypeError, "bfloat16 and float32", sta.forward, *(x.half() for x in (q, k, v)), GEOM, _index())


def test_forward_rejects_token_count_and_index_heads():
    q, k, v = (x[:, :, :300].contiguous() for x in _qkv())
    _raises(ValueError, "token axis", sta.forward, q, k, v, GEOM, _index())
    q, k, v = _qkv()
    _raises(ValueError, "list sets", sta.forward, q, k, v, GEOM, _index(heads=3))


def test_forward_rejects_host_tensors_last():
    q, k, v = _qkv()
    _raises(ValueError, "GPU", sta.forward, q, k, v, GEOM, _index())


def test_backward_checks_every_tensor_and_lse():
    q, k, v = _qkv()
    o, do = torch.zeros_like(q), torch.zeros_like(q)
    lse = torch.zeros(B, H, S)
    _raises(ValueError, "dout must be contiguous", sta.backward, q, k, v, o,
            lse, torch.zeros(B, S, H, D, dtype=torch.bfloat16).transpose(1, 2), GEOM, _index())
    _raises(TypeError, "o is torch.float32", sta.backward, q, k, v, o.float(), lse, do, GEOM, _index())
    _raises(ValueError, "lse must be", sta.backward, q, k, v, o, lse.double(), do, GEOM, _index())
    _raises(ValueError, "lse must be", sta.backward, q, k, v, o, lse[:, :, :100], do, GEOM, _index())
    _raises(ValueError, "GPU", sta.backward, q, k, v, o, lse, do, GEOM, _index())


def test_window_shifts_checks_q_and_k():
    q, k, _ = _qkv()
    _raises(TypeError, "k is torch.float32", sta.window_shifts, q, k.float(), GEOM, [(3, 3, 3)] * H, (1, 1, 1))
    _raises(ValueError, "GPU", sta.window_shifts, q, k, GEOM, [(3, 3, 3)] * H, (1, 1, 1))


@pytest.mark.parametrize("bad,exc,match", [
    (torch.zeros(12, 3, dtype=torch.int64), TypeError, "int32"),
    (torch.zeros(11, 3, dtype=torch.int32), ValueError, "T = 12"),
    (torch.zeros(1, 12, 3, dtype=torch.int32), ValueError, "H = 2"),
    (torch.zeros(3, 12, 3, dtype=torch.int32), ValueError, "H = 2"),
    (torch.zeros(2, 1, 12, 3, dtype=torch.int32), ValueError, "H = 2"),
    (torch.zeros(3, 12, dtype=torch.int32).t(), ValueError, "contiguous"),
    (torch.zeros(2, 3, 12, dtype=torch.int32).transpose(1, 2), ValueError, "contiguous"),
    (torch.zeros(12, 3, dtype=torch.int32), ValueError, "offsets are on cpu"),
])
def test_index_rejects_bad_offsets(bad, exc, match):
    _raises(exc, match, sta.StaIndex, GEOM, [(3, 3, 3)] * H, bad)


def test_index_is_built_on_a_gpu_device():
    _raises(ValueError, "GPU device", sta.StaIndex, GEOM, [(3, 3, 3)] * H, None, device="cpu")


def test_attention_function_checks_like_forward():
    q, k, v = _qkv()
    _raises(ValueError, "GPU", sta.attention, q, k, v, GEOM, _index())
    _raises(TypeError, "k is torch.float32", sta.attention, q, k.float(), v, GEOM, _index())


def test_tile_reorder_checks_input_and_out():
    x = torch.zeros(B, H, S, D, dtype=torch.bfloat16)
    _raises(ValueError, r"\[\.\.\., 384, C\]", sta.tile_reorder, x[:, :, :100], GEOM)
    _raises(ValueError, "x must be contiguous", sta.tile_reorder,
            torch.zeros(B, H, D, S, dtype=torch.bfloat16).transpose(2, 3), GEOM)
    # an out smaller than x, of another dtype, or strided would be written past its end or misread
    _raises(ValueError, "out is", sta.tile_reorder, x, GEOM, out=torch.zeros(B, 1, S, D, dtype=torch.bfloat16))
    _raises(ValueError, "out is", sta.tile_reorder, x, GEOM, out=torch.zeros_like(x, dtype=torch.float32))
    _raises(ValueError, "out must be contiguous", sta.tile_reorder, x, GEOM,
            out=torch.zeros(B, H, D, S, dtype=torch.bfloat16).transpose(2, 3))
    _raises(ValueError, "GPU", sta.tile_reorder, x, GEOM)
