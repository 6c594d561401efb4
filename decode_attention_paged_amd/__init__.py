"""Paged split-KV decode attention for MI355X (gfx950).

A thin binding over libpa_decode.so: every step of the computation runs in
the library's HIP kernels; this module only checks tensors, sizes the
workspace (a torch allocation) and passes pointers and the current stream.

Layouts (see include/pa_decode.h):
    q            [B][Hq][D], or [B][q_len][Hq][D] for several query rows
                 (the sequence's last q_len tokens, causal)  float32 or bfloat16
    k_cache      [num_blocks][Hkv][bs][D]
    v_cache      [num_blocks][Hkv][D][bs]
    kv_cache     [num_blocks][bs][Dqk]      (MLA latent; values = first Dv entries)
    block_table  [B][max_blocks_per_seq]    int32
    context_lens [B]                        int32
"""

from __future__ import annotations

import ctypes
import weakref

import torch

from . import _lib
from ._lib import PaError, PaShape  # noqa: F401

__all__ = [
    "decode", "decode_mla", "decode_partial", "decode_mla_partial", "reduce",
    "append_kv", "append_latent", "choose_num_splits", "decode_launches", "workspace_size",
    "workspace_init", "make_shape", "PaError", "library_path", "stream_read",
]

_DTYPES = {torch.float32: _lib.PA_F32, torch.bfloat16: _lib.PA_BF16}
# cache dtypes: the query's, or FP8 E4M3 codes (with bf16 queries and per-tensor scales)
_FP8 = getattr(torch, "float8_e4m3fn", None)


def library_path() -> str:
    return _lib.LIB_PATH


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def make_shape(*, batch, num_q_heads, num_kv_heads, head_dim, head_dim_v, block_size,
               max_blocks_per_seq, num_blocks, max_context_len, scale, dtype, q_len=1,
               kv_dtype=0, k_scale=1.0, v_scale=1.0) -> PaShape:
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    if isinstance(kv_dtype, torch.dtype):
        kv_dtype = _lib.PA_FP8_E4M3 if kv_dtype == _FP8 else _DTYPES[kv_dtype]
    return PaShape(batch, num_q_heads, num_kv_heads, head_dim, head_dim_v, block_size,
                   max_blocks_per_seq, num_blocks, int(max_context_len), float(scale), code,
                   int(q_len), int(kv_dtype), float(k_scale), float(v_scale))


def _kv_dtype(cache, q_dtype, k_scale, v_scale):
    """(kv_dtype code, k_scale, v_scale) for a cache tensor."""
    if _FP8 is not None and cache.dtype == _FP8:
        if k_scale is None or v_scale is None:
            raise ValueError("FP8 caches need k_scale and v_scale")
        return _lib.PA_FP8_E4M3, float(k_scale), float(v_scale)
    if cache.dtype != q_dtype:
        raise ValueError(f"cache dtype {cache.dtype} differs from the query's {q_dtype}")
    return 0, 1.0, 1.0


def _q_dims(q):
    """(B, q_len, Hq, D) of a [B][Hq][D] or [B][q_len][Hq][D] query tensor."""
    if q.dim() == 3:
        B, Hq, D = q.shape
        return B, 1, Hq, D
    if q.dim() == 4:
        return tuple(q.shape)
    raise ValueError("q must be [B][Hq][D] or [B][q_len][Hq][D]")


def _mha_shape(q, k_cache, v_cache, block_table, context_lens, max_context_len, scale,
               k_scale=None, v_scale=None):
    _need(q, "q")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _need(k_cache, "k_cache", None, 4, dev)
    _need(v_cache, "v_cache", k_cache.dtype, 4, dev)
    kvd, ks, vs = _kv_dtype(k_cache, q.dtype, k_scale, v_scale)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, L, Hq, D = _q_dims(q)
    nb, Hkv, bs, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("k_cache head dim differs from q")
    if tuple(v_cache.shape[:2]) != (nb, Hkv) or v_cache.shape[3] != bs:
        raise ValueError("v_cache must be [num_blocks][Hkv][Dv][bs]")
    if block_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_table / context_lens batch differs from q")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    if scale is None:
        scale = D ** -0.5
    return make_shape(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                      head_dim_v=v_cache.shape[2], block_size=bs,
                      max_blocks_per_seq=block_table.shape[1], num_blocks=nb,
                      max_context_len=max_context_len, scale=scale, dtype=q.dtype, q_len=L,
                      kv_dtype=kvd, k_scale=ks, v_scale=vs)


def _mla_shape(q, kv_cache, block_table, context_lens, max_context_len, scale, head_dim_v,
               k_scale=None, v_scale=None):
    _need(q, "q")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    _need(kv_cache, "kv_cache", None, 3, dev)
    kvd, ks, vs = _kv_dtype(kv_cache, q.dtype, k_scale, v_scale)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, L, Hq, D = _q_dims(q)
    nb, bs, Dc = kv_cache.shape
    if Dc != D:
        raise ValueError("kv_cache width differs from q")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    return make_shape(batch=B, num_q_heads=Hq, num_kv_heads=1, head_dim=D, head_dim_v=head_dim_v,
                      block_size=bs, max_blocks_per_seq=block_table.shape[1], num_blocks=nb,
                      max_context_len=max_context_len, scale=scale, dtype=q.dtype, q_len=L,
                      kv_dtype=kvd, k_scale=ks, v_scale=vs)


def choose_num_splits(shape: PaShape, num_cus: int = 0, mla: bool = False) -> int:
    s = _lib.load().pa_choose_num_splits(ctypes.byref(shape), int(num_cus), int(mla))
    if s <= 0:
        raise PaError(_lib.PA_ERR_INVALID, "pa_choose_num_splits")
    return s


def decode_launches(shape: PaShape, num_splits: int = 0, mla: bool = False) -> int:
    """Kernel launches one decode call makes (1: fused or a single split; 2: + reduction)."""
    n = _lib.load().pa_decode_launches(ctypes.byref(shape), int(num_splits), int(mla))
    if n <= 0:
        raise PaError(_lib.PA_ERR_INVALID, "pa_decode_launches")
    return n


def workspace_size(shape: PaShape, num_splits: int = 0, mla: bool = False) -> int:
    return int(_lib.load().pa_decode_workspace_size(ctypes.byref(shape), int(num_splits), int(mla)))


# Arrival counters of the in-kernel merge: the first 4 bytes per row (R = B x
# q_len x Hq rows) of a workspace, which must be zero when a pa_decode call
# that merges in-kernel starts.  Each completed call leaves its own counters
# zero, but its partials follow its own R counters and may overwrite the
# counters of a larger R.  For each workspace tensor this binding has used:
# (weak reference, rows whose counters are known to be zero).
_WS_ZERO_ROWS = {}


def _rows(shape):
    return shape.batch * max(1, shape.q_len) * shape.num_q_heads


def _zero_rows(ws):
    ent = _WS_ZERO_ROWS.get(id(ws))
    return ent[1] if ent is not None and ent[0]() is ws else 0


def _note_workspace(ws, rows):
    """Record that a call with `rows` rows used `ws` (counters past them may be overwritten)."""
    if ws is not None:
        _WS_ZERO_ROWS[id(ws)] = (weakref.ref(ws), min(rows, _zero_rows(ws)))


def _outputs(shape, q, out, lse, workspace, num_splits, mla):
    B, Hq, Dv = shape.batch, shape.num_q_heads, shape.head_dim_v
    rows = (B, Hq) if q.dim() == 3 else (B, q.shape[1], Hq)
    if out is None:
        out = torch.empty(rows + (Dv,), dtype=q.dtype, device=q.device)
    else:
        _need(out, "out", q.dtype, q.dim(), q.device)
        if tuple(out.shape) != rows + (Dv,):
            raise ValueError("out must be [B][Hq][Dv] (or [B][q_len][Hq][Dv])")
    if lse is None:
        lse = torch.empty(rows, dtype=torch.float32, device=q.device)
    elif lse is not False:
        _need(lse, "lse", torch.float32, q.dim() - 1, q.device)
        if tuple(lse.shape) != rows:
            raise ValueError("lse must be [B][Hq] (or [B][q_len][Hq])")
    need = workspace_size(shape, num_splits, mla)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        # zero-filled: the fused reduction's arrival counters must start at 0
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
        _WS_ZERO_ROWS[id(workspace)] = (weakref.ref(workspace), _rows(shape))
    return out, (None if lse is False else lse), workspace


def decode(q, k_cache, v_cache, block_table, context_lens, *, max_context_len=None, scale=None,
           num_splits=0, out=None, lse=None, workspace=None, stream=None, k_scale=None,
           v_scale=None):
    """Decode attention over a paged K/V cache (MHA/GQA).  Returns (out, lse).

    num_splits <= 0 lets the library choose.  Pass lse=False to skip it.
    FP8 caches (torch.float8_e4m3fn, bf16 q) need k_scale and v_scale: a key
    is k_scale times its code's value, a value v_scale times its code's.
    """
    shape = _mha_shape(q, k_cache, v_cache, block_table, context_lens, max_context_len, scale,
                       k_scale, v_scale)
    out, lse, ws = _outputs(shape, q, out, lse, workspace, num_splits, False)
    rows = _rows(shape)
    if (ws is not None and _zero_rows(ws) < rows and workspace_size(shape, num_splits) > 0
            and decode_launches(shape, num_splits) == 1):
        # an in-kernel merge over counters not known to be zero: zero them first
        workspace_init(shape, ws, num_splits, False, stream)
    _note_workspace(ws, rows)
    st = _lib.load().pa_decode(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_table), _ptr(context_lens), int(num_splits), _ptr(out),
                               _ptr(lse), _ptr(ws), _nbytes(ws),
                               _stream(stream))
    _lib.check(st, "pa_decode")
    return out, lse


def decode_mla(q, kv_cache, block_table, context_lens, *, max_context_len=None, scale=None,
               head_dim_v=512, num_splits=0, out=None, lse=None, workspace=None, stream=None,
               k_scale=None, v_scale=None):
    """MLA latent decode: keys = latent rows, values = their first head_dim_v entries.

    An FP8 latent cache (torch.float8_e4m3fn, bf16 q) needs k_scale and
    v_scale: a key is k_scale times the row's values, a value v_scale times
    its first head_dim_v.
    """
    if scale is None:
        raise ValueError("MLA needs an explicit scale")
    shape = _mla_shape(q, kv_cache, block_table, context_lens, max_context_len, scale, head_dim_v,
                       k_scale, v_scale)
    out, lse, ws = _outputs(shape, q, out, lse, workspace, num_splits, True)
    _note_workspace(ws, _rows(shape))
    st = _lib.load().pa_decode_mla(ctypes.byref(shape), _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                   _ptr(context_lens), int(num_splits), _ptr(out), _ptr(lse),
                                   _ptr(ws), _nbytes(ws), _stream(stream))
    _lib.check(st, "pa_decode_mla")
    return out, lse


def workspace_init(shape: PaShape, workspace, num_splits: int = 0, mla: bool = False, stream=None):
    """Zero the workspace's arrival counters (needed once per new workspace)."""
    st = _lib.load().pa_workspace_init(ctypes.byref(shape), int(num_splits), int(mla),
                                       _ptr(workspace), _nbytes(workspace), _stream(stream))
    _lib.check(st, "pa_workspace_init")
    if workspace is not None:
        _WS_ZERO_ROWS[id(workspace)] = (weakref.ref(workspace), _rows(shape))


def decode_partial(shape: PaShape, q, k_cache, v_cache, block_table, context_lens, num_splits,
                   out, lse, workspace, stream=None):
    """Only the per-split partial step (writes out/lse directly when S == 1)."""
    _note_workspace(workspace, _rows(shape))
    st = _lib.load().pa_decode_partial(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(block_table), _ptr(context_lens), int(num_splits),
                                       _ptr(out), _ptr(lse), _ptr(workspace),
                                       _nbytes(workspace),
                                       _stream(stream))
    _lib.check(st, "pa_decode_partial")


def decode_mla_partial(shape: PaShape, q, kv_cache, block_table, context_lens, num_splits, out,
                       lse, workspace, stream=None):
    _note_workspace(workspace, _rows(shape))
    st = _lib.load().pa_decode_mla_partial(ctypes.byref(shape), _ptr(q), _ptr(kv_cache),
                                           _ptr(block_table), _ptr(context_lens), int(num_splits),
                                           _ptr(out), _ptr(lse), _ptr(workspace),
                                           _nbytes(workspace),
                                           _stream(stream))
    _lib.check(st, "pa_decode_mla_partial")


def reduce(shape: PaShape, context_lens, num_splits, workspace, out, lse, mla=False, stream=None):
    """Only the log-sum-exp weighted merge of the split partials."""
    st = _lib.load().pa_reduce(ctypes.byref(shape), _ptr(context_lens), int(num_splits), int(mla),
                               _ptr(workspace), _nbytes(workspace),
                               _ptr(out), _ptr(lse), _stream(stream))
    _lib.check(st, "pa_reduce")


def append_kv(k_new, v_new, k_cache, v_cache, block_table, context_lens, stream=None):
    """Write one new token per sequence into the paged K/V cache.

    k_new [B][Hkv][D], v_new [B][Hkv][Dv] (in the caches' dtype: FP8 codes for
    FP8 caches, quantised by the caller); the token goes to position
    context_lens[b] (the length before the append).  context_lens is not
    changed: the caller increments it before decoding the new token.
    """
    _need(k_new, "k_new", ndim=3)
    fp8 = _FP8 is not None and k_new.dtype == _FP8
    if k_new.dtype not in _DTYPES and not fp8:
        raise ValueError(f"unsupported dtype {k_new.dtype}")
    dev = k_new.device
    _need(v_new, "v_new", k_new.dtype, 3, dev)
    _need(k_cache, "k_cache", k_new.dtype, 4, dev)
    _need(v_cache, "v_cache", k_new.dtype, 4, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, Hkv, D = k_new.shape
    nb, Hk, bs, Dk = k_cache.shape
    Dv = v_new.shape[2]
    if (Hk, Dk) != (Hkv, D) or tuple(v_new.shape[:2]) != (B, Hkv):
        raise ValueError("k_new / v_new do not match the cache heads or dims")
    if tuple(v_cache.shape) != (nb, Hkv, Dv, bs):
        raise ValueError("v_cache must be [num_blocks][Hkv][Dv][bs]")
    if block_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_table / context_lens batch differs from k_new")
    # FP8 rows are moved as codes (a bf16 shape with FP8 caches: one byte per element)
    shape = make_shape(batch=B, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D, head_dim_v=Dv,
                       block_size=bs, max_blocks_per_seq=block_table.shape[1], num_blocks=nb,
                       max_context_len=0, scale=1.0,
                       dtype=torch.bfloat16 if fp8 else k_new.dtype,
                       kv_dtype=_lib.PA_FP8_E4M3 if fp8 else 0)
    st = _lib.load().pa_append_kv(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(block_table), _ptr(context_lens),
                                  _stream(stream))
    _lib.check(st, "pa_append_kv")


def append_latent(c_new, kv_cache, block_table, context_lens, stream=None):
    """MLA: write one new latent row per sequence (c_new [B][D]) into the paged cache
    (FP8 codes for an FP8 cache, quantised by the caller)."""
    _need(c_new, "c_new", ndim=2)
    fp8 = _FP8 is not None and c_new.dtype == _FP8
    if c_new.dtype not in _DTYPES and not fp8:
        raise ValueError(f"unsupported dtype {c_new.dtype}")
    dev = c_new.device
    _need(kv_cache, "kv_cache", c_new.dtype, 3, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(context_lens, "context_lens", torch.int32, 1, dev)
    B, D = c_new.shape
    nb, bs, Dc = kv_cache.shape
    if Dc != D:
        raise ValueError("c_new width differs from kv_cache")
    if block_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_table / context_lens batch differs from c_new")
    shape = make_shape(batch=B, num_q_heads=1, num_kv_heads=1, head_dim=D, head_dim_v=D,
                       block_size=bs, max_blocks_per_seq=block_table.shape[1], num_blocks=nb,
                       max_context_len=0, scale=1.0,
                       dtype=torch.bfloat16 if fp8 else c_new.dtype,
                       kv_dtype=_lib.PA_FP8_E4M3 if fp8 else 0)
    st = _lib.load().pa_append_latent(ctypes.byref(shape), _ptr(c_new), _ptr(kv_cache),
                                      _ptr(block_table), _ptr(context_lens), _stream(stream))
    _lib.check(st, "pa_append_latent")


def stream_read(src, sink, stream=None):
    """Measurement helper: stream-read every byte of the device tensor `src`
    (size a multiple of 16) with the KV gather's load form; `sink` is a
    one-word device tensor (int32/uint32), written only in a practically
    impossible case."""
    _need(src, "src")
    _need(sink, "sink", device=src.device)
    if _nbytes(sink) < 4:
        raise ValueError("sink must hold one 32-bit word")
    st = _lib.load().pa_stream_read(_ptr(src), _nbytes(src), _ptr(sink), _stream(stream))
    _lib.check(st, "pa_stream_read")
