"""ctypes view of libpa_decode.so (declarations mirror include/pa_decode.h)."""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa_decode.so")

PA_OK = 0
PA_ERR_INVALID = 1
PA_ERR_UNSUPPORTED = 2
PA_ERR_WORKSPACE = 3
PA_ERR_HIP = 4
PA_ERR_SCRATCH = 5

PA_F32 = 0
PA_BF16 = 1
PA_FP8_E4M3 = 2


class PaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_context_len", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


_P = ctypes.c_void_p
_SH = ctypes.POINTER(PaShape)
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); every function the header declares
SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [_I32]),
    "pa_version": (_I32, []),
    "pa_choose_num_splits": (_I32, [_SH, _I32, _I32]),
    "pa_decode_launches": (_I32, [_SH, _I32, _I32]),
    "pa_decode_workspace_size": (_SZ, [_SH, _I32, _I32]),
    "pa_workspace_init": (_I32, [_SH, _I32, _I32, _P, _SZ, _P]),
    "pa_decode": (_I32, [_SH, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "pa_decode_static": (_I32, [_SH, _P, _P, _P, _P, _P, _I32, _P, _P, _P]),
    "pa_decode_mla": (_I32, [_SH, _P, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "pa_decode_partial": (_I32, [_SH, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "pa_decode_mla_partial": (_I32, [_SH, _P, _P, _P, _P, _I32, _P, _P, _P, _SZ, _P]),
    "pa_reduce": (_I32, [_SH, _P, _I32, _I32, _P, _SZ, _P, _P, _P]),
    "pa_append_kv": (_I32, [_SH, _P, _P, _P, _P, _P, _P, _P]),
    "pa_append_latent": (_I32, [_SH, _P, _P, _P, _P, _P]),
    "pa_stream_read": (_I32, [_P, _SZ, _P, _P]),
}

_lib = None


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m decode_attention_paged_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().pa_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != PA_OK:
        raise PaError(status, where)
