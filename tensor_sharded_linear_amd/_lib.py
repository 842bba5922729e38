"""ctypes declarations of the C interface in include/tp.h (libtp_amd.so, built in-tree).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any kind.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtp_amd.so")

TP_OK = 0
STATUS_NAMES = {
    0: "TP_OK",
    1: "TP_ERR_NULL",
    2: "TP_ERR_DTYPE",
    3: "TP_ERR_SHAPE",
    4: "TP_ERR_INDIVISIBLE",
    5: "TP_ERR_SHARD_RANGE",
    6: "TP_ERR_STRIDE",
    7: "TP_ERR_ALIAS",
    8: "TP_ERR_WORKSPACE",
    9: "TP_ERR_HIP",
    10: "TP_ERR_TOO_LARGE",
}
TP_F32, TP_BF16 = 0, 1
TP_SPLIT_COLS, TP_SPLIT_ROWS, TP_SPLIT_TOKENS = 0, 1, 2
TP_ACT_NONE, TP_ACT_GELU = 0, 1

# Every function the header declares, with its ctypes signature.
EXPORTS = (
    "tp_col_linear",
    "tp_row_linear",
    "tp_reduce_partials",
    "tp_mlp",
    "tp_mlp_noalloc",
    "tp_mlp_noalloc_max_scratch",
    "tp_col_linear_backward",
    "tp_row_linear_backward",
    "tp_mlp_backward",
    "tp_attention",
    "tp_sp_layernorm",
    "tp_status_string",
    "tp_version",
)


class TpMatrix(ctypes.Structure):
    _fields_ = [
        ("ptr", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("ld", ctypes.c_int64),
        ("shard_stride", ctypes.c_int64),
    ]


_M = ctypes.POINTER(TpMatrix)
_lib = None


class TpError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


def load() -> ctypes.CDLL:
    """Load libtp_amd.so once; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m tensor_sharded_linear_amd.build` "
            "(the HIP library is the only implementation)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    lib.tp_col_linear.argtypes = [_M, _M, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _M,
                                  ctypes.c_void_p]
    lib.tp_col_linear.restype = ctypes.c_int32
    lib.tp_row_linear.argtypes = [_M, _M, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _M, ctypes.c_void_p]
    lib.tp_row_linear.restype = ctypes.c_int32
    lib.tp_reduce_partials.argtypes = [_M, ctypes.c_int32, ctypes.c_int32, _M, ctypes.c_void_p]
    lib.tp_reduce_partials.restype = ctypes.c_int32
    lib.tp_mlp.argtypes = [_M, _M, _M, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                           ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t), _M, ctypes.c_void_p]
    lib.tp_mlp.restype = ctypes.c_int32
    lib.tp_mlp_noalloc.argtypes = [_M, _M, _M, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _M,
                                   ctypes.c_void_p]
    lib.tp_mlp_noalloc.restype = ctypes.c_int32
    lib.tp_mlp_noalloc_max_scratch.argtypes = []
    lib.tp_mlp_noalloc_max_scratch.restype = ctypes.c_size_t
    lib.tp_col_linear_backward.argtypes = [_M, _M, _M, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _M, _M,
                                           ctypes.c_void_p]
    lib.tp_col_linear_backward.restype = ctypes.c_int32
    lib.tp_row_linear_backward.argtypes = [_M, _M, _M, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _M, _M,
                                           ctypes.c_void_p]
    lib.tp_row_linear_backward.restype = ctypes.c_int32
    lib.tp_mlp_backward.argtypes = [_M, _M, _M, _M, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t), _M, _M, _M, ctypes.c_void_p]
    lib.tp_mlp_backward.restype = ctypes.c_int32
    lib.tp_attention.argtypes = [_M, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, _M, ctypes.c_void_p]
    lib.tp_attention.restype = ctypes.c_int32
    lib.tp_sp_layernorm.argtypes = [_M, ctypes.c_int32, _M, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    _M, _M, ctypes.c_void_p]
    lib.tp_sp_layernorm.restype = ctypes.c_int32
    lib.tp_status_string.argtypes = [ctypes.c_int32]
    lib.tp_status_string.restype = ctypes.c_char_p
    lib.tp_version.argtypes = []
    lib.tp_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().tp_status_string(int(status)).decode()


def matrix(ptr: int, dtype: int, rows: int, cols: int, ld: int, shard_stride: int = 0) -> TpMatrix:
    return TpMatrix(ctypes.c_void_p(ptr), dtype, 0, rows, cols, ld, shard_stride)


def check(status: int, where: str) -> None:
    if status != TP_OK:
        raise TpError(status, where)
