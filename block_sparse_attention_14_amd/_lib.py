"""ctypes loader of libsolattn.so (the C ABI declared in include/sol_attn.h)."""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsolattn.so")

SOL_OK = 0
SOL_EINVAL = -1
SOL_EUNSUPPORTED = -2
SOL_EWORKSPACE = -3
SOL_EHIP = -4
SOL_ESCRATCH = -5

SOL_F_POOLED = 1 << 0
SOL_F_EXACT_ONLY = 1 << 1
SOL_F_PLANNED = 1 << 2
SOL_F_ROW_CORRECTION = 1 << 3
SOL_F_OUT_BF16 = 1 << 4
SOL_F_GROUP2 = 1 << 5
SOL_F_GROUP4 = 2 << 5
SOL_F_GROUP8 = 3 << 5
SOL_F_GROUP16 = 1 << 8
SOL_F_GROUP6 = 1 << 9
SOL_F_PREPARED = 1 << 7

SOL_ROUTE_ROWMAX = 0
SOL_ROUTE_GAUSS = 1
SOL_ROUTE_GAUSS_DIAG = 2

SOL_ATTN_MAX_N = 4096 * 64
SOL_ATTN_SCRATCH_BYTES = 128 << 20

EXPORTS = (
    "sol_attn_workspace_bytes",
    "sol_attn_pool",
    "sol_attn_plan",
    "sol_attn_prepare",
    "sol_attn_forward",
    "sol_attn_forward_ex",
    "sol_attn_forward_debug",
    "sol_attn_mask_workspace_bytes",
    "sol_attn_mask_threshold",
    "sol_attn_mask_topk",
    "sol_attn_mask_topp",
    "sol_attn_forward_noalloc",
    "sol_attn_strerror",
)


class SolAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


class sol_attn_stats(ctypes.Structure):
    _fields_ = [
        ("kept_blocks", ctypes.c_ulonglong),
        ("total_blocks", ctypes.c_ulonglong),
        ("kept_pairs", ctypes.c_ulonglong),
        ("min_kept", ctypes.c_uint),
        ("max_kept", ctypes.c_uint),
    ]


class sol_attn_route(ctypes.Structure):
    _fields_ = [
        ("rule", ctypes.c_int),
        ("tau", ctypes.c_float),
        ("beta", ctypes.c_float),
        ("sink_first", ctypes.c_int),
        ("sink_count", ctypes.c_int),
    ]


_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_fwd_args = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.c_float, ctypes.c_uint, _vp,
             _vp, _vp, _vp, ctypes.c_size_t, _vp]


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        f"{LIB_PATH} is missing: build it with "
                        "`python -m block_sparse_attention_14_amd.build` before use"
                    )
                L = ctypes.CDLL(LIB_PATH)
                L.sol_attn_workspace_bytes.argtypes = [_i] * 6
                L.sol_attn_workspace_bytes.restype = ctypes.c_size_t
                L.sol_attn_pool.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
                L.sol_attn_pool.restype = _i
                L.sol_attn_plan.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.c_float, _vp, ctypes.c_size_t, _vp]
                L.sol_attn_plan.restype = _i
                L.sol_attn_prepare.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.c_uint, _vp,
                                               ctypes.c_size_t, _vp]
                L.sol_attn_prepare.restype = _i
                L.sol_attn_forward.argtypes = _fwd_args
                L.sol_attn_forward.restype = _i
                L.sol_attn_forward_ex.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                                  ctypes.POINTER(sol_attn_route), ctypes.c_uint, _vp, _vp, _vp, _vp,
                                                  ctypes.c_size_t, _vp, _vp]
                L.sol_attn_forward_ex.restype = _i
                L.sol_attn_forward_debug.argtypes = _fwd_args + [_vp]
                L.sol_attn_forward_debug.restype = _i
                L.sol_attn_mask_workspace_bytes.argtypes = [_i] * 6
                L.sol_attn_mask_workspace_bytes.restype = ctypes.c_size_t
                L.sol_attn_mask_threshold.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _i,
                                                      ctypes.POINTER(sol_attn_route), _vp, _vp, ctypes.c_size_t,
                                                      _vp]
                L.sol_attn_mask_threshold.restype = _i
                L.sol_attn_mask_topk.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, ctypes.c_size_t, _vp]
                L.sol_attn_mask_topk.restype = _i
                L.sol_attn_mask_topp.argtypes = [_vp, _vp, _i, _i, _i, _i, _i, _i, ctypes.c_float, _vp, _vp,
                                                 ctypes.c_size_t, _vp]
                L.sol_attn_mask_topp.restype = _i
                L.sol_attn_forward_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                                       ctypes.POINTER(sol_attn_route), ctypes.c_uint, _vp, _vp, _vp]
                L.sol_attn_forward_noalloc.restype = _i
                L.sol_attn_strerror.argtypes = [_i]
                L.sol_attn_strerror.restype = ctypes.c_char_p
                _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().sol_attn_strerror(int(code)).decode()


def check(code: int, where: str) -> None:
    if code != SOL_OK:
        raise SolAttnError(code, where)
