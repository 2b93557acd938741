"""ctypes view of the C ABI declared in include/fa_mi355x.h.

Loads the in-tree ``libfa_mi355x.so`` (built by ``build.py``).  There is no
fallback: if the library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa_mi355x.so")

(FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE_TOO_SMALL, FA_ERR_HIP, FA_ERR_SCRATCH_LIMIT,
 FA_ERR_COMPILE) = range(7)
FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_MOD_NONE, FA_MOD_ALIBI, FA_MOD_CHECKERBOARD, FA_MOD_CUSTOM = 0, 1, 2, 3
FA_DQ_AUTO, FA_DQ_SEPARATE, FA_DQ_ATOMIC = 0, 1, 2
FA_MAX_KV_SPLITS = 256

# every function the header declares, with (restype, argtypes)
_c_void_p = ctypes.c_void_p


class FaProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("seq_q", ctypes.c_int64),
        ("seq_kv", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
        ("mod_kind", ctypes.c_int32), ("alibi_slopes", _c_void_p),
        ("checker_even", ctypes.c_float), ("checker_odd", ctypes.c_float),
        ("key_mask", _c_void_p), ("q_offset", ctypes.c_int64),
        ("block_mask", _c_void_p),
        ("dq_mode", ctypes.c_int32), ("kv_splits", ctypes.c_int32),
        ("custom_mod", _c_void_p), ("mod_params", _c_void_p),
    ]

FA_ABI_VERSION = 7
FA_BLOCK_MASK_BLOCK = 128
FA_BLOCK_MASK_MAX_SEQ = 131072
FA_DECODE_SCRATCH_BYTES = 16 << 20


_P = ctypes.POINTER(FaProblem)
SIGNATURES = {
    "fa_forward": (ctypes.c_int, [_P, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "fa_forward_split_workspace_size": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
    "fa_forward_split": (ctypes.c_int, [_P] + [_c_void_p] * 6 + [ctypes.c_size_t, _c_void_p]),
    "fa_backward_workspace_size": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
    "fa_backward": (ctypes.c_int, [_P] + [_c_void_p] * 10 + [ctypes.c_size_t, _c_void_p]),
    "fa_decode_workspace_size": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
    "fa_decode": (ctypes.c_int, [_P] + [_c_void_p] * 6 + [ctypes.c_size_t, _c_void_p]),
    "fa_decode_noalloc": (ctypes.c_int, [_P] + [_c_void_p] * 6),
    "fa_score_mod_create": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(_c_void_p), ctypes.c_char_p,
                                           ctypes.c_size_t]),
    "fa_score_mod_destroy": (ctypes.c_int, [_c_void_p]),
    "fa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fa_abi_version": (ctypes.c_int, []),
}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = load().fa_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} (status {status})" + (f"\n{detail}" if detail else ""))


def load() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m tiled_online_softmax_flashattention_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaError(status, where)
