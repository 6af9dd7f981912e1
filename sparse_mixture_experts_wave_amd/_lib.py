"""ctypes view of libmoe.so (the C ABI in include/moe.h).

Loading fails loudly when the library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = 0, 1, 2, 3
MOE_F32, MOE_BF16 = 0, 1
MOE_TIMING_POINTS = 6


class MoEShape(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("wt", ctypes.c_int32),
    ]


class MoEAttnShape(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("d", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("G", ctypes.c_int32),
        ("d_h", ctypes.c_int32),
        ("act", ctypes.c_int32),
    ]


class MoEExpertBias(ctypes.Structure):
    _fields_ = [("b1", ctypes.c_void_p), ("b3", ctypes.c_void_p), ("b2", ctypes.c_void_p)]


_vp = ctypes.c_void_p
_sp = ctypes.POINTER(MoEShape)
_bp = ctypes.POINTER(MoEExpertBias)
_ap = ctypes.POINTER(MoEAttnShape)

# name -> (restype, argtypes)
SIGNATURES = {
    "moe_workspace_size": (ctypes.c_size_t, [_sp]),
    "moe_expert_ffn_workspace_size": (ctypes.c_size_t, [_sp]),
    "moe_route": (ctypes.c_int, [_sp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_dispatch": (ctypes.c_int, [_sp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "moe_expert_ffn": (ctypes.c_int, [_sp, _vp, _vp, _vp, _vp, _vp, _vp, _bp, _vp, _vp, ctypes.c_size_t, _vp]),
    "moe_combine": (ctypes.c_int, [_sp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_forward": (ctypes.c_int, [_sp, _vp, _vp, _vp, _vp, _vp, _vp, _bp, _vp, _vp, ctypes.c_size_t, _vp]),
    "moe_forward_noalloc": (ctypes.c_int, [_sp, _vp, _vp, _vp, _vp, _vp, _vp, _bp, _vp, _vp]),
    "moe_block_forward": (ctypes.c_int, [_sp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _bp, _vp,
                                         ctypes.c_size_t, _vp]),
    "moe_aux_loss": (ctypes.c_int, [_sp, _vp, ctypes.c_int32, _vp, ctypes.c_float, _vp, _vp, _vp]),
    "moe_attention_workspace_size": (ctypes.c_size_t, [_ap]),
    "moe_gqa_attention": (ctypes.c_int, [_ap, _vp, _vp, _vp, _vp, _vp]),
    "moe_attention_block_forward": (ctypes.c_int, [_ap, _vp, _vp, ctypes.c_float, _vp, _vp, ctypes.c_float,
                                                   ctypes.c_int64, _vp, ctypes.c_size_t, _vp]),
    "moe_set_timing_events": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]),
    "moe_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python -m sparse_mixture_experts_wave_amd.build); there is no CPU fallback")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


def check(status: int) -> None:
    """Raise ValueError (invalid argument), NotImplementedError (unsupported) or MoEError."""
    if status == MOE_OK:
        return
    msg = load().moe_last_error().decode()
    if status == MOE_ERR_INVALID_ARG:
        raise ValueError(msg)
    if status == MOE_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise MoEError(status, msg)
