"""ctypes view of libra.so, the C-ABI declared in include/ra.h.

Loading fails loudly when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libra.so")

RA_OK = 0
RA_ERR_INVALID_ARG = -1
RA_ERR_UNSUPPORTED = -2
RA_ERR_WORKSPACE = -3
RA_ERR_HIP = -4

RA_LAYOUT = {"contiguous": 0, "striped": 1, "zigzag": 2}
RA_F32, RA_BF16 = 0, 1
RA_MAX_TIMED_STEPS = 64
RA_NOALLOC_SCRATCH_BYTES = 64 << 20


class RaProblem(ctypes.Structure):
    _fields_ = [
        ("b", ctypes.c_int32), ("L", ctypes.c_int32), ("h", ctypes.c_int32),
        ("n_kv", ctypes.c_int32), ("d", ctypes.c_int32), ("N", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("layout", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("doc_begin", ctypes.c_void_p), ("doc_end", ctypes.c_void_p),
        ("steps_per_launch", ctypes.c_int32),
    ]


class RaRingTiming(ctypes.Structure):
    _fields_ = [
        ("n_steps", ctypes.c_int32),
        ("step_begin_ms", ctypes.c_float * RA_MAX_TIMED_STEPS),
        ("step_end_ms", ctypes.c_float * RA_MAX_TIMED_STEPS),
        ("copy_begin_ms", ctypes.c_float * RA_MAX_TIMED_STEPS),
        ("copy_end_ms", ctypes.c_float * RA_MAX_TIMED_STEPS),
        ("total_ms", ctypes.c_float),
        ("launch_steps", ctypes.c_int32 * RA_MAX_TIMED_STEPS),
    ]


class RaUlyssesTiming(ctypes.Structure):
    _fields_ = [("gather_ms", ctypes.c_float), ("attend_ms", ctypes.c_float),
                ("scatter_ms", ctypes.c_float), ("total_ms", ctypes.c_float)]


class RaUspTiming(ctypes.Structure):
    _fields_ = [("others_gather_ms", ctypes.c_float), ("gather_ms", ctypes.c_float),
                ("ring_ms", ctypes.c_float), ("scatter_ms", ctypes.c_float), ("total_ms", ctypes.c_float)]


# (name, restype, argtypes) of every exported entry point, in include/ra.h order.
_P = ctypes.POINTER(RaProblem)
_V = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t
SIGNATURES = [
    ("ra_step_fwd", _I, [_P, _I, _I, _V, _V, _V, _V, _V, _V]),
    ("ra_merge_lse", _I, [_P, _V, _V, _V, _V, _V]),
    ("ra_finalize", _I, [_P, _V, _V, _V]),
    ("ra_ring_fwd_workspace", _S, [_P]),
    ("ra_fwd_step_plan", _I, [_P, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I), _I, ctypes.POINTER(_I),
                              ctypes.POINTER(_I)]),
    ("ra_ring_fwd", _I, [_P, _I, _V, _V, _V, _V, _V, _V, _S, _V, _V]),
    ("ra_ring_fwd_timed", _I, [_P, _I, _V, _V, _V, _V, _V, _V, _S, _V, _V,
                               ctypes.POINTER(RaRingTiming)]),
    ("ra_ring_fwd_noalloc", _I, [_P, _I, _V, _V, _V, _V, _V, _V, _V]),
    ("ra_bwd_preprocess", _I, [_P, _V, _V, _V, _V]),
    ("ra_step_bwd", _I, [_P, _I, _I, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V]),
    ("ra_ring_bwd_workspace", _S, [_P]),
    ("ra_ring_bwd_workspace_min", _S, [_P]),
    ("ra_ring_bwd", _I, [_P, _I, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _S, _V, _V]),
    ("ra_ring_bwd_timed", _I, [_P, _I, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _S, _V, _V,
                               ctypes.POINTER(RaRingTiming)]),
    ("ra_ring_bwd_kv_stationary_workspace", _S, [_P]),
    ("ra_ring_bwd_kv_stationary", _I, [_P, _I, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _S, _V, _V]),
    ("ra_ulysses_fwd_workspace", _S, [_P]),
    ("ra_ulysses_fwd", _I, [_P, _I, _V, _V, _V, _V, _V, _V, _S, _V]),
    ("ra_ulysses_fwd_timed", _I, [_P, _I, _V, _V, _V, _V, _V, _V, _S, _V,
                                  ctypes.POINTER(RaUlyssesTiming)]),
    ("ra_ulysses_bwd_workspace", _S, [_P]),
    ("ra_ulysses_bwd", _I, [_P, _I, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _S, _V]),
    ("ra_usp_fwd_workspace", _S, [_P, _I]),
    ("ra_usp_fwd", _I, [_P, _I, _I, _I, _V, _V, _V, _V, _V, _V, _S, _V, _V]),
    ("ra_usp_fwd_timed", _I, [_P, _I, _I, _I, _V, _V, _V, _V, _V, _V, _S, _V, _V,
                              ctypes.POINTER(RaUspTiming)]),
    ("ra_allowed_pairs", ctypes.c_int64, [_P, _I, _I]),
    ("ra_allowed_pairs_packed", ctypes.c_int64, [_P, _I, _I, _V, _V]),
    ("ra_document_ranges", _I, [_P, _I, _V, _I, _V, _V]),
    ("ra_status_string", ctypes.c_char_p, [_I]),
    ("ra_last_error", ctypes.c_char_p, []),
]

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libra.so (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m ring_attention_long_amd.build` "
                "(there is no non-HIP fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class RaError(RuntimeError):
    def __init__(self, status: int, where: str):
        L = lib()
        self.status = status
        self.detail = (L.ra_last_error() or b"").decode()
        super().__init__(f"{where}: {L.ra_status_string(status).decode()} ({self.detail})")


def check(status: int, where: str) -> None:
    if status != RA_OK:
        raise RaError(status, where)
