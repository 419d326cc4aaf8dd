"""ctypes binding of libkivi.so: the C ABI of include/kivi.h, same names.

Argument marshalling only: every computation runs in the library's HIP
kernels.  Loading fails loudly when the library has not been built; there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkivi.so")

KIVI_OK = 0
KIVI_EINVAL = 1
KIVI_ESHAPE = 2
KIVI_EALIGN = 3
KIVI_ECAPACITY = 4
KIVI_EWORKSPACE = 5
KIVI_EUNSUPPORTED = 6
KIVI_EHIP = 7

STATUS_NAMES = {
    0: "KIVI_OK", 1: "KIVI_EINVAL", 2: "KIVI_ESHAPE", 3: "KIVI_EALIGN", 4: "KIVI_ECAPACITY",
    5: "KIVI_EWORKSPACE", 6: "KIVI_EUNSUPPORTED", 7: "KIVI_EHIP",
}


class kivi_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_kv_heads", "gqa_ratio", "head_dim", "bits", "group", "residual",
        "capacity", "meta_half", "outliers")] + [("rope_theta", ctypes.c_float),
                                                  ("deterministic", ctypes.c_int32),
                                                  ("v_window", ctypes.c_int32)]


class kivi_cache(ctypes.Structure):
    _fields_ = [
        ("shape", kivi_shape),
        ("k_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("k_zero", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
        ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
        ("tq", ctypes.c_int32), ("tr", ctypes.c_int32),
        ("k_outliers", ctypes.c_void_p),
    ]


class kivi_ragged_cache(ctypes.Structure):
    _fields_ = [
        ("shape", kivi_shape),
        ("k_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("k_zero", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
        ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
        ("tq", ctypes.POINTER(ctypes.c_int32)), ("tr", ctypes.POINTER(ctypes.c_int32)),
        ("k_outliers", ctypes.c_void_p),
    ]


class kivi_paged_cache(ctypes.Structure):
    _fields_ = [
        ("shape", kivi_shape),
        ("page_tokens", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("k_zero", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
        ("k_res", ctypes.c_void_p), ("v_res", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("tq", ctypes.POINTER(ctypes.c_int32)), ("tr", ctypes.POINTER(ctypes.c_int32)),
        ("k_outliers", ctypes.c_void_p),
    ]


# name -> (restype, argtypes), mirroring include/kivi.h
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_SZP = ctypes.POINTER(ctypes.c_size_t)
_SHP = ctypes.POINTER(kivi_shape)
_CP = ctypes.POINTER(kivi_cache)
_RP = ctypes.POINTER(kivi_ragged_cache)
_I32P = ctypes.POINTER(ctypes.c_int32)
_PP = ctypes.POINTER(kivi_paged_cache)
PROTOTYPES = {
    "kivi_cache_bytes": (ctypes.c_int, [_SHP, _SZP, _SZP, _SZP, _SZP, _SZP, _SZP]),
    "kivi_outlier_bytes": (ctypes.c_int, [_SHP, _i32, _i32, _SZP]),
    "kivi_quantize_k": (ctypes.c_int, [_SHP, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "kivi_quantize_k_outliers": (ctypes.c_int, [_SHP, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                                _vp]),
    "kivi_quantize_v": (ctypes.c_int, [_SHP, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "kivi_prefill": (ctypes.c_int, [_CP, _vp, _vp, _i32, _i32, _vp]),
    "kivi_append": (ctypes.c_int, [_CP, _vp, _vp, _vp]),
    "kivi_decode_auto_splits": (ctypes.c_int, [_CP]),
    "kivi_decode_workspace_bytes": (ctypes.c_size_t, [_SHP, _i32]),
    "kivi_decode_attn": (ctypes.c_int, [_CP, _vp, ctypes.c_float, _vp, _vp, _sz, _i32, _vp]),
    "kivi_append_decode_attn": (ctypes.c_int, [_CP, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _sz,
                                               _i32, _vp]),
    "kivi_decode_attn_noalloc": (ctypes.c_int, [_CP, _vp, ctypes.c_float, _vp, _i32, _vp]),
    "kivi_ragged_prefill": (ctypes.c_int, [_RP, _vp, _vp, _i32, _I32P, _I32P, _vp]),
    "kivi_ragged_append": (ctypes.c_int, [_RP, _vp, _vp, _vp]),
    "kivi_ragged_decode_auto_splits": (ctypes.c_int, [_RP]),
    "kivi_ragged_decode_attn": (ctypes.c_int, [_RP, _vp, ctypes.c_float, _vp, _vp, _sz, _i32, _vp]),
    "kivi_ragged_append_decode_attn": (ctypes.c_int, [_RP, _vp, _vp, _vp, ctypes.c_float, _vp, _vp,
                                                      _sz, _i32, _vp]),
    "kivi_paged_pool_bytes": (ctypes.c_int, [_SHP, _i32, _i32, _SZP, _SZP, _SZP, _SZP]),
    "kivi_paged_prefill": (ctypes.c_int, [_PP, _vp, _vp, _i32, _I32P, _I32P, _vp]),
    "kivi_paged_append": (ctypes.c_int, [_PP, _vp, _vp, _vp]),
    "kivi_paged_decode_auto_splits": (ctypes.c_int, [_PP]),
    "kivi_paged_decode_attn": (ctypes.c_int, [_PP, _vp, ctypes.c_float, _vp, _vp, _sz, _i32, _vp]),
    "kivi_paged_append_decode_attn": (ctypes.c_int, [_PP, _vp, _vp, _vp, ctypes.c_float, _vp, _vp,
                                                     _sz, _i32, _vp]),
    "kivi_strerror": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


class KiviError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS_NAMES.get(status, str(status))
        msg = lib().kivi_strerror(status).decode() if _lib is not None else ""
        super().__init__(f"{where}: {name} ({msg})")


def lib():
    """Load libkivi.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} not found: build it with `python -m kv_cache_bit_kivi_amd.build`")
        # The caller's device memory and streams come from PyTorch, so the
        # library must run on PyTorch's HIP runtime.  PyTorch loads its own
        # copy of libamdhip64 by the unversioned name; loaded first, the
        # library's own dependency (by its versioned soname) would pull in a
        # second HIP runtime that sees no device.  Importing torch first makes
        # the dynamic linker bind the library to torch's copy.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int, where: str) -> None:
    if status != KIVI_OK:
        raise KiviError(status, where)


def _fn(name):
    def call(*args):
        return getattr(lib(), name)(*args)
    call.__name__ = name
    call.__doc__ = f"Direct call of `{name}` from include/kivi.h."
    return call


kivi_cache_bytes = _fn("kivi_cache_bytes")
kivi_outlier_bytes = _fn("kivi_outlier_bytes")
kivi_quantize_k = _fn("kivi_quantize_k")
kivi_quantize_k_outliers = _fn("kivi_quantize_k_outliers")
kivi_quantize_v = _fn("kivi_quantize_v")
kivi_prefill = _fn("kivi_prefill")
kivi_append = _fn("kivi_append")
kivi_decode_auto_splits = _fn("kivi_decode_auto_splits")
kivi_decode_workspace_bytes = _fn("kivi_decode_workspace_bytes")
kivi_decode_attn = _fn("kivi_decode_attn")
kivi_append_decode_attn = _fn("kivi_append_decode_attn")
kivi_decode_attn_noalloc = _fn("kivi_decode_attn_noalloc")
kivi_ragged_prefill = _fn("kivi_ragged_prefill")
kivi_ragged_append = _fn("kivi_ragged_append")
kivi_ragged_decode_auto_splits = _fn("kivi_ragged_decode_auto_splits")
kivi_ragged_decode_attn = _fn("kivi_ragged_decode_attn")
kivi_ragged_append_decode_attn = _fn("kivi_ragged_append_decode_attn")
kivi_paged_pool_bytes = _fn("kivi_paged_pool_bytes")
kivi_paged_prefill = _fn("kivi_paged_prefill")
kivi_paged_append = _fn("kivi_paged_append")
kivi_paged_decode_auto_splits = _fn("kivi_paged_decode_auto_splits")
kivi_paged_decode_attn = _fn("kivi_paged_decode_attn")
kivi_paged_append_decode_attn = _fn("kivi_paged_append_decode_attn")
kivi_strerror = _fn("kivi_strerror")
