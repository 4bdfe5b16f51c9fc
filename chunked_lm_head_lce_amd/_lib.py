"""ctypes view of the C ABI in include/lce.h (liblce.so, built in-tree).

Loading fails loudly when the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblce.so")

LCE_OK = 0
LCE_ERR_INVALID_ARG = 1
LCE_ERR_UNSUPPORTED = 2
LCE_ERR_WORKSPACE = 3
LCE_ERR_HIP = 4
LCE_ERR_LABEL_RANGE = 5
LCE_ERR_TOO_LARGE = 6
LCE_NOALLOC_SCRATCH_BYTES = 64 << 20

LCE_REDUCTION = {"none": 0, "sum": 1, "mean": 2}
LCE_DTYPE_BF16 = 0
LCE_DTYPE_F32 = 1
LCE_WS_FORWARD = 0
LCE_WS_BACKWARD = 1
LCE_WS_BACKWARD_EXTERNAL_F32 = 2

EXPORTED = ("lce_workspace_bytes", "lce_forward", "lce_forward_backward", "lce_forward_traced",
            "lce_forward_backward_traced", "lce_forward_backward_ex", "lce_scale", "lce_status_string",
            "lce_abi_version", "lce_forward_noalloc")

KERNEL_KINDS = ("zero", "prepare_labels", "fwd_lse", "finalize_rows", "finalize_loss", "transpose",
                "bwd_dlogits", "grad_hidden", "grad_weight", "cast", "label_logit", "row_ref", "fwd_retry",
                "bias_sums", "partition", "gather_rows")


class LceProblem(ctypes.Structure):
    _fields_ = [
        ("n_rows", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("vocab", ctypes.c_int64),
        ("ld_hidden", ctypes.c_int64),
        ("ld_weight", ctypes.c_int64),
        ("ignore_index", ctypes.c_int64),
        ("chunk_rows", ctypes.c_int64),
        ("rows_in_flight", ctypes.c_int64),
        ("reduction", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class LceTrace(ctypes.Structure):
    _fields_ = [
        ("events", ctypes.POINTER(ctypes.c_void_p)),
        ("kinds", ctypes.POINTER(ctypes.c_int32)),
        ("capacity", ctypes.c_int32),
        ("count", ctypes.c_int32),
        ("dims", ctypes.POINTER(ctypes.c_int64)),
    ]


class LceBackwardOptions(ctypes.Structure):
    _fields_ = [
        ("row_scale", ctypes.c_void_p),
        ("accumulate", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m chunked_lm_head_lce_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(LceProblem)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    lib.lce_workspace_bytes.argtypes = [P, i32]
    lib.lce_workspace_bytes.restype = sz
    lib.lce_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lce_forward.restype = i32
    lib.lce_forward_backward.argtypes = [P, vp, vp, vp, vp, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         vp, sz, vp]
    lib.lce_forward_backward.restype = i32
    T = ctypes.POINTER(LceTrace)
    lib.lce_forward_traced.argtypes = lib.lce_forward.argtypes + [T]
    lib.lce_forward_traced.restype = i32
    lib.lce_forward_backward_traced.argtypes = lib.lce_forward_backward.argtypes + [T]
    lib.lce_forward_backward_traced.restype = i32
    lib.lce_forward_backward_ex.argtypes = lib.lce_forward_backward.argtypes + [ctypes.POINTER(LceBackwardOptions), T]
    lib.lce_forward_backward_ex.restype = i32
    lib.lce_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.lce_forward_noalloc.restype = i32
    lib.lce_scale.argtypes = [vp, i32, ctypes.c_int64, vp, vp]
    lib.lce_scale.restype = i32
    lib.lce_status_string.argtypes = [i32]
    lib.lce_status_string.restype = ctypes.c_char_p
    lib.lce_abi_version.argtypes = []
    lib.lce_abi_version.restype = i32
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().lce_status_string(code).decode()
