"""ctypes view of libsharq.so (the C ABI declared in include/sharq.h).

Argument marshalling only: every step of the SharQ hot path runs in the HIP
kernels behind these symbols.  Loading fails loudly when the library has not
been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

# SHARQ_LIBRARY selects another build of the same library (the tile-timeline
# build, libsharq_timeline.so); by default the in-tree libsharq.so
LIB_PATH = os.environ.get("SHARQ_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsharq.so")

SHARQ_OK = 0
SHARQ_ERR_INVALID_ARGUMENT = 1
SHARQ_ERR_UNSUPPORTED_SHAPE = 2
SHARQ_ERR_FORMAT_MISMATCH = 3
SHARQ_ERR_WORKSPACE_TOO_SMALL = 4
SHARQ_ERR_HIP = 5

SHARQ_MXFP4 = 0
SHARQ_NVFP4_EMU = 1
SHARQ_MXFP4_24 = 2          # activations only: MXFP4 with the 2:4 element-wise backbone
SHARQ_F32 = 0
SHARQ_BF16 = 1

FORMATS = {"mxfp4": SHARQ_MXFP4, "nvfp4": SHARQ_NVFP4_EMU, "mxfp4_24": SHARQ_MXFP4_24}

# every entry point include/sharq.h declares
EXPORTS = ("sharq_weight_sizes", "sharq_act_sizes", "sharq_pack_weight", "sharq_prepare", "sharq_prepare_no_alloc",
           "sharq_linear",
           "sharq_prepare_linear", "sharq_prepare_linear_status", "sharq_rmsnorm", "sharq_quantize_mx", "sharq_linear_dense",
           "sharq_timeline_records", "sharq_timeline_clear", "sharq_timeline_read",
           "sharq_status_string", "sharq_last_error")


class SharqWeight(ctypes.Structure):
    _fields_ = [("fmt", c_int32), ("K", c_int32), ("D", c_int32), ("n_groups", c_int32),
                ("payload", c_void_p), ("scale_sp", c_void_p), ("scale_dn", c_void_p),
                ("tensor_scale", c_void_p)]


class SharqAct(ctypes.Structure):
    _fields_ = [("fmt", c_int32), ("T", c_int32), ("K", c_int32),
                ("bb_codes", c_void_p), ("bb_meta", c_void_p), ("bb_scale", c_void_p),
                ("res_codes", c_void_p), ("res_scale", c_void_p), ("tensor_scales", c_void_p)]


class SharqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparsity_sharq_prepare_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.sharq_weight_sizes.argtypes = [c_int32, c_int32, c_int32, c_int32, POINTER(c_size_t)]
        L.sharq_act_sizes.argtypes = [c_int32, c_int32, c_int32, POINTER(c_size_t)]
        L.sharq_pack_weight.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int64, c_int64,
                                        POINTER(SharqWeight), c_void_p, c_size_t, c_void_p]
        L.sharq_prepare.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int64, c_void_p, c_float,
                                    POINTER(SharqAct), c_void_p, c_size_t, c_void_p]
        L.sharq_prepare_no_alloc.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int64, c_void_p, c_float,
                                             POINTER(SharqAct), c_void_p]
        L.sharq_linear.argtypes = [POINTER(SharqAct), POINTER(SharqWeight), c_void_p, c_void_p, c_int32,
                                   c_void_p, c_int64, c_void_p]
        L.sharq_prepare_linear.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int64, c_void_p, c_float,
                                           POINTER(SharqAct), POINTER(SharqWeight), c_void_p, c_int64, c_void_p,
                                           c_size_t, c_void_p]
        L.sharq_prepare_linear_status.argtypes = [c_void_p, c_size_t, c_void_p]
        L.sharq_rmsnorm.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int64, c_void_p, c_float, c_void_p,
                                    c_int64, c_void_p]
        L.sharq_quantize_mx.argtypes = [c_void_p, c_int32, c_int32, c_int64, c_void_p, c_void_p, c_void_p]
        L.sharq_linear_dense.argtypes = [c_void_p, c_void_p, c_int32, POINTER(SharqWeight), c_void_p, c_int64,
                                         c_void_p]
        for name in ("sharq_weight_sizes", "sharq_act_sizes", "sharq_pack_weight", "sharq_prepare",
                     "sharq_prepare_no_alloc", "sharq_linear",
                     "sharq_prepare_linear", "sharq_prepare_linear_status", "sharq_rmsnorm", "sharq_quantize_mx", "sharq_linear_dense"):
            getattr(L, name).restype = c_int32
        L.sharq_timeline_records.argtypes = [POINTER(c_size_t)]
        L.sharq_timeline_clear.argtypes = []
        L.sharq_timeline_read.argtypes = [c_void_p, c_size_t]
        for name in ("sharq_timeline_records", "sharq_timeline_clear", "sharq_timeline_read"):
            getattr(L, name).restype = c_int32
        L.sharq_status_string.argtypes = [c_int32]
        L.sharq_status_string.restype = c_char_p
        L.sharq_last_error.argtypes = []
        L.sharq_last_error.restype = c_char_p
        _lib = L
    return _lib


def status_name(s: int) -> str:
    return lib().sharq_status_string(s).decode()


def check(s: int) -> None:
    if s != SHARQ_OK:
        raise SharqError(s, lib().sharq_last_error().decode())


def weight_sizes(fmt: int, K: int, D: int, n_groups: int = 1):
    out = (c_size_t * 5)()
    check(lib().sharq_weight_sizes(fmt, K, D, n_groups, out))
    return list(out)


def act_sizes(fmt: int, T: int, K: int):
    out = (c_size_t * 7)()
    check(lib().sharq_act_sizes(fmt, T, K, out))
    return list(out)
