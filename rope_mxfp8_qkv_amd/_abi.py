"""ctypes declarations of the C ABI (``include/qkvmx.h``).  Loading fails loudly when the
in-tree ``libqkvmx.so`` is missing: build it with ``python -m rope_mxfp8_qkv_amd.build``."""
from __future__ import annotations

import ctypes
import os

NORM_Q = 1
NORM_K = 2
FUSED_ROPE = 4
LAYOUT_BSD = 0
LAYOUT_NBSD = 1
HEAD_RMS_NORM = 1
HEAD_LAYER_NORM = 2
DTYPE_F32 = 0
DTYPE_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqkvmx.so")
_lib = None

c_i64 = ctypes.c_int64
c_i32 = ctypes.c_int32
c_u32 = ctypes.c_uint32
c_vp = ctypes.c_void_p
c_sz = ctypes.c_size_t
c_f = ctypes.c_float

# name -> (restype, argtypes); mirrors include/qkvmx.h
SIGNATURES = {
    "qkvmx_status_string": (ctypes.c_char_p, [c_i32]),
    "qkvmx_last_error": (ctypes.c_char_p, []),
    "mx_weight_quantize": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "qkv_weight_packed_bytes": (c_sz, [c_i64, c_i64]),
    "qkv_weight_prepack": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_vp, c_sz, c_vp]),
    "row_quantize_packed": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_vp, c_vp]),
    "rmsnorm_mx_quantize": (c_i32, [c_vp, c_vp, c_vp, c_f, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "qkvmx_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64]),
    "qkv_rowmx_project": (c_i32, [c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64, c_i32,
                                  c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "mx_block_quantize": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "rmsnorm_mx_block_quantize": (c_i32, [c_vp, c_vp, c_vp, c_f, c_i64, c_i64, c_i64, c_vp, c_vp,
                                          c_vp, c_vp, c_vp]),
    "qkv_mx_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64]),
    "qkv_rowmx_project_headnorm": (c_i32, [c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_i64, c_i32,
                                           c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_f,
                                           c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "qkv_rowmx_project_headnorm_staged": (c_i32, [c_vp, c_sz, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                  c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp,
                                                  c_vp, c_vp, c_f, c_vp, c_vp, c_vp, c_vp, c_sz,
                                                  c_vp]),
    "qkv_mx_project": (c_i32, [c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64, c_i32,
                               c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "qkv_act_image_bytes": (c_sz, [c_i64, c_i64]),
    "row_quantize_staged": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_vp, c_sz, c_vp, c_vp]),
    "rmsnorm_mx_quantize_staged": (c_i32, [c_vp, c_vp, c_vp, c_f, c_i64, c_i64, c_i64, c_vp, c_vp,
                                           c_sz, c_vp, c_vp]),
    "qkv_staged_workspace_bytes": (c_sz, [c_i64, c_i64]),
    "qkvmx_projection_k_chunks": (c_i32, [c_i64, c_i64, c_i64, c_i32]),
    "qkv_rowmx_project_staged": (c_i32, [c_vp, c_sz, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i32,
                                         c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "qkv_act_exp_image_bytes": (c_sz, [c_i64, c_i64]),
    "mx_block_quantize_staged": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_vp, c_sz, c_vp, c_sz, c_vp]),
    "rmsnorm_mx_block_quantize_staged": (c_i32, [c_vp, c_vp, c_vp, c_f, c_i64, c_i64, c_i64, c_vp,
                                                 c_vp, c_sz, c_vp, c_sz, c_vp, c_vp]),
    "qkv_mx_project_staged": (c_i32, [c_vp, c_sz, c_vp, c_sz, c_vp, c_vp, c_vp, c_i64, c_i64, c_i32,
                                      c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "qkvmx_noalloc_scratch_bytes": (c_sz, []),
    "qkv_rowmx_project_staged_noalloc": (c_i32, [c_vp, c_sz, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                 c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "qkvmx_mfma_rate_probe": (c_i32, [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "qkvmx_e4m3_convert_check": (c_i32, [c_vp, c_vp, c_vp]),
    "qk_norm_rope_apply": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i32, c_i32, c_i32,
                                   c_f, c_u32, c_i32, c_vp]),
}


class QkvmxError(RuntimeError):
    def __init__(self, msg, status: int = -1):
        super().__init__(msg)
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise QkvmxError(f"{_LIB_PATH} is missing: build it with "
                             "`python -m rope_mxfp8_qkv_amd.build` (no fallback path exists)")
        # torch (which brings its own HIP runtime) is loaded before the library: loaded first,
        # the library's HIP calls later failed in the same process ("no ROCm-capable device")
        # once torch had initialised the GPU
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().qkvmx_status_string(s).decode()


def last_error() -> str:
    return lib().qkvmx_last_error().decode()
