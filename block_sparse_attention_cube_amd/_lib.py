"""ctypes view of libvsa.so (the C ABI declared in include/vsa.h).

Argument marshalling only.  Loading fails loudly if the library has not been
built: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvsa.so")

VSA_OK = 0
VSA_ERR_NULL = 1
VSA_ERR_SHAPE = 2
VSA_ERR_UNSUPPORTED = 3
VSA_ERR_ALIGN = 4
VSA_ERR_WORKSPACE = 5
VSA_ERR_LAUNCH = 6

VSA_F32 = 0
VSA_BF16 = 1

VSA_OP_FORWARD = 0
VSA_OP_BACKWARD = 1
VSA_OP_COARSE = 2
VSA_OP_FINE = 3
VSA_OP_FORWARD_FP8 = 4
VSA_OP_FORWARD_CUBE = 5
VSA_OP_BACKWARD_CUBE = 6

EXPORTS = ("vsa_workspace_bytes", "vsa_check_problem", "vsa_reorder", "vsa_coarse",
           "vsa_fine", "vsa_fine_raster", "vsa_dense", "vsa_forward", "vsa_forward_static",
           "vsa_forward_cube", "vsa_backward_cube", "vsa_backward", "vsa_quantize_fp8", "vsa_fine_fp8",
           "vsa_forward_fp8", "vsa_status_string")


class VSAProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32),
                ("T", ctypes.c_int32), ("Hh", ctypes.c_int32), ("Ww", ctypes.c_int32),
                ("d", ctypes.c_int32),
                ("cube_t", ctypes.c_int32), ("cube_h", ctypes.c_int32), ("cube_w", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class VSAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lib = None

_P = ctypes.POINTER(VSAProblem)
_V = ctypes.c_void_p
_SIG = {
    "vsa_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int]),
    "vsa_check_problem": (ctypes.c_int, [_P]),
    "vsa_reorder": (ctypes.c_int, [_P, _V, _V, ctypes.c_int, _V]),
    "vsa_coarse": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "vsa_fine": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "vsa_fine_raster": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V]),
    "vsa_dense": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V]),
    "vsa_forward": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t,
                                   _V]),
    "vsa_forward_static": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V]),
    "vsa_forward_cube": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V,
                                        ctypes.c_size_t, _V]),
    "vsa_backward_cube": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V,
                                         ctypes.c_size_t, _V]),
    "vsa_backward": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V,
                                    ctypes.c_size_t, _V]),
    "vsa_quantize_fp8": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V]),
    "vsa_fine_fp8": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V]),
    "vsa_forward_fp8": (ctypes.c_int, [_P, _V, _V, _V, _V, _V, _V, _V, _V, ctypes.c_size_t, _V]),
    "vsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}


def lib():
    """The loaded library (loaded once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first "
                "(python -m block_sparse_attention_cube_amd.build)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().vsa_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != VSA_OK:
        raise VSAError(status, what)
