"""ctypes binding of libwtconv (the C ABI declared in include/wtconv.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libwtconv.so.  Tensors are PyTorch tensors on the GPU; PyTorch provides device
memory and the stream, nothing else.  If the library is missing this module
raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libwtconv.so")

WTCONV_OK = 0
STATUS = {0: "WTCONV_OK", 1: "WTCONV_ERR_NULL", 2: "WTCONV_ERR_SHAPE", 3: "WTCONV_ERR_UNSUPPORTED",
          4: "WTCONV_ERR_WORKSPACE", 5: "WTCONV_ERR_HIP", 6: "WTCONV_ERR_ALIAS"}
F32, F16 = 0, 1
OP_FWD, OP_BWD_DATA, OP_BWD_WEIGHT, OP_BWD = 0, 1, 2, 3


class WtconvDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("c", ctypes.c_int64), ("h", ctypes.c_int64), ("w", ctypes.c_int64),
                ("k", ctypes.c_int32), ("levels", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class WtconvError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s returned %s" % (what, STATUS.get(status, status)))
        self.status = status


_lib = None

# name -> argument types (pointers as void*), all return wtconv_status_t (int)
_vp, _sz, _dp = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(WtconvDesc)
SIGNATURES = {
    "wtconv_workspace_size": [_dp, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)],
    "wtconv_forward": [_dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "wtconv_backward_data": [_dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "wtconv_backward_weight": [_dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "wtconv_backward": [_dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "wtconv_backward_weight_noalloc": [_dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "wtconv_unfused_workspace_size": [_dp, ctypes.POINTER(ctypes.c_size_t)],
    "wtconv_unfused_forward": [_dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "wtconv_unfused_backward_data": [_dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "wtconv_unfused_backward_weight": [_dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                       _vp],
}


def load(path: str = LIB_PATH):
    """Load libwtconv.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise OSError("libwtconv.so not built: run `python -m level_haar_wavelet_amd.build` (%s)" % path)
        lib = ctypes.CDLL(path)
        for name, args in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.wtconv_status_string.argtypes = [ctypes.c_int]
        lib.wtconv_status_string.restype = ctypes.c_char_p
        lib.wtconv_version.argtypes = []
        lib.wtconv_version.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def desc(n, c, h, w, k, levels, dtype):
    return WtconvDesc(int(n), int(c), int(h), int(w), int(k), int(levels), int(dtype))


def check(status, what):
    if status != WTCONV_OK:
        raise WtconvError(status, what)
