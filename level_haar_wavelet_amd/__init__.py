"""libwtconv: the WTConv layer (wavelet convolution) for AMD MI355X (gfx950).

The functions here carry the names of the C entry points in include/wtconv.h
and only marshal PyTorch GPU tensors into them; every step of the layer runs in
the library's HIP kernels.  Parameter tensors are float32 on the GPU:
    w_base (C, k, k), bias (C,) or None, s_base (C,),
    w_lvl (L, 4C, k, k), s_lvl (L, 4C)   (band b of channel c at index 4c+b).
Activations are (N, C, H, W) float32 or float16, contiguous.
"""
from __future__ import annotations

import ctypes

from . import _native

__all__ = ["wtconv_forward", "wtconv_backward_data", "wtconv_backward_weight", "wtconv_backward",
           "wtconv_backward_weight_noalloc", "wtconv_workspace_size", "library_path"]


def library_path() -> str:
    return _native.LIB_PATH


def _torch():
    import torch

    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return _native.F32
    if t.dtype == torch.float16:
        return _native.F16
    raise TypeError("activations must be float32 or float16, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check_param(t, name):
    torch = _torch()
    if t is None:
        return
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise TypeError("%s must be a contiguous float32 GPU tensor" % name)


def _levels_of(w_lvl):
    return 0 if w_lvl is None else int(w_lvl.shape[0])


def _desc_for(x, w_base, levels):
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("activations must be a contiguous (N, C, H, W) GPU tensor")
    n, c, h, w = x.shape
    k = int(w_base.shape[-1])
    return _native.desc(n, c, h, w, k, levels, _dtype_code(x))


def wtconv_workspace_size(shape, k, levels, dtype_code, op) -> int:
    lib = _native.load()
    d = _native.desc(*shape, k, levels, dtype_code)
    out = ctypes.c_size_t(0)
    _native.check(lib.wtconv_workspace_size(ctypes.byref(d), op, ctypes.byref(out)), "wtconv_workspace_size")
    return out.value


def _workspace_for(lib, d, op, workspace, device):
    """The caller's workspace, or a new one when the op needs one (planes too
    large for one workgroup with L >= 2 keep the level-1 low-pass map and the
    deeper levels' term there)."""
    need = ctypes.c_size_t(0)
    _native.check(lib.wtconv_workspace_size(ctypes.byref(d), op, ctypes.byref(need)), "wtconv_workspace_size")
    if need.value == 0:
        return None, 0
    if workspace is None:
        workspace = _torch().empty(need.value, dtype=_torch().uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def wtconv_forward(x, w_base, bias, s_base, w_lvl, s_lvl, y=None, stream=None, workspace=None):
    """y = WTConv(x), enqueued on `stream` (default: torch's current stream)."""
    lib = _native.load()
    for t, name in ((w_base, "w_base"), (bias, "bias"), (s_base, "s_base"), (w_lvl, "w_lvl"), (s_lvl, "s_lvl")):
        _check_param(t, name)
    d = _desc_for(x, w_base, _levels_of(w_lvl))
    if y is None:
        y = _torch().empty_like(x)
    ws, nbytes = _workspace_for(lib, d, _native.OP_FWD, workspace, x.device)
    st = lib.wtconv_forward(ctypes.byref(d), _ptr(x), _ptr(w_base), _ptr(bias), _ptr(s_base), _ptr(w_lvl),
                            _ptr(s_lvl), _ptr(y), _ptr(ws), nbytes, _stream(stream))
    _native.check(st, "wtconv_forward")
    return y


def wtconv_backward_data(dy, w_base, s_base, w_lvl, s_lvl, dx=None, stream=None, workspace=None):
    """dx = d<dy, WTConv(x)>/dx, enqueued on `stream`."""
    lib = _native.load()
    for t, name in ((w_base, "w_base"), (s_base, "s_base"), (w_lvl, "w_lvl"), (s_lvl, "s_lvl")):
        _check_param(t, name)
    d = _desc_for(dy, w_base, _levels_of(w_lvl))
    if dx is None:
        dx = _torch().empty_like(dy)
    ws, nbytes = _workspace_for(lib, d, _native.OP_BWD_DATA, workspace, dy.device)
    st = lib.wtconv_backward_data(ctypes.byref(d), _ptr(dy), _ptr(w_base), _ptr(s_base), _ptr(w_lvl), _ptr(s_lvl),
                                  _ptr(dx), _ptr(ws), nbytes, _stream(stream))
    _native.check(st, "wtconv_backward_data")
    return dx


def wtconv_backward_weight(x, dy, w_base, bias, s_base, w_lvl, s_lvl, workspace=None, grads=None, stream=None):
    """Parameter gradients of <dy, WTConv(x)>: (dw_base, dbias, ds_base, dw_lvl, ds_lvl).

    `workspace` is a uint8 GPU tensor of at least wtconv_workspace_size(...,
    OP_BWD_WEIGHT) bytes (allocated here if None); `grads` optionally supplies
    the five output tensors (overwritten)."""
    torch = _torch()
    lib = _native.load()
    for t, name in ((w_base, "w_base"), (bias, "bias"), (s_base, "s_base"), (w_lvl, "w_lvl"), (s_lvl, "s_lvl")):
        _check_param(t, name)
    levels = _levels_of(w_lvl)
    d = _desc_for(x, w_base, levels)
    if dy.shape != x.shape or dy.dtype != x.dtype or not dy.is_contiguous():
        raise TypeError("dy must match x in shape, dtype and layout")
    need = ctypes.c_size_t(0)
    _native.check(lib.wtconv_workspace_size(ctypes.byref(d), _native.OP_BWD_WEIGHT, ctypes.byref(need)),
                  "wtconv_workspace_size")
    if workspace is None:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=x.device)
    if grads is None:
        c, k = x.shape[1], w_base.shape[-1]
        grads = (torch.empty_like(w_base), torch.empty((c,), dtype=torch.float32, device=x.device),
                 torch.empty_like(s_base),
                 torch.empty_like(w_lvl) if levels else None, torch.empty_like(s_lvl) if levels else None)
    dw0, db0, ds0, dwl, dsl = grads
    st = lib.wtconv_backward_weight(ctypes.byref(d), _ptr(x), _ptr(dy), _ptr(w_base), _ptr(bias), _ptr(s_base),
                                    _ptr(w_lvl), _ptr(s_lvl), _ptr(dw0), _ptr(db0), _ptr(ds0), _ptr(dwl),
                                    _ptr(dsl), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream))
    _native.check(st, "wtconv_backward_weight")
    return dw0, db0, ds0, dwl, dsl


def wtconv_backward(x, dy, w_base, bias, s_base, w_lvl, s_lvl, dx=None, grads=None, workspace=None, stream=None):
    """dx and the parameter gradients in one call: (dx, (dw_base, dbias,
    ds_base, dw_lvl, ds_lvl)).  One fused pass over x and dy where a plane fits
    one workgroup, else the data and weight backward one after the other.
    `workspace` is a uint8 GPU tensor of at least wtconv_workspace_size(...,
    OP_BWD) bytes (allocated here if None)."""
    torch = _torch()
    lib = _native.load()
    for t, name in ((w_base, "w_base"), (bias, "bias"), (s_base, "s_base"), (w_lvl, "w_lvl"), (s_lvl, "s_lvl")):
        _check_param(t, name)
    levels = _levels_of(w_lvl)
    d = _desc_for(x, w_base, levels)
    if dy.shape != x.shape or dy.dtype != x.dtype or not dy.is_contiguous():
        raise TypeError("dy must match x in shape, dtype and layout")
    if dx is None:
        dx = torch.empty_like(dy)
    need = ctypes.c_size_t(0)
    _native.check(lib.wtconv_workspace_size(ctypes.byref(d), _native.OP_BWD, ctypes.byref(need)),
                  "wtconv_workspace_size")
    if workspace is None:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=x.device)
    if grads is None:
        c = x.shape[1]
        grads = (torch.empty_like(w_base), torch.empty((c,), dtype=torch.float32, device=x.device),
                 torch.empty_like(s_base),
                 torch.empty_like(w_lvl) if levels else None, torch.empty_like(s_lvl) if levels else None)
    dw0, db0, ds0, dwl, dsl = grads
    st = lib.wtconv_backward(ctypes.byref(d), _ptr(x), _ptr(dy), _ptr(w_base), _ptr(bias), _ptr(s_base),
                             _ptr(w_lvl), _ptr(s_lvl), _ptr(dx), _ptr(dw0), _ptr(db0), _ptr(ds0), _ptr(dwl),
                             _ptr(dsl), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream))
    _native.check(st, "wtconv_backward")
    return dx, (dw0, db0, ds0, dwl, dsl)


def wtconv_backward_weight_noalloc(x, dy, w_base, bias, s_base, w_lvl, s_lvl, grads=None, stream=None):
    """wtconv_backward_weight without a workspace argument: the library keeps
    the partial results in its own static device array (no allocation by the
    call; calls that overlap on one GPU race).  `grads` optionally supplies the
    five output tensors (overwritten); they are allocated here if None."""
    torch = _torch()
    lib = _native.load()
    for t, name in ((w_base, "w_base"), (bias, "bias"), (s_base, "s_base"), (w_lvl, "w_lvl"), (s_lvl, "s_lvl")):
        _check_param(t, name)
    levels = _levels_of(w_lvl)
    d = _desc_for(x, w_base, levels)
    if dy.shape != x.shape or dy.dtype != x.dtype or not dy.is_contiguous():
        raise TypeError("dy must match x in shape, dtype and layout")
    if grads is None:
        c = x.shape[1]
        grads = (torch.empty_like(w_base), torch.empty((c,), dtype=torch.float32, device=x.device),
                 torch.empty_like(s_base),
                 torch.empty_like(w_lvl) if levels else None, torch.empty_like(s_lvl) if levels else None)
    dw0, db0, ds0, dwl, dsl = grads
    st = lib.wtconv_backward_weight_noalloc(ctypes.byref(d), _ptr(x), _ptr(dy), _ptr(w_base), _ptr(bias),
                                            _ptr(s_base), _ptr(w_lvl), _ptr(s_lvl), _ptr(dw0), _ptr(db0), _ptr(ds0),
                                            _ptr(dwl), _ptr(dsl), _stream(stream))
    _native.check(st, "wtconv_backward_weight_noalloc")
    return dw0, db0, ds0, dwl, dsl
