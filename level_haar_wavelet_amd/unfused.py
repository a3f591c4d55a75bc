"""Binding of the unfused baseline (test and benchmark use only): the layer
as separate kernels with every intermediate in HBM, for the fused-versus-
unfused comparison.  Same names as the C entry points in include/wtconv.h;
argument marshalling only.  One workspace (allocated by `workspace`) carries
the forward's intermediates to the two backward calls."""
from __future__ import annotations

import ctypes

from . import _native
from . import _desc_for, _levels_of, _ptr, _stream

__all__ = ["wtconv_unfused_workspace_size", "wtconv_unfused_forward", "wtconv_unfused_backward_data",
           "wtconv_unfused_backward_weight", "workspace"]


def wtconv_unfused_workspace_size(shape, k, levels, dtype_code) -> int:
    lib = _native.load()
    d = _native.desc(*shape, k, levels, dtype_code)
    out = ctypes.c_size_t(0)
    _native.check(lib.wtconv_unfused_workspace_size(ctypes.byref(d), ctypes.byref(out)),
                  "wtconv_unfused_workspace_size")
    return out.value


def workspace(x, k, levels):
    import torch

    code = _native.F32 if x.dtype == torch.float32 else _native.F16
    n = wtconv_unfused_workspace_size(tuple(x.shape), k, levels, code)
    return torch.empty(n, dtype=torch.uint8, device=x.device)


def _nbytes(ws):
    return ws.numel() * ws.element_size()


def wtconv_unfused_forward(x, w_base, bias, s_base, w_lvl, s_lvl, ws, y=None, stream=None):
    import torch

    lib = _native.load()
    d = _desc_for(x, w_base, _levels_of(w_lvl))
    if y is None:
        y = torch.empty_like(x)
    st = lib.wtconv_unfused_forward(ctypes.byref(d), _ptr(x), _ptr(w_base), _ptr(bias), _ptr(s_base), _ptr(w_lvl),
                                    _ptr(s_lvl), _ptr(y), _ptr(ws), _nbytes(ws), _stream(stream))
    _native.check(st, "wtconv_unfused_forward")
    return y


def wtconv_unfused_backward_data(dy, w_base, s_base, w_lvl, s_lvl, ws, dx=None, stream=None):
    import torch

    lib = _native.load()
    d = _desc_for(dy, w_base, _levels_of(w_lvl))
    if dx is None:
        dx = torch.empty_like(dy)
    st = lib.wtconv_unfused_backward_data(ctypes.byref(d), _ptr(dy), _ptr(w_base), _ptr(s_base), _ptr(w_lvl),
                                          _ptr(s_lvl), _ptr(dx), _ptr(ws), _nbytes(ws), _stream(stream))
    _native.check(st, "wtconv_unfused_backward_data")
    return dx


def wtconv_unfused_backward_weight(x, dy, w_base, bias, s_base, w_lvl, s_lvl, ws, grads=None, stream=None):
    import torch

    lib = _native.load()
    levels = _levels_of(w_lvl)
    d = _desc_for(x, w_base, levels)
    if grads is None:
        c = x.shape[1]
        grads = (torch.empty_like(w_base), torch.empty((c,), dtype=torch.float32, device=x.device),
                 torch.empty_like(s_base), torch.empty_like(w_lvl) if levels else None,
                 torch.empty_like(s_lvl) if levels else None)
    dw0, db0, ds0, dwl, dsl = grads
    st = lib.wtconv_unfused_backward_weight(ctypes.byref(d), _ptr(x), _ptr(dy), _ptr(w_base), _ptr(bias),
                                            _ptr(s_base), _ptr(w_lvl), _ptr(s_lvl), _ptr(dw0), _ptr(db0), _ptr(ds0),
                                            _ptr(dwl), _ptr(dsl), _ptr(ws), _nbytes(ws), _stream(stream))
    _native.check(st, "wtconv_unfused_backward_weight")
    return grads


class UnfusedWTConvFunction:
    """The unfused baseline as a PyTorch autograd function (benchmark use): the
    forward keeps its intermediates (subbands, convolution outputs, partial
    reconstructions) in a workspace saved for the backward, as autograd keeps
    the tensors of a layer composed of separate operations."""

    @staticmethod
    def apply(x, w_base, bias, s_base, w_lvl, s_lvl):
        import torch

        class _Fn(torch.autograd.Function):
            @staticmethod
            def forward(ctx, x, w_base, bias, s_base, w_lvl, s_lvl):
                x = x.contiguous()
                k = int(w_base.shape[-1])
                levels = 0 if w_lvl is None else int(w_lvl.shape[0])
                ws = workspace(x, k, levels)
                y = wtconv_unfused_forward(x, w_base, bias, s_base, w_lvl, s_lvl, ws)
                ctx.save_for_backward(x, w_base, bias, s_base, w_lvl, s_lvl, ws)
                ctx.has_bias = bias is not None
                return y

            @staticmethod
            def backward(ctx, dy):
                x, w_base, bias, s_base, w_lvl, s_lvl, ws = ctx.saved_tensors
                dy = dy.contiguous().to(x.dtype)
                dx = wtconv_unfused_backward_data(dy, w_base, s_base, w_lvl, s_lvl, ws)
                dw0, db0, ds0, dwl, dsl = wtconv_unfused_backward_weight(x, dy, w_base, bias, s_base, w_lvl, s_lvl,
                                                                         ws)
                return dx, dw0, db0 if ctx.has_bias else None, ds0, dwl, dsl

        return _Fn.apply(x, w_base, bias, s_base, w_lvl, s_lvl)
