"""PyTorch autograd wrapper and nn.Module over libwtconv.

The layer (the depthwise base convolution with bias and scale, plus L levels of
orthonormal Haar analysis, per-level depthwise convolutions over the 4C
subbands with per-band scales, and the synthesis cascade) is the one described
in "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
Reformulation" (arXiv 2608.10805), technical summary, Methodology, and the
WTConv layer it reformulates.  Forward, data backward and parameter gradients
all run in libwtconv's kernels (wtconv_forward, wtconv_backward_data,
wtconv_backward_weight); this module only hands tensors to them.  The layer
saves only its input for the backward pass.
"""
from __future__ import annotations

import torch

from . import wtconv_backward_data, wtconv_backward_weight, wtconv_forward

__all__ = ["WTConvFunction", "WTConv2d"]


class WTConvFunction(torch.autograd.Function):
    """y = WTConv(x; w_base, bias, s_base, w_lvl, s_lvl).

    x: (N, C, H, W) float32 or float16, contiguous, on the GPU (sides 2^L
    does not divide: odd level maps zero-padded at the bottom / right, each
    level's synthesis cropped back).  Parameters are float32: w_base (C, k, k), bias (C,) or
    None, s_base (C,), w_lvl (L, 4C, k, k) and s_lvl (L, 4C), or None for
    both when L = 0.
    """

    @staticmethod
    def forward(ctx, x, w_base, bias, s_base, w_lvl, s_lvl):
        x = x.contiguous()
        y = wtconv_forward(x, w_base, bias, s_base, w_lvl, s_lvl)
        ctx.save_for_backward(x, w_base, bias, s_base, w_lvl, s_lvl)
        ctx.has_bias = bias is not None
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w_base, bias, s_base, w_lvl, s_lvl = ctx.saved_tensors
        dy = dy.contiguous().to(x.dtype)
        need = ctx.needs_input_grad
        dx = wtconv_backward_data(dy, w_base, s_base, w_lvl, s_lvl) if need[0] else None
        dw0 = db0 = ds0 = dwl = dsl = None
        if any(need[1:]):
            dw0, db0, ds0, dwl, dsl = wtconv_backward_weight(x, dy, w_base, bias, s_base, w_lvl, s_lvl)
        return (dx, dw0 if need[1] else None, db0 if (ctx.has_bias and need[2]) else None,
                ds0 if need[3] else None, dwl if need[4] else None, dsl if need[5] else None)


class WTConv2d(torch.nn.Module):
    """Drop-in WTConv layer: a depthwise k x k convolution with an L-level
    Haar wavelet branch (same channels in and out, stride 1, 'same' padding).

    Initialisation: weights N(0, 0.05^2), bias zero, base scale 1 and
    level scales 0.1 (the wavelet branch starts small next to the base
    convolution).
    """

    def __init__(self, channels: int, kernel_size: int = 5, levels: int = 1, bias: bool = True,
                 device=None):
        super().__init__()
        if kernel_size not in (1, 3, 5, 7):
            raise ValueError("kernel_size must be 1, 3, 5 or 7")
        if levels < 0:
            raise ValueError("levels must be >= 0")
        c, k = channels, kernel_size
        f = dict(device=device, dtype=torch.float32)
        self.channels, self.kernel_size, self.levels = c, k, levels
        self.w_base = torch.nn.Parameter(torch.randn(c, k, k, **f) * 0.05)
        self.bias = torch.nn.Parameter(torch.zeros(c, **f)) if bias else None
        self.s_base = torch.nn.Parameter(torch.ones(c, **f))
        if levels > 0:
            self.w_lvl = torch.nn.Parameter(torch.randn(levels, 4 * c, k, k, **f) * 0.05)
            self.s_lvl = torch.nn.Parameter(torch.full((levels, 4 * c), 0.1, **f))
        else:
            self.register_parameter("w_lvl", None)
            self.register_parameter("s_lvl", None)

    def forward(self, x):
        return WTConvFunction.apply(x, self.w_base, self.bias, self.s_base, self.w_lvl, self.s_lvl)

    def extra_repr(self):
        return "channels=%d, kernel_size=%d, levels=%d, bias=%s" % (self.channels, self.kernel_size, self.levels,
                                                                   self.bias is not None)
