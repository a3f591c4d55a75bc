"""The weight backward without a workspace argument (its partial results in
the library's static device array) through the C ABI: the same gradients as
wtconv_backward_weight with a caller's workspace, bit for bit (same kernels,
same plans, same reduction order), on two calls in a row, the second on a
smaller input, and the refusal of a call whose workspace would not fit."""
import ctypes

import numpy as np
import pytest
import torch

from level_haar_wavelet_amd import _native
from level_haar_wavelet_amd.synthetic import make_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests.gpu_util import DevInputs


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _grads_like(d):
    return [torch.full_like(t, float("nan")) if t is not None else None
            for t in (d.w_base, d.s_base, d.s_base, d.w_lvl, d.s_lvl)]


def _call_noalloc(lib, desc, d, g):
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.wtconv_backward_weight_noalloc(ctypes.byref(desc), _ptr(d.x), _ptr(d.dy), _ptr(d.w_base),
                                              _ptr(d.bias), _ptr(d.s_base), _ptr(d.w_lvl), _ptr(d.s_lvl),
                                              *[_ptr(t) for t in g], s)


def _call_workspace(lib, desc, d, g):
    need = ctypes.c_size_t(0)
    assert lib.wtconv_workspace_size(ctypes.byref(desc), _native.OP_BWD_WEIGHT, ctypes.byref(need)) == 0
    ws = torch.empty(max(need.value, 1), dtype=torch.uint8, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.wtconv_backward_weight(ctypes.byref(desc), _ptr(d.x), _ptr(d.dy), _ptr(d.w_base), _ptr(d.bias),
                                    _ptr(d.s_base), _ptr(d.w_lvl), _ptr(d.s_lvl), *[_ptr(t) for t in g],
                                    _ptr(ws), ws.numel(), s)
    return st, ws


@pytest.mark.parametrize("first,second", [
    ((6, 16, 56, 56, 5, 3, "f32"), (2, 8, 28, 28, 5, 3, "f32")),
    ((4, 12, 28, 28, 5, 2, "f16"), (3, 5, 16, 24, 3, 2, "f16")),
    ((2, 4, 64, 96, 5, 1, "f32"), (1, 2, 17, 21, 5, 1, "f32")),   # tiles, then sides 2^L does not divide
])
def test_noalloc_weight_backward_equals_the_workspace_call(first, second):
    lib = _native.load()
    for case in (first, second):
        n, c, h, w, k, L, dt = case
        print("case", case, flush=True)
        inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=n + c + h + w + k + L)
        d = DevInputs(inp, dt)
        desc = _native.desc(n, c, h, w, k, L, _native.F32 if dt == "f32" else _native.F16)
        g_ref, g_new = _grads_like(d), _grads_like(d)
        st, ws = _call_workspace(lib, desc, d, g_ref)
        assert st == 0
        assert _call_noalloc(lib, desc, d, g_new) == 0
        torch.cuda.synchronize()
        for a, b in zip(g_ref, g_new):
            if a is None:
                continue
            assert torch.isfinite(b).all()
            assert torch.equal(a, b), float((a - b).abs().max())
        del ws


def test_noalloc_refuses_a_workspace_beyond_its_array():
    """The 256 x 256 L = 4 layer keeps level-1 low-pass maps in its workspace
    (hundreds of MB): refused before anything is enqueued."""
    lib = _native.load()
    desc = _native.desc(16, 256, 256, 256, 5, 4, _native.F16)
    need = ctypes.c_size_t(0)
    assert lib.wtconv_workspace_size(ctypes.byref(desc), _native.OP_BWD_WEIGHT, ctypes.byref(need)) == 0
    assert need.value > 16 << 20
    p = ctypes.c_void_p(0x10000)  # never dereferenced: the size check comes first
    assert lib.wtconv_backward_weight_noalloc(ctypes.byref(desc), p, p, p, None, p, p, p, p, p, p, p, p,
                                              None) == 4
