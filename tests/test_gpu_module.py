"""The autograd wrapper and nn.Module over libwtconv: forward and every
gradient against the CPU oracle (the backward pass is the oracle's with the
upstream gradient as dy), and the layer's saved-tensor footprint."""
import numpy as np
import pytest
import torch

from level_haar_wavelet_amd.synthetic import make_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from level_haar_wavelet_amd.module import WTConv2d, WTConvFunction
    from tests.gpu_util import assert_close, assert_grads_close


def _module_from(inp, k, L, bias=True):
    c = inp.x.shape[1]
    m = WTConv2d(c, k, L, bias=bias, device="cuda")
    with torch.no_grad():
        m.w_base.copy_(torch.from_numpy(inp.w_base))
        if bias:
            m.bias.copy_(torch.from_numpy(inp.bias))
        m.s_base.copy_(torch.from_numpy(inp.s_base))
        if L:
            m.w_lvl.copy_(torch.from_numpy(inp.w_lvl))
            m.s_lvl.copy_(torch.from_numpy(inp.s_lvl))
    return m


@pytest.mark.parametrize("case", [(2, 8, 16, 16, 5, 2, "f32", True), (2, 4, 56, 56, 5, 3, "f32", False),
                                  (2, 6, 28, 28, 3, 2, "f16", True), (2, 3, 12, 20, 7, 0, "f32", True)],
                         ids=lambda c: "x".join(map(str, c)))
def test_module_forward_and_gradients(orc, case):
    n, c, h, w, k, L, dt, bias = case
    print("case", case, flush=True)
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h + w + k + L)
    if not bias:
        inp.bias = None
    m = _module_from(inp, k, L, bias)
    tdt = torch.float32 if dt == "f32" else torch.float16
    x = torch.from_numpy(inp.x).to("cuda", tdt).requires_grad_(True)
    y = m(x)
    y.backward(torch.from_numpy(inp.dy).to("cuda", tdt))
    torch.cuda.synchronize()
    ref_y = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    ref_dx = orc.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    ref_g = orc.backward_weight(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    assert_close(y, ref_y, dt, "y")
    assert_close(x.grad, ref_dx, dt, "dx")
    got = (m.w_base.grad, m.bias.grad if bias else None, m.s_base.grad,
           m.w_lvl.grad if L else None, m.s_lvl.grad if L else None)
    ref = list(ref_g)
    if not bias:
        ref[1] = None
    assert_grads_close(got, ref, dt, "module")


def test_function_skips_unneeded_gradients(orc):
    n, c, h, w, k, L = 1, 4, 16, 16, 3, 2
    inp = make_inputs(n, c, h, w, k, L, seed=5)
    dev = lambda a: torch.from_numpy(a).cuda()
    x = dev(inp.x).requires_grad_(True)
    params = [dev(inp.w_base), dev(inp.bias), dev(inp.s_base), dev(inp.w_lvl), dev(inp.s_lvl)]
    y = WTConvFunction.apply(x, *params)
    (dx,) = torch.autograd.grad(y, x, torch.from_numpy(inp.dy).cuda())
    ref_dx = orc.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    assert_close(dx, ref_dx, "f32", "dx only")


def test_saved_activation_memory_is_the_input_only():
    """Between forward and backward the layer holds its input and output
    only (no subbands): the memory allocated by the forward is the output."""
    n, c, h, w, k, L = 8, 32, 56, 56, 5, 3
    m = WTConv2d(c, k, L, device="cuda")
    x = torch.randn(n, c, h, w, device="cuda", requires_grad=True)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    y = m(x)
    torch.cuda.synchronize()
    held = torch.cuda.memory_allocated() - before
    assert held <= y.numel() * y.element_size() + (1 << 20), held


def test_block_with_fused_and_unfused_layer_gives_the_same_gradients():
    """The synthetic WTConvNeXt-style block that bench.py measures peak memory
    on: with the fused layer and with the unfused baseline as autograd
    functions, every gradient (input, layer parameters, block parameters)
    agrees."""
    import bench
    from level_haar_wavelet_amd.module import WTConvFunction
    from level_haar_wavelet_amd.synthetic import make_inputs
    from level_haar_wavelet_amd.unfused import UnfusedWTConvFunction

    n, c, h, w, k, L = 2, 16, 32, 32, 5, 3
    inp = make_inputs(n, c, h, w, k, L, seed=5)
    dev = torch.device("cuda:0")
    mods = bench.make_block(c, torch.float32)
    grads = []
    for layer in (WTConvFunction.apply, UnfusedWTConvFunction.apply):
        x = torch.from_numpy(inp.x).to(dev).requires_grad_(True)
        params = [torch.from_numpy(a).to(dev).requires_grad_(True)
                  for a in (inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl)]
        for p in mods.parameters():
            p.grad = None
        bench.block_step(mods, layer, x, params)
        grads.append([x.grad.clone()] + [p.grad.clone() for p in params] + [p.grad.clone() for p in mods.parameters()])
    for a, b in zip(*grads):
        rel = float((a - b).norm() / b.norm().clamp_min(1e-30))
        assert rel <= 1e-4, rel
