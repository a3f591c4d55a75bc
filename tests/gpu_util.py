"""Helpers of the GPU parity tests: device copies of seeded inputs, the
tolerances, and the comparison against the oracle."""
import numpy as np
import torch

import level_haar_wavelet_amd as wt

# Tolerances: fp32 outputs max |err| <= 1e-4 (1 + |ref|) elementwise; fp32 weight
# gradients relative L2 <= 1e-4 per tensor; fp16 storage: relative L2 <= 5e-3.
TOL_F32_ELEM = 1e-4
TOL_F32_GRAD_L2 = 1e-4
TOL_F16_L2 = 5e-3


def dev(a, dtype=torch.float32):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dtype)


class DevInputs:
    def __init__(self, inp, act_dtype="f32"):
        tdt = torch.float32 if act_dtype == "f32" else torch.float16
        self.x = dev(inp.x, tdt)
        self.dy = dev(inp.dy, tdt)
        self.w_base = dev(inp.w_base)
        self.bias = dev(inp.bias)
        self.s_base = dev(inp.s_base)
        L = inp.w_lvl.shape[0]
        self.w_lvl = dev(inp.w_lvl) if L > 0 else None
        self.s_lvl = dev(inp.s_lvl) if L > 0 else None


def forward(d, **kw):
    return wt.wtconv_forward(d.x, d.w_base, d.bias, d.s_base, d.w_lvl, d.s_lvl, **kw)


def backward_data(d, **kw):
    return wt.wtconv_backward_data(d.dy, d.w_base, d.s_base, d.w_lvl, d.s_lvl, **kw)


def assert_close(got, ref, act_dtype, what=""):
    got = got.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(got) else got
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), what + ": non-finite output"
    if act_dtype == "f32":
        err = np.abs(got - ref) / (1.0 + np.abs(ref))
        worst = np.unravel_index(np.argmax(err), err.shape)
        assert err.max() <= TOL_F32_ELEM, "%s: max scaled err %.3e at %s (got %r ref %r)" % (
            what, err.max(), worst, got[worst], ref[worst])
    else:
        rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
        assert rel <= TOL_F16_L2, "%s: rel L2 %.3e" % (what, rel)


def assert_grad_close(got, ref, act_dtype, what=""):
    got = got.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(got) else got
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), what
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    tol = TOL_F32_GRAD_L2 if act_dtype == "f32" else TOL_F16_L2
    assert rel <= tol, "%s: rel L2 %.3e > %.1e" % (what, rel, tol)


def backward_weight(d, **kw):
    return wt.wtconv_backward_weight(d.x, d.dy, d.w_base, d.bias, d.s_base, d.w_lvl, d.s_lvl, **kw)


GRAD_NAMES = ("dw_base", "dbias", "ds_base", "dw_lvl", "ds_lvl")


def assert_grads_close(got, ref, act_dtype, what=""):
    for name, g, r in zip(GRAD_NAMES, got, ref):
        if r is None or np.asarray(r).size == 0:
            continue
        assert_grad_close(g, np.asarray(r), act_dtype, "%s %s" % (what, name))
