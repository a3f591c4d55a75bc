"""Helpers of the GPU parity tests: device copies of seeded inputs, the
tolerances, and the comparison against the oracle."""
import numpy as np
import torch

import level_haar_wavelet_amd as wt

# Tolerances: fp32 outputs max |err| <= 1e-4 (1 + |ref|) elementwise; fp32 weight
# gradients relative L2 <= 1e-4 per tensor; fp16 storage: relative L2 <= 5e-3
# per tensor and, elementwise, max |err| <= 4 * 2^-11 (1 + |ref|): an fp16
# output is the fp32 result rounded once (half an ulp is 2^-11 relative), so a
# wrong row, band or tile edge that the tensor-wide norm would average away
# still fails.  Gradients are also checked per channel (per row of dw, per
# entry of db and ds) against the same tolerance, with a floor of a tenth of
# the rows' RMS norm for rows that nearly cancel.
TOL_F32_ELEM = 1e-4
TOL_F32_GRAD_L2 = 1e-4
TOL_F16_L2 = 5e-3
TOL_F16_ELEM = 4 * 2.0 ** -11


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


def _np64(got):
    return got.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(got) else np.asarray(got)


def assert_close(got, ref, act_dtype, what=""):
    got = _np64(got)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), what + ": non-finite output"
    err = np.abs(got - ref) / (1.0 + np.abs(ref))
    worst = np.unravel_index(np.argmax(err), err.shape)
    tol = TOL_F32_ELEM if act_dtype == "f32" else TOL_F16_ELEM
    assert err.max() <= tol, "%s: max scaled err %.3e > %.2e at %s (got %r ref %r)" % (
        what, err.max(), tol, worst, got[worst], ref[worst])
    if act_dtype != "f32":
        rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
        assert rel <= TOL_F16_L2, "%s: rel L2 %.3e" % (what, rel)


def assert_grad_close(got, ref, act_dtype, what="", per_channel=True):
    got = _np64(got)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), what
    tol = TOL_F32_GRAD_L2 if act_dtype == "f32" else TOL_F16_L2
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= tol, "%s: rel L2 %.3e > %.1e" % (what, rel, tol)
    if not per_channel:
        return
    # per channel: one row per channel (and band) -- the k*k taps of dw_base
    # (C, k, k) and dw_lvl (L, 4C, k, k), one entry of dbias, ds_base (C) and
    # ds_lvl (L, 4C)
    width = ref.shape[-1] * ref.shape[-2] if ref.ndim >= 3 else 1
    g2, r2 = got.reshape(-1, width), ref.reshape(-1, width)
    en = np.linalg.norm(g2 - r2, axis=1)
    rn = np.linalg.norm(r2, axis=1)
    floor = 0.1 * np.sqrt(np.mean(rn ** 2))
    ratio = en / (tol * np.maximum(rn, floor))
    worst = int(np.argmax(ratio))
    assert ratio.max() <= 1.0, "%s: %d of %d channel rows off, worst row %d: err %.3e ref norm %.3e" % (
        what, int((ratio > 1.0).sum()), len(rn), worst, en[worst], rn[worst])


def backward_weight(d, **kw):
    return wt.wtconv_backward_weight(d.x, d.dy, d.w_base, d.bias, d.s_base, d.w_lvl, d.s_lvl, **kw)


GRAD_NAMES = ("dw_base", "dbias", "ds_base", "dw_lvl", "ds_lvl")


def assert_grads_close(got, ref, act_dtype, what="", per_channel=True):
    for name, g, r in zip(GRAD_NAMES, got, ref):
        if r is None or np.asarray(r).size == 0:
            continue
        assert_grad_close(g, np.asarray(r), act_dtype, "%s %s" % (what, name), per_channel)
