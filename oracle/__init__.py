"""Python loader for the CPU oracle of the WTConv layer (test infrastructure).

Only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``level_haar_wavelet_amd``) never imports it.

The oracle itself is plain C in ``wtconv_oracle.c``, computing in double.  The
wrappers here only marshal numpy arrays (converted to float64, C-contiguous) and
return numpy float64 results.  See the header of ``wtconv_oracle.c`` for the
definition of the layer, the readings of the pages it takes, and the parameter
layout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wtconv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_wtconv.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math) into liboracle_wtconv.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-Wall", "-Wextra",
               "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        d = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        lib.oracle_wtconv_forward.argtypes = [i64, i64, i64, i64, ci, ci, d, d, d, d, d, d, d, ci]
        lib.oracle_wtconv_backward_data.argtypes = [i64, i64, i64, i64, ci, ci, d, d, d, d, d, d, ci]
        lib.oracle_wtconv_backward_weight.argtypes = [i64, i64, i64, i64, ci, ci, d, d, d, d, d, d, d,
                                                      d, d, d, d, d, ci]
        lib.oracle_wtconv_level_outputs.argtypes = [i64, i64, ci, ci, d, d, d, d]
        lib.oracle_haar_analysis.argtypes = [d, i64, i64, d]
        lib.oracle_haar_synthesis.argtypes = [d, i64, i64, d]
        lib.oracle_corr_same.argtypes = [d, i64, i64, d, ci, d]
        for name in ("oracle_wtconv_forward", "oracle_wtconv_backward_data",
                     "oracle_wtconv_backward_weight", "oracle_wtconv_level_outputs",
                     "oracle_haar_analysis", "oracle_haar_synthesis", "oracle_corr_same"):
            getattr(lib, name).restype = ci
        _lib = lib
    return _lib


def _d(a):
    """float64 C-contiguous copy/view of a, and its pointer (None -> NULL)."""
    if a is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    return max(1, min(64, os.cpu_count() or 1))


def _check(rc, what):
    if rc != 0:
        raise ValueError("%s failed with code %d" % (what, rc))


def _shape(x):
    n, c, h, w = x.shape
    return int(n), int(c), int(h), int(w)


def _params(k, levels, c, w_base, bias, s_base, w_lvl, s_lvl):
    w0, pw0 = _d(np.reshape(w_base, (c, k, k)))
    b0, pb0 = _d(None if bias is None else np.reshape(bias, (c,)))
    s0, ps0 = _d(np.reshape(s_base, (c,)))
    if levels > 0:
        wl, pwl = _d(np.reshape(w_lvl, (levels, 4 * c, k, k)))
        sl, psl = _d(np.reshape(s_lvl, (levels, 4 * c)))
    else:
        wl, pwl = _d(np.zeros(1))
        sl, psl = _d(np.zeros(1))
    keep = (w0, b0, s0, wl, sl)
    return keep, (pw0, pb0, ps0, pwl, psl)


def forward(x, w_base, bias, s_base, w_lvl, s_lvl, k, levels, nthreads=None):
    """y = WTConv(x) in double; x is (N, C, H, W)."""
    lib = _load()
    n, c, h, w = _shape(x)
    xd, px = _d(x)
    keep, (pw0, pb0, ps0, pwl, psl) = _params(k, levels, c, w_base, bias, s_base, w_lvl, s_lvl)
    y = np.empty((n, c, h, w), dtype=np.float64)
    py = y.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    rc = lib.oracle_wtconv_forward(n, c, h, w, k, levels, px, pw0, pb0, ps0, pwl, psl, py,
                                   nthreads or default_threads())
    _check(rc, "oracle_wtconv_forward")
    del keep, xd
    return y


def backward_data(dy, w_base, s_base, w_lvl, s_lvl, k, levels, nthreads=None):
    """dx = d<dy, WTConv(x)>/dx in double."""
    lib = _load()
    n, c, h, w = _shape(dy)
    dyd, pdy = _d(dy)
    keep, (pw0, _pb0, ps0, pwl, psl) = _params(k, levels, c, w_base, None, s_base, w_lvl, s_lvl)
    dx = np.empty((n, c, h, w), dtype=np.float64)
    pdx = dx.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    rc = lib.oracle_wtconv_backward_data(n, c, h, w, k, levels, pdy, pw0, ps0, pwl, psl, pdx,
                                         nthreads or default_threads())
    _check(rc, "oracle_wtconv_backward_data")
    del keep, dyd
    return dx


def backward_weight(x, dy, w_base, bias, s_base, w_lvl, s_lvl, k, levels, nthreads=None):
    """Parameter gradients of <dy, WTConv(x)>: (dw_base, dbias, ds_base, dw_lvl, ds_lvl)."""
    lib = _load()
    n, c, h, w = _shape(x)
    xd, px = _d(x)
    dyd, pdy = _d(dy)
    keep, (pw0, pb0, ps0, pwl, psl) = _params(k, levels, c, w_base, bias, s_base, w_lvl, s_lvl)
    dw0 = np.empty((c, k, k))
    db0 = np.empty((c,))
    ds0 = np.empty((c,))
    dwl = np.empty((max(levels, 1), 4 * c, k, k))
    dsl = np.empty((max(levels, 1), 4 * c))
    P = ctypes.POINTER(ctypes.c_double)
    rc = lib.oracle_wtconv_backward_weight(
        n, c, h, w, k, levels, px, pdy, pw0, pb0, ps0, pwl, psl,
        dw0.ctypes.data_as(P), db0.ctypes.data_as(P), ds0.ctypes.data_as(P),
        dwl.ctypes.data_as(P), dsl.ctypes.data_as(P), nthreads or default_threads())
    _check(rc, "oracle_wtconv_backward_weight")
    del keep, xd, dyd
    return dw0, db0, ds0, dwl[:levels], dsl[:levels]


def level_outputs(xplane, wl_c, sl_c, k, levels):
    """Scaled band outputs Z_l^b of one plane: list over l of arrays
    (4, ceil(H / 2^l), ceil(W / 2^l))."""
    lib = _load()
    h, w = xplane.shape
    xd, px = _d(xplane)
    wd, pw = _d(np.reshape(wl_c, (levels, 4, k, k)))
    sd, ps = _d(np.reshape(sl_c, (levels, 4)))
    dim = lambda n, l: -(-n // (1 << l))
    total = sum(4 * dim(h, l) * dim(w, l) for l in range(1, levels + 1))
    z = np.empty(total)
    rc = lib.oracle_wtconv_level_outputs(h, w, k, levels, px, pw, ps,
                                         z.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    _check(rc, "oracle_wtconv_level_outputs")
    out, off = [], 0
    for l in range(1, levels + 1):
        m = 4 * dim(h, l) * dim(w, l)
        out.append(z[off:off + m].reshape(4, dim(h, l), dim(w, l)))
        off += m
    del xd, wd, sd
    return out


def haar_analysis(plane):
    """One Haar analysis level of an (H, W) map -> (4, H/2, W/2)."""
    lib = _load()
    h, w = plane.shape
    xd, px = _d(plane)
    out = np.empty((4, h // 2, w // 2))
    _check(lib.oracle_haar_analysis(px, h, w, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))),
           "oracle_haar_analysis")
    del xd
    return out


def haar_synthesis(bands):
    """One Haar synthesis level of (4, h, w) bands -> (2h, 2w)."""
    lib = _load()
    _, h, w = bands.shape
    bd, pb = _d(bands)
    out = np.empty((2 * h, 2 * w))
    _check(lib.oracle_haar_synthesis(pb, h, w, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))),
           "oracle_haar_synthesis")
    del bd
    return out


def corr_same(plane, kern):
    """Zero-padded 'same' cross-correlation of one (H, W) map with a (k, k) kernel."""
    lib = _load()
    h, w = plane.shape
    k = kern.shape[0]
    xd, px = _d(plane)
    kd, pk = _d(kern)
    out = np.empty((h, w))
    _check(lib.oracle_corr_same(px, h, w, pk, k, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))),
           "oracle_corr_same")
    del xd, kd
    return out
