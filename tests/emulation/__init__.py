"""Loader of the CPU emulation of the fused kernels (test tool, see wtconv_emu.cpp)."""
import ctypes
import os
import shutil
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(os.path.dirname(_HERE))
_SRC = os.path.join(_HERE, "wtconv_emu.cpp")
_DEPS = [_SRC] + [os.path.join(_ROOT, "level_haar_wavelet_amd", "csrc", f)
                  for f in ("wtconv_fused_body.h", "wtconv_plan.h", "wtconv_whole_body.h", "wtconv_wgrad_body.h",
                            "wtconv_wgrad_tile_body.h", "wtconv_large_body.h", "wtconv_bwd_body.h")]
_LIB = os.path.join(_ROOT, "_build", "libwtconv_emu.so")
_lib = None


def _compiler():
    for cand in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if cand and os.path.exists(cand):
            return cand
    return None


def available():
    return _compiler() is not None


def build():
    stale = not os.path.exists(_LIB) or any(os.path.getmtime(d) > os.path.getmtime(_LIB) for d in _DEPS)
    if stale:
        os.makedirs(os.path.dirname(_LIB), exist_ok=True)
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run([_compiler(), "-std=c++17", "-O2", "-fno-strict-aliasing", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        vp = ctypes.c_void_p
        ci = ctypes.c_int
        lib.emu_fused.argtypes = [ci, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, ci, ci]
        lib.emu_fused.restype = ci
        lib.emu_fused_plan.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(ci)]
        lib.emu_fused_plan.restype = ci
        lib.emu_whole.argtypes = [ci, vp, vp, ci, ci, ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci]
        lib.emu_whole.restype = ci
        lib.emu_whole_tiled.argtypes = [ci, vp, vp, vp] + [ci] * 9 + [vp] * 5 + [ci, ci, ci, ci]
        lib.emu_whole_tiled.restype = ci
        lib.emu_whole_plan.argtypes = [ci] * 12 + [ctypes.POINTER(ci)]
        lib.emu_wgrad_tiles.argtypes = [ci, vp, vp] + [ci] * 8 + [vp] * 12 + [ci, ci, ci, ci]
        lib.emu_wgrad_tiles.restype = ci
        lib.emu_whole_plan.restype = ci
        lib.emu_wgrad.argtypes = [ci, vp, vp] + [ci] * 6 + [vp] * 10 + [ci, ci, ci, ci]
        lib.emu_wgrad.restype = ci
        lib.emu_wgrad_plan.argtypes = [ci] * 10 + [ctypes.POINTER(ci)]
        lib.emu_wgrad_plan.restype = ci
        lib.emu_wgrad_tiled.argtypes = [ci, vp, vp] + [ci] * 6 + [vp] * 10 + [ci, ci, ci]
        lib.emu_wgrad_tiled.restype = ci
        lib.emu_large.argtypes = [ci, vp, vp] + [ci] * 9 + [vp] * 5 + [ci, ci, ci, ctypes.POINTER(ci)]
        lib.emu_large.restype = ci
        lib.emu_bwd.argtypes = [ci, vp, vp, vp] + [ci] * 6 + [vp] * 10 + [ci, ci, ci]
        lib.emu_bwd.restype = ci
        _lib = lib
    return _lib


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def fused_plan(n, c, h, w, k, levels, rotate=0, nthreads=256, budget_floats=16384):
    out = (ctypes.c_int * 8)()
    rc = _load().emu_fused_plan(n, c, h, w, k, levels, rotate, nthreads, budget_floats, out)
    if rc != 0:
        raise ValueError("no plan")
    keys = ("tile_h", "tile_w", "strip_h", "out_bw", "tiles_y", "tiles_x", "lds_floats", "nthreads")
    return dict(zip(keys, list(out)))


def fused(x, w_base, bias, s_base, w_lvl, s_lvl, k, levels, rotate=0, dtype="f32", nthreads=256,
          budget_floats=16384):
    """Run the fused pass on the CPU emulation.  x: (N, C, H, W) float array."""
    lib = _load()
    n, c, h, w = x.shape
    npdt = np.float32 if dtype == "f32" else np.float16
    xin = np.ascontiguousarray(x, dtype=npdt)
    out = np.full_like(xin, np.nan)
    keep = [_f32(w_base), _f32(bias), _f32(s_base), _f32(w_lvl), _f32(s_lvl)]
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib.emu_fused(0 if dtype == "f32" else 1, xin.ctypes.data, out.ctypes.data, n, c, h, w, k, levels,
                       rotate, *[ptr(a) for a in keep], nthreads, budget_floats)
    if rc != 0:
        raise ValueError("emu_fused failed: %d" % rc)
    return out.astype(np.float64)


def whole_plan(n, c, h, w, k, levels, rotate=0, nthreads=256, planes=1, dtype="f32", budget_floats=40960, stack=1):
    out = (ctypes.c_int * 12)()
    rc = _load().emu_whole_plan(n, c, h, w, k, levels, rotate, nthreads, planes, 4 if dtype == "f32" else 2,
                                budget_floats, stack, out)
    keys = ("planes", "vec", "out_bw", "lds_floats", "items", "nthreads", "ok", "stage_l3", "rows", "gap", "units",
            "tail")
    d = dict(zip(keys, list(out)))
    d["ok"] = rc == 0
    return d


def whole(x, w_base, bias, s_base, w_lvl, s_lvl, k, levels, rotate=0, dtype="f32", nthreads=256, planes=1,
          budget_floats=40960, nobase=False, stack=1):
    """Run the whole-plane kernel on the CPU emulation (nobase: without the
    base path, as in the nested call for the deeper levels; stack: images
    stacked per plane)."""
    lib = _load()
    n, c, h, w = x.shape
    npdt = np.float32 if dtype == "f32" else np.float16
    xin = np.ascontiguousarray(x, dtype=npdt)
    out = np.full_like(xin, np.nan)
    keep = [_f32(w_base), _f32(bias), _f32(s_base), _f32(w_lvl), _f32(s_lvl)]
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib.emu_whole(0 if dtype == "f32" else 1, xin.ctypes.data, out.ctypes.data, n, c, h, w, k, levels,
                       rotate, *[ptr(a) for a in keep], nthreads, planes, budget_floats, int(nobase), stack)
    if rc != 0:
        raise ValueError("emu_whole failed: %d" % rc)
    return out.astype(np.float64)


def whole_tiled(x, low, w_base, bias, s_base, w_lvl, s_lvl, k, th, tw, rotate=0, dtype="f32", nthreads=256, planes=1,
                budget_floats=40960, nobase=False):
    """Run the tiled whole-plane kernel (base and level-1 convolutions on th x tw
    tiles, plus the deeper levels' low-pass term `low`) on the CPU emulation.
    w_lvl / s_lvl: the level-1 weights and scales (1, 4C, k, k) / (1, 4C), or
    None for L = 0 (the base convolution alone)."""
    lib = _load()
    n, c, ih, iw = x.shape
    npdt = np.float32 if dtype == "f32" else np.float16
    xin = np.ascontiguousarray(x, dtype=npdt)
    lin = None if low is None else np.ascontiguousarray(low, dtype=np.float32)  # fp32 intermediate
    out = np.full_like(xin, np.nan)
    keep = [_f32(w_base), _f32(bias), _f32(s_base), _f32(w_lvl), _f32(s_lvl)]
    ptr = lambda a: None if a is None else a.ctypes.data
    levels = 0 if w_lvl is None else 1
    rc = lib.emu_whole_tiled(0 if dtype == "f32" else 1, xin.ctypes.data, out.ctypes.data, ptr(lin), n, c, ih, iw,
                             th, tw, k, levels, rotate, *[ptr(a) for a in keep], nthreads, planes, budget_floats,
                             int(nobase))
    if rc != 0:
        raise ValueError("emu_whole_tiled failed: %d" % rc)
    return out.astype(np.float64)


def wgrad_tiles(x, dy, w_base, bias, s_base, w_lvl, s_lvl, k, th, tw, dtype="f32", nthreads=256, planes=1,
                budget_floats=40960, lowpass=False, nobase=False):
    """Base and level-1 parameter gradients through the emulated tiled
    weight-gradient pass (w_lvl / s_lvl: level 1 only, or None for L = 0);
    with lowpass=True also the level-1 low-pass maps of x and dy it writes."""
    lib = _load()
    n, c, ih, iw = x.shape
    npdt = np.float32 if dtype == "f32" else np.float16
    xin = np.ascontiguousarray(x, dtype=npdt)
    dyin = np.ascontiguousarray(dy, dtype=npdt)
    keep = [_f32(w_base), _f32(bias), _f32(s_base), _f32(w_lvl), _f32(s_lvl)]
    levels = 0 if w_lvl is None else 1
    outs = [np.full((c, k, k), np.nan, np.float32), np.full((c,), np.nan, np.float32),
            np.full((c,), np.nan, np.float32), np.full((1, 4 * c, k, k), np.nan, np.float32),
            np.full((1, 4 * c), np.nan, np.float32)][:3 + 2 * levels]
    ptr = lambda a: None if a is None else a.ctypes.data
    optr = [o.ctypes.data for o in outs] + [None] * (5 - len(outs))
    lls = [np.full((n, c, ih // 2, iw // 2), np.nan, np.float32) for _ in range(2)] if lowpass else [None, None]
    rc = lib.emu_wgrad_tiles(0 if dtype == "f32" else 1, xin.ctypes.data, dyin.ctypes.data, n, c, ih, iw, th, tw, k,
                             levels, *[ptr(a) for a in keep], *optr, *[ptr(a) for a in lls], nthreads, planes,
                             budget_floats, int(nobase))
    if rc != 0:
        raise ValueError("emu_wgrad_tiles failed: %d" % rc)
    res = [o.astype(np.float64) for o in outs]
    return (res, [a.astype(np.float64) for a in lls]) if lowpass else res


def wgrad_plan(n, c, h, w, k, levels, nthreads=256, planes=1, dtype="f32", budget_floats=40960):
    out = (ctypes.c_int * 7)()
    rc = _load().emu_wgrad_plan(n, c, h, w, k, levels, nthreads, planes, 4 if dtype == "f32" else 2,
                                budget_floats, out)
    keys = ("lds_floats", "npieces", "q", "groups", "plen", "vec", "tail")
    d = dict(zip(keys, list(out)))
    d["ok"] = rc == 0
    return d


def choose_planes(n, c, slots, fixed):
    lib = _load()
    lib.emu_choose_planes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double]
    return lib.emu_choose_planes(n, c, slots, fixed)


def wgrad(x, dy, w_base, bias, s_base, w_lvl, s_lvl, k, levels, dtype="f32", nthreads=256, planes=1,
          budget_floats=40960, tiled=False, nobase=False):
    """Parameter gradients through the emulated fused weight-gradient kernel
    (nobase: the base gradients skipped and written as 0; whole-plane only)."""
    lib = _load()
    n, c, h, w = x.shape
    npdt = np.float32 if dtype == "f32" else np.float16
    xin = np.ascontiguousarray(x, dtype=npdt)
    dyin = np.ascontiguousarray(dy, dtype=npdt)
    keep = [_f32(w_base), _f32(bias), _f32(s_base), _f32(w_lvl if levels else np.zeros(1)),
            _f32(s_lvl if levels else np.zeros(1))]
    outs = [np.full((c, k, k), np.nan, np.float32), np.full((c,), np.nan, np.float32),
            np.full((c,), np.nan, np.float32), np.full((max(levels, 1), 4 * c, k, k), np.nan, np.float32),
            np.full((max(levels, 1), 4 * c), np.nan, np.float32)]
    ptr = lambda a: None if a is None else a.ctypes.data
    fn = lib.emu_wgrad_tiled if tiled else lib.emu_wgrad
    rc = fn(0 if dtype == "f32" else 1, xin.ctypes.data, dyin.ctypes.data, n, c, h, w, k, levels,
            *[ptr(a) for a in keep], *[o.ctypes.data for o in outs], nthreads, planes, budget_floats,
            *(() if tiled else (int(nobase),)))
    if rc != 0:
        raise ValueError("emu_wgrad failed: %d" % rc)
    outs[3] = outs[3][:levels]
    outs[4] = outs[4][:levels]
    return [o.astype(np.float64) for o in outs]


def large(x, w_base, bias, s_base, w_lvl, s_lvl, k, levels, th, tw, rotate=0, dtype="f32", planes=1,
          budget_floats=40960, nobase=False):
    """Run the fused large-plane kernel (deeper levels staged from x and kept
    on chip, base and level 1 on th x tw tiles; nobase: without the base path)
    on the CPU emulation.  Returns (output, info) with info = images per
    workgroup, LDS floats, deeper-levels map floats, tiles per image, and the
    pieces and one-row tail pieces of the deeper-levels and tile plans, and
    whether the tiles run their pieces as 2-row halves."""
    lib = _load()
    n, c, h, w = x.shape
    npdt = np.float32 if dtype == "f32" else np.float16
    xin = np.ascontiguousarray(x, dtype=npdt)
    out = np.full_like(xin, np.nan)
    keep = [_f32(w_base), _f32(bias), _f32(s_base), _f32(w_lvl), _f32(s_lvl)]
    ptr = lambda a: None if a is None else a.ctypes.data
    info = (ctypes.c_int * 9)()
    rc = lib.emu_large(0 if dtype == "f32" else 1, xin.ctypes.data, out.ctypes.data, n, c, h, w, th, tw, k, levels,
                       rotate, *[ptr(a) for a in keep], planes, budget_floats, int(bool(nobase)), info)
    if rc != 0:
        raise ValueError("emu_large failed: %d" % rc)
    return out.astype(np.float64), list(info)


def large_plan(n, c, h, w, th, tw, k, levels, dtype="f32", planes=1, budget_floats=40960, nobase=False):
    info = (ctypes.c_int * 9)()
    rc = _load().emu_large(0 if dtype == "f32" else 1, None, None, n, c, h, w, th, tw, k, levels, 0, None, None, None,
                           None, None, planes, budget_floats, int(bool(nobase)), info)
    return None if rc != 0 else list(info)


def bwd(x, dy, w_base, bias, s_base, w_lvl, s_lvl, k, dtype="f32", nthreads=512, planes=1,
        budget_floats=40960):
    """The fused single-pass backward on the CPU emulation: (dx, [dw_base,
    dbias, ds_base, dw_lvl, ds_lvl])."""
    lib = _load()
    n, c, h, w = x.shape
    levels = w_lvl.shape[0]
    npdt = np.float32 if dtype == "f32" else np.float16
    xin = np.ascontiguousarray(x, dtype=npdt)
    dyin = np.ascontiguousarray(dy, dtype=npdt)
    dx = np.full_like(xin, np.nan)
    keep = [_f32(w_base), _f32(bias), _f32(s_base), _f32(w_lvl), _f32(s_lvl)]
    outs = [np.full((c, k, k), np.nan, np.float32), np.full((c,), np.nan, np.float32),
            np.full((c,), np.nan, np.float32), np.full((levels, 4 * c, k, k), np.nan, np.float32),
            np.full((levels, 4 * c), np.nan, np.float32)]
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib.emu_bwd(0 if dtype == "f32" else 1, xin.ctypes.data, dyin.ctypes.data, dx.ctypes.data, n, c, h, w, k,
                     levels, *[ptr(a) for a in keep], *[o.ctypes.data for o in outs], nthreads, planes,
                     budget_floats)
    if rc != 0:
        raise ValueError("emu_bwd failed: %d" % rc)
    return dx.astype(np.float64), [o.astype(np.float64) for o in outs]
