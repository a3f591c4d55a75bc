"""The C ABI of libwtconv without a GPU: the library loads, exports every
function include/wtconv.h declares, and rejects bad arguments with the
documented status codes before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

from level_haar_wavelet_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wtconv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wtconv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_native.LIB_PATH):
        from level_haar_wavelet_amd import build

        build.build(verbose=False)
    return _native.load()


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert "wtconv_forward" in names and "wtconv_backward_data" in names
    for name in names:
        assert hasattr(lib, name), name


def test_python_binding_names_match_the_abi():
    import level_haar_wavelet_amd as pkg

    for name in pkg.__all__:
        if name.startswith("wtconv_"):
            assert name in declared_functions(), name


def test_version_and_status_strings(lib):
    assert re.match(r"^\d+\.\d+\.\d+$", lib.wtconv_version().decode())
    for code in range(7):
        assert lib.wtconv_status_string(code)


def _ws(lib, d, op=0):
    out = ctypes.c_size_t(123)
    return lib.wtconv_workspace_size(ctypes.byref(d) if d is not None else None, op, ctypes.byref(out)), out.value


@pytest.mark.parametrize("shape,expect", [
    ((2, 8, 16, 16, 5, 2, 0), 0),
    ((2, 8, 16, 16, 4, 2, 0), 3),    # even k
    ((2, 8, 16, 16, 9, 2, 0), 3),    # k not built
    ((2, 8, 16, 16, 5, 7, 0), 2),    # too many levels
    ((2, 8, 16, 16, 5, -1, 0), 2),
    ((0, 8, 16, 16, 5, 2, 0), 2),
    ((2, 8, 16, 16, 5, 2, 2), 3),    # unknown dtype
    ((1, 1, 8192, 16, 5, 2, 0), 2),  # too tall
])
def test_validation(lib, shape, expect):
    st, val = _ws(lib, _native.desc(*shape))
    assert st == expect
    if expect == 0:
        assert val == 0


@pytest.mark.parametrize("shape", [(2, 8, 18, 16, 5, 2, 0), (1, 3, 7, 9, 3, 3, 1), (2, 2, 5, 12, 5, 1, 0)])
def test_ragged_sides_take_padded_copies_in_the_workspace(lib, shape):
    """Sides 2^L does not divide are accepted; every op then needs room for
    two zero-padded activation copies (256-byte aligned) ahead of the padded
    layer's own workspace."""
    n, c, h, w, k, L, dt = shape
    g = 2 ** L
    hp, wp = -(-h // g) * g, -(-w // g) * g
    copy = -(-(n * c * hp * wp * (4 if dt == 0 else 2)) // 256) * 256
    padded = _native.desc(n, c, hp, wp, k, L, dt)
    for op in (0, 1, 2):
        st, val = _ws(lib, _native.desc(*shape), op)
        st_p, val_p = _ws(lib, padded, op)
        assert st == 0 and st_p == 0
        assert val == 2 * copy + val_p


def test_null_arguments_are_rejected_before_any_launch(lib):
    st, _ = _ws(lib, None)
    assert st == 1
    d = _native.desc(2, 8, 16, 16, 5, 2, 0)
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first
    vp = lambda: fake
    # missing x
    assert lib.wtconv_forward(ctypes.byref(d), None, vp(), None, vp(), vp(), vp(), vp(), None, 0, None) == 1
    # missing per-level weights with L > 0
    assert lib.wtconv_forward(ctypes.byref(d), vp(), vp(), None, vp(), None, vp(), ctypes.c_void_p(0x20000),
                              None, 0, None) == 1
    # bad shape wins over anything else
    bad = _native.desc(2, 8, 16, 16, 5, 7, 0)
    assert lib.wtconv_backward_data(ctypes.byref(bad), vp(), vp(), vp(), vp(), vp(), vp(), None, 0, None) == 2
    # odd sides without the workspace for their padded copies
    rag = _native.desc(2, 8, 18, 16, 5, 2, 0)
    assert lib.wtconv_forward(ctypes.byref(rag), vp(), vp(), None, vp(), vp(), vp(), ctypes.c_void_p(0x200000),
                              None, 0, None) == 4
    assert lib.wtconv_backward_weight(ctypes.byref(rag), vp(), ctypes.c_void_p(0x200000), vp(), None, vp(), vp(),
                                      vp(), vp(), vp(), vp(), vp(), vp(), None, 0, None) == 4


def test_alias_and_alignment_are_rejected(lib):
    d = _native.desc(2, 8, 16, 16, 5, 2, 0)
    p = ctypes.c_void_p(0x100000)
    same = lib.wtconv_forward(ctypes.byref(d), p, p, None, p, p, p, p, None, 0, None)
    assert same == 6
    overlap = lib.wtconv_forward(ctypes.byref(d), p, p, None, p, p, p, ctypes.c_void_p(0x100000 + 1024), None, 0,
                                 None)
    assert overlap == 6
    misaligned = lib.wtconv_forward(ctypes.byref(d), ctypes.c_void_p(0x100004), p, None, p, p, p,
                                    ctypes.c_void_p(0x900000), None, 0, None)
    assert misaligned == 3


def test_unfused_binding_names_match_the_abi():
    from level_haar_wavelet_amd import unfused

    for name in unfused.__all__:
        if name.startswith("wtconv_"):
            assert name in declared_functions(), name


def test_unfused_validation_before_any_launch(lib):
    import ctypes

    size = ctypes.c_size_t(0)
    good = _native.desc(2, 3, 16, 16, 5, 2, _native.F32)
    assert lib.wtconv_unfused_workspace_size(ctypes.byref(good), ctypes.byref(size)) == 0 and size.value > 0
    bad = _native.desc(2, 3, 18, 16, 5, 2, _native.F32)  # 18 not divisible by 4 (the baseline needs it)
    assert lib.wtconv_unfused_workspace_size(ctypes.byref(bad), ctypes.byref(size)) == 2
    # null pointers and a short workspace are rejected before anything is launched
    assert lib.wtconv_unfused_forward(ctypes.byref(good), None, None, None, None, None, None, None, None, 0,
                                      None) == 1
    one = ctypes.c_void_p(16)
    assert lib.wtconv_unfused_forward(ctypes.byref(good), one, one, None, one, one, one, one, one, 8, None) == 4


def _no_device():
    import torch

    return torch.cuda.device_count() == 0


def _fake(addr):
    return ctypes.c_void_p(addr)


@pytest.mark.skipif(not _no_device(), reason="calls the ops with fake pointers: only where no GPU is visible")
def test_nested_plan_is_checked_before_anything_is_enqueued(lib, monkeypatch):
    """A 272 x 272 plane tiles (16 x 16), but its 136 x 136 level-1 low-pass
    map fits neither one workgroup nor a tile shape; with the strip fallbacks
    taken away (WTCONV_NO_STRIPS) the nested call for the deeper levels has no
    plan.  The whole recursion is planned before the first launch, so the call
    returns WTCONV_ERR_UNSUPPORTED; were the level-1 low-pass pass launched
    first, the GPU-less runtime would report WTCONV_ERR_HIP instead."""
    monkeypatch.setenv("WTCONV_NO_STRIPS", "1")
    d = _native.desc(1, 2, 272, 272, 5, 2, _native.F32)
    st, need = _ws(lib, d, 0)
    assert st == 0 and need > 0
    p = _fake(0x10000000)
    out = _fake(0x20000000)
    ws = _fake(0x40000000)
    assert lib.wtconv_forward(ctypes.byref(d), p, p, None, p, p, p, out, ws, need, None) == 3
    assert lib.wtconv_backward_data(ctypes.byref(d), p, p, p, p, p, out, ws, need, None) == 3
    st, _ = _ws(lib, d, 2)
    assert st == 3
    assert lib.wtconv_backward_weight(ctypes.byref(d), p, out, p, None, p, p, p, p, p, p, p, p, ws, 1 << 40,
                                      None) == 3


@pytest.mark.skipif(not _no_device(), reason="calls the ops with fake pointers: only where no GPU is visible")
@pytest.mark.parametrize("shape", [(1, 2, 128, 128, 5, 3, 0), (2, 1, 256, 256, 5, 4, 1), (1, 1, 128, 256, 3, 5, 1)])
def test_workspace_size_is_what_the_launch_plan_needs(lib, monkeypatch, shape):
    """For every LDS budget of the whole-plane and tiled plans
    (WTCONV_WHOLE_LDS_KB, which moves the choice between whole planes, tiles
    and the nested calls with and without their base path), the size that
    wtconv_workspace_size reports is exactly what the call checks: 256 bytes
    less is refused with WTCONV_ERR_WORKSPACE before anything is enqueued,
    the reported size passes every check (the GPU-less runtime then fails the
    first launch: WTCONV_ERR_HIP)."""
    d = _native.desc(*shape)
    p, out, ws = _fake(0x10000000), _fake(0x80000000), _fake(0x100000000)
    seen = 0
    for kb in range(8, 161, 2):
        monkeypatch.setenv("WTCONV_WHOLE_LDS_KB", str(kb))
        for op in (0, 1):
            st, need = _ws(lib, d, op)
            if st != 0:
                continue
            call = (lambda n: lib.wtconv_forward(ctypes.byref(d), p, p, None, p, p, p, out, ws, n, None)) if op == 0 \
                else (lambda n: lib.wtconv_backward_data(ctypes.byref(d), p, p, p, p, p, out, ws, n, None))
            if need > 0:
                seen += 1
                assert call(need - 256) == 4, (kb, op, need)
            assert call(need) == 5, (kb, op, need)
        st, need = _ws(lib, d, 2)
        if st == 0:
            assert lib.wtconv_backward_weight(ctypes.byref(d), p, out, p, None, p, p, p, p, p, p, p, p, ws,
                                              need - 256, None) == 4
            assert lib.wtconv_backward_weight(ctypes.byref(d), p, out, p, None, p, p, p, p, p, p, p, p, ws, need,
                                              None) == 5
    assert seen > 0
