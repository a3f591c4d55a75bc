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
