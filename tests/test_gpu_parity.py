"""GPU parity: libwtconv against the CPU oracle, element by element, on the
same seeded inputs, through the C ABI.  Small shapes span several tiles, strips
and ragged edges; the workload shapes are compared in full where the oracle is
fast enough and on sampled planes otherwise."""
import sys

import numpy as np
import pytest
import torch

from level_haar_wavelet_amd.synthetic import WORKLOADS, make_inputs, sweep_workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests.gpu_util import (DevInputs, assert_close, assert_grad_close, assert_grads_close, backward_data,
                                backward_weight, forward)


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SMALL = [
    # n, c, h, w, k, L, dtype
    (2, 8, 16, 16, 5, 2, "f32"),
    (1, 3, 16, 24, 3, 3, "f32"),
    (2, 2, 8, 8, 7, 1, "f32"),
    (1, 4, 12, 20, 1, 2, "f32"),
    (2, 3, 10, 14, 5, 1, "f32"),
    (1, 2, 64, 48, 5, 4, "f32"),
    (1, 2, 32, 32, 5, 5, "f32"),
    (1, 1, 64, 64, 3, 6, "f32"),
    (2, 3, 9, 13, 5, 0, "f32"),
    (2, 3, 16, 16, 7, 0, "f16"),
    (2, 8, 16, 16, 5, 2, "f16"),
    (1, 3, 24, 40, 3, 3, "f16"),
    (1, 2, 28, 28, 5, 2, "f16"),
    (1, 2, 96, 160, 5, 4, "f32"),
]


# the largest side the ABI takes (WTCONV_MAX_SIDE) with the most levels: the
# tiled passes and their nested calls on the low-pass maps recurse down to
# planes one workgroup holds
MAXIMUM = [
    (1, 2, 4096, 64, 5, 6, "f32"),
    (1, 1, 64, 4096, 3, 6, "f16"),
    (1, 1, 4096, 4096, 5, 6, "f16"),
    (1, 1, 4096, 64, 7, 6, "f32"),
    (2, 1, 64, 4096, 1, 6, "f32"),
    (1, 1, 4095, 65, 5, 6, "f32"),   # ragged: zero-padded to 4096 x 128
]


@pytest.mark.parametrize("case", MAXIMUM, ids=lambda c: "x".join(map(str, c)))
def test_maximum_side_and_levels(orc, case):
    n, c, h, w, k, L, dt = case
    _log("case %s" % (case,))
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h + 2 * w + k + L)
    d = DevInputs(inp, dt)
    y = forward(d)
    dx = backward_data(d)
    grads = backward_weight(d)
    torch.cuda.synchronize()
    ref_y = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    assert_close(y, ref_y, dt, "y")
    ref_dx = orc.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    assert_close(dx, ref_dx, dt, "dx")
    ref_g = orc.backward_weight(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    assert_grads_close(grads, ref_g, dt, str(case))


# the level sweep's 128 x 128 planes with the other kernel sizes: the fused
# large-plane kernel's k = 1, 3 and 7 instances (one per deeper-levels count
# where L - 1 <= 3, the generic one beyond), the tiled weight pass and its
# nested call, at their real shape
SWEEP_K = [
    (2, 3, 128, 128, 3, 2, "f32"),
    (2, 3, 128, 128, 7, 5, "f32"),
    (1, 2, 128, 128, 7, 2, "f32"),
    (2, 3, 128, 128, 7, 3, "f16"),
    (2, 3, 128, 128, 1, 4, "f16"),
    (1, 2, 128, 128, 3, 5, "f16"),
]


@pytest.mark.parametrize("case", SWEEP_K, ids=lambda c: "x".join(map(str, c)))
def test_sweep_planes_other_kernel_sizes(orc, case):
    test_maximum_side_and_levels(orc, case)


# the 256 x 256 planes (tiles plus a nested call on the 128 x 128 level-1
# map, itself fused without its base path) with the other kernel sizes
LARGE_K = [
    (1, 2, 256, 256, 7, 3, "f32"),
    (1, 2, 256, 256, 3, 5, "f16"),
    (1, 1, 256, 256, 1, 2, "f32"),
    (1, 1, 256, 256, 7, 4, "f16"),
]


@pytest.mark.parametrize("case", LARGE_K, ids=lambda c: "x".join(map(str, c)))
def test_large_planes_other_kernel_sizes(orc, case):
    test_maximum_side_and_levels(orc, case)


# degenerate shapes: single pixels, 2-pixel sides, level maps of one pixel,
# planes one pixel wide or high, ragged sides smaller than 2^L, many channels
DEGENERATE = [
    (1, 1, 1, 1, 5, 0, "f32"),
    (1, 3, 1, 7, 5, 0, "f16"),
    (1, 1, 4096, 1, 5, 0, "f32"),
    (3, 2, 2, 2, 3, 1, "f32"),
    (2, 2, 3, 3, 5, 2, "f32"),
    (2, 3, 2, 4096, 5, 1, "f16"),
    (1, 2, 4096, 2, 3, 1, "f32"),
    (8, 2048, 8, 8, 5, 3, "f16"),
]


@pytest.mark.parametrize("case", DEGENERATE, ids=lambda c: "x".join(map(str, c)))
def test_degenerate_shapes(orc, case):
    test_maximum_side_and_levels(orc, case)


def _random_shapes(count, seed=2024):
    """Seeded random layers: 1-3 images, 1-4 channels, sides 1-300 (mostly
    ragged against 2^L), every k and L = 0..6, fp32 and fp16."""
    import random

    rng = random.Random(seed)
    out = []
    for _ in range(count):
        n, c = rng.randint(1, 3), rng.randint(1, 4)
        h, w = rng.randint(1, 300), rng.randint(1, 300)
        k, L = rng.choice([1, 3, 5, 7]), rng.randint(0, 6)
        out.append((n, c, h, w, k, L, rng.choice(["f32", "f16"])))
    return out


@pytest.mark.parametrize("case", _random_shapes(40), ids=lambda c: "x".join(map(str, c)))
def test_random_shapes(orc, case):
    test_maximum_side_and_levels(orc, case)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c)))
def test_small_shapes(orc, case):
    n, c, h, w, k, L, dt = case
    _log("case %s" % (case,))
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=n * 1000 + h + w + k + L)
    d = DevInputs(inp, dt)
    y = forward(d)
    dx = backward_data(d)
    torch.cuda.synchronize()
    ref_y = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    ref_dx = orc.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    assert_close(y, ref_y, dt, "y")
    assert_close(dx, ref_dx, dt, "dx")


WIDE = [
    # n, c, h, w, k, L, dtype, threads, planes
    (3, 4, 16, 16, 5, 2, "f32", 512, 2),
    (5, 2, 56, 56, 5, 3, "f32", 512, 3),
    (2, 3, 24, 40, 3, 3, "f16", 512, 1),
    (5, 2, 56, 56, 5, 3, "f32", 256, 2),
    # pieces past the last full round run as one-row pieces: 144 on 64
    # threads (16 of them), 265 on 256 threads (9)
    (3, 2, 32, 32, 5, 2, "f32", 64, 2),
    (2, 3, 44, 44, 5, 1, "f16", 256, 1),
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: "x".join(map(str, c)))
def test_whole_plane_thread_counts_and_image_groups(orc, case, monkeypatch):
    """The whole-plane kernel at 64, 256 and 512 threads, with image groups
    that leave a ragged last group, and with plans whose last pieces run as
    one-row pieces."""
    n, c, h, w, k, L, dt, th, planes = case
    _log("case %s" % (case,))
    monkeypatch.setenv("WTCONV_WHOLE_THREADS", str(th))
    monkeypatch.setenv("WTCONV_PLANES", str(planes))
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h + w + th + planes)
    d = DevInputs(inp, dt)
    y = forward(d)
    dx = backward_data(d)
    torch.cuda.synchronize()
    ref_y = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    ref_dx = orc.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    assert_close(y, ref_y, dt, "y")
    assert_close(dx, ref_dx, dt, "dx")


@pytest.mark.parametrize("case", [(1, 2, 272, 272, 5, 2, "f32"), (1, 2, 272, 272, 3, 3, "f16")],
                         ids=lambda c: "x".join(map(str, c)))
def test_nested_call_on_the_strip_fallback(orc, case):
    """272 x 272 planes tile only at 16 x 16, and their 136 x 136 level-1
    low-pass map fits neither one workgroup nor any tile shape: the nested
    call for the deeper levels then takes the strip kernel, which runs the
    base path with a zero scale written to the workspace (the whole-plane and
    tiled kernels skip it).  The weight backward's nested call takes the
    level-by-level fallback the same way."""
    n, c, h, w, k, L, dt = case
    _log("case %s" % (case,))
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=272 + L)
    d = DevInputs(inp, dt)
    y, dx = forward(d), backward_data(d)
    g = backward_weight(d)
    torch.cuda.synchronize()
    assert_close(y, orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L), dt, "y")
    assert_close(dx, orc.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L), dt, "dx")
    ref = orc.backward_weight(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    for gg, rr, name in zip(g, ref, ("dw_base", "dbias", "ds_base", "dw_lvl", "ds_lvl")):
        assert_grad_close(gg, rr, dt, name)


STACKED = [
    # n, c, h, w, k, L, dtype, images per workgroup: odd batches and odd image
    # groups leave half-empty stacks
    (5, 6, 28, 28, 5, 2, "f16", 0),
    (3, 4, 16, 24, 3, 3, "f32", 0),
    (7, 3, 28, 28, 5, 2, "f32", 3),
    (4, 2, 12, 20, 7, 1, "f32", 1),
]


@pytest.mark.parametrize("case", STACKED, ids=lambda c: "x".join(map(str, c)))
def test_stacked_small_planes_equal_one_image_per_pass(orc, case, monkeypatch):
    """Small planes run two images per pass, stacked with zero rows between
    them.  Every output is the same sum in the same order either way, so the
    stacked result must equal the one-image-per-pass result bit for bit, and
    the oracle's within the tolerance."""
    n, c, h, w, k, L, dt, planes = case
    _log("case %s" % (case,))
    if planes:
        monkeypatch.setenv("WTCONV_PLANES", str(planes))
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=17 * h + w + L)
    d = DevInputs(inp, dt)
    y, dx = forward(d), backward_data(d)
    monkeypatch.setenv("WTCONV_STACK", "1")
    y1, dx1 = forward(d), backward_data(d)
    torch.cuda.synchronize()
    assert torch.equal(y, y1), "stacked forward differs from one image per pass"
    assert torch.equal(dx, dx1), "stacked data backward differs from one image per pass"
    assert_close(y, orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L), dt, "y")
    assert_close(dx, orc.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L), dt, "dx")


TILED = [(2, 3, 64, 64, 5, 3, "f32"), (1, 4, 64, 96, 5, 2, "f16"), (2, 2, 48, 64, 3, 1, "f32"),
         (1, 2, 64, 64, 7, 4, "f32"), (2, 2, 128, 64, 5, 5, "f32"), (3, 2, 128, 128, 1, 3, "f16"),
         (2, 3, 64, 64, 7, 0, "f32"), (1, 4, 32, 64, 5, 0, "f16"),  # L = 0: a depthwise conv on tiles
         # level-1 maps too large for the fused kernel: tiles plus a nested
         # call, which itself runs fused without its base path
         (1, 2, 256, 256, 5, 3, "f32"), (2, 1, 256, 128, 3, 4, "f16")]


@pytest.mark.parametrize("case", TILED, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("nested", [False, True], ids=["fused", "nested"])
def test_tiled_planes(orc, case, nested, monkeypatch):
    """The paths for planes too large for one workgroup, forced on small
    planes: base and level-1 convolutions on tiles with halos, and the deeper
    levels either in the same kernel, staged from x and kept on chip (fused),
    or from a stored level-1 low-pass map through a nested call (nested, the
    path of planes whose level-1 map is itself too large)."""
    n, c, h, w, k, L, dt = case
    _log("case %s %s" % (case, "nested" if nested else "fused"))
    monkeypatch.setenv("WTCONV_NO_WHOLE", "1")
    if nested:
        monkeypatch.setenv("WTCONV_NO_LARGE", "1")
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h * w + L)
    d = DevInputs(inp, dt)
    y = forward(d)
    dx = backward_data(d)
    torch.cuda.synchronize()
    ref_y = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    ref_dx = orc.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    assert_close(y, ref_y, dt, "y")
    assert_close(dx, ref_dx, dt, "dx")


def test_no_bias_and_forced_tiling(orc, monkeypatch):
    """The strip kernel (used where no tile shape divides the plane), small LDS
    budget: several tiles per plane, strips, XCD remap of tiles."""
    monkeypatch.setenv("WTCONV_LDS_KB", "16")
    monkeypatch.setenv("WTCONV_NO_TILES", "1")  # the strip kernel (planes no tile shape divides)
    n, c, h, w, k, L = 1, 8, 128, 96, 5, 3
    inp = make_inputs(n, c, h, w, k, L, seed=77)
    inp.bias = None
    d = DevInputs(inp, "f32")
    y = forward(d)
    torch.cuda.synchronize()
    ref = orc.forward(inp.x, inp.w_base, None, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    assert_close(y, ref, "f32", "y tiled")


def test_deterministic_and_guarded(orc):
    """Two runs are bitwise equal and nothing is written outside the output."""
    n, c, h, w, k, L = 2, 4, 56, 56, 5, 3
    inp = make_inputs(n, c, h, w, k, L, seed=3)
    d = DevInputs(inp, "f32")
    numel = n * c * h * w
    guard = 4096
    buf = torch.full((numel + 2 * guard,), 12345.0, device="cuda")
    out = buf[guard:guard + numel].view(n, c, h, w)
    forward(d, y=out)
    first = out.clone()
    forward(d, y=out)
    torch.cuda.synchronize()
    assert torch.equal(first, out)
    assert bool((buf[:guard] == 12345.0).all()) and bool((buf[guard + numel:] == 12345.0).all())


def _workload_case(orc, wl, planes=None):
    inp = make_inputs(wl.n, wl.c, wl.h, wl.w, wl.k, wl.levels, dtype=wl.dtype, seed=wl.seed)
    d = DevInputs(inp, wl.dtype)
    y = forward(d)
    dx = backward_data(d)
    torch.cuda.synchronize()
    sel = slice(None) if planes is None else planes
    xs, dys = inp.x[sel], inp.dy[sel]
    ref_y = orc.forward(xs, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, wl.k, wl.levels)
    ref_dx = orc.backward_data(dys, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, wl.k, wl.levels)
    assert_close(y[sel], ref_y, wl.dtype, "%s y" % wl.name)
    assert_close(dx[sel], ref_dx, wl.dtype, "%s dx" % wl.name)


def test_workload_tiny(orc):
    _workload_case(orc, WORKLOADS["tiny"])


def test_workload_stage1_full(orc):
    _log("stage1 64x96x56x56 L=3 fp32, full comparison")
    _workload_case(orc, WORKLOADS["stage1"])


def test_workload_stage2_full(orc):
    _log("stage2 64x192x28x28 L=2 fp16, full comparison")
    _workload_case(orc, WORKLOADS["stage2"])


def _workload_chunked(orc, wl, chunk):
    """Every image of the workload against the oracle, the oracle run on
    `chunk` images at a time (bounded host memory); the library runs the whole
    batch in one launch, as bench.py times it."""
    inp = make_inputs(wl.n, wl.c, wl.h, wl.w, wl.k, wl.levels, dtype=wl.dtype, seed=wl.seed)
    d = DevInputs(inp, wl.dtype)
    y = forward(d)
    dx = backward_data(d)
    torch.cuda.synchronize()
    for n0 in range(0, wl.n, chunk):
        sel = slice(n0, n0 + chunk)
        _log("  images %d..%d" % (n0, min(n0 + chunk, wl.n) - 1))
        ref = orc.forward(inp.x[sel], inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, wl.k, wl.levels)
        assert_close(y[sel], ref, wl.dtype, "%s L=%d y images %d+" % (wl.name, wl.levels, n0))
        ref = orc.backward_data(inp.dy[sel], inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, wl.k, wl.levels)
        assert_close(dx[sel], ref, wl.dtype, "%s L=%d dx images %d+" % (wl.name, wl.levels, n0))
        del ref


@pytest.mark.parametrize("wl", sweep_workloads(), ids=lambda w: "L%d_%s" % (w.levels, w.dtype))
def test_workload_sweep_full(orc, wl):
    _log("sweep 32x128x128x128 L=%d %s, every image" % (wl.levels, wl.dtype))
    _workload_chunked(orc, wl, chunk=8)


def test_workload_large_full(orc):
    _log("large 16x256x256x256 L=4 fp16, every image")
    _workload_chunked(orc, WORKLOADS["large"], chunk=4)
