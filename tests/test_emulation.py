"""The fused kernels' phase code run on the CPU (bounds-checked emulation)
against the oracle.  Small LDS budgets force tiling and short strips so that
the halo, clipping and strip logic is exercised on shapes the oracle finishes
instantly."""
import numpy as np
import pytest

from level_haar_wavelet_amd.synthetic import make_inputs
from tests import emulation as emu

pytestmark = pytest.mark.skipif(not emu.available(), reason="no clang++ for the emulation")


def _check(y, ref, tol=1e-4):
    assert not np.isnan(y).any()
    err = np.abs(y - ref) / (1.0 + np.abs(ref))
    assert err.max() <= tol, err.max()


CASES = [
    # n, c, h, w, k, L, budget floats (None: whole plane)
    (2, 3, 16, 16, 5, 2, None),
    (1, 2, 16, 24, 3, 3, None),
    (1, 2, 8, 8, 7, 1, None),
    (1, 2, 12, 20, 1, 2, None),
    (1, 1, 56, 56, 5, 3, None),
    (1, 2, 28, 28, 5, 2, None),
    (1, 1, 32, 32, 5, 5, None),
    (1, 1, 64, 64, 5, 4, 9000),    # strips
    (1, 1, 64, 96, 3, 3, 4000),    # tiles and strips
    (1, 1, 64, 64, 5, 2, 3500),    # small tiles, short strips
    (1, 2, 48, 80, 5, 4, 5000),
    (1, 2, 10, 14, 5, 1, None),    # 2-row staging groups (4 does not divide the height)
    (2, 1, 6, 20, 3, 1, None),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("rotate", [0, 1])
def test_emulated_fused_matches_oracle(orc, case, rotate):
    n, c, h, w, k, L, budget = case
    inp = make_inputs(n, c, h, w, k, L, seed=h + w + k + L)
    budget = budget or 1 << 22
    y = emu.fused(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L, rotate=rotate,
                  budget_floats=budget)
    if rotate == 0:
        ref = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    else:
        ref = orc.backward_data(inp.x, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    _check(y, ref)


def test_emulated_fp16(orc):
    n, c, h, w, k, L = 1, 2, 32, 32, 5, 3
    inp = make_inputs(n, c, h, w, k, L, dtype="f16", seed=9)
    y = emu.fused(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L, dtype="f16")
    ref = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel <= 5e-3, rel
    # one rounding to fp16 of an fp32 result: within half an fp16 ulp plus fp32 noise
    assert np.abs(y - ref).max() <= np.abs(ref).max() * 2.0 ** -10


def test_plans_fit_and_tile():
    p = emu.fused_plan(64, 96, 56, 56, 5, 3, budget_floats=1 << 22)
    assert (p["tile_h"], p["tile_w"], p["strip_h"]) == (56, 56, 56)
    p = emu.fused_plan(1, 1, 64, 64, 5, 4, budget_floats=9000)
    assert p["lds_floats"] <= 9000 and p["strip_h"] < p["tile_h"]
    p = emu.fused_plan(1, 1, 64, 96, 3, 3, budget_floats=4000)
    assert p["lds_floats"] <= 4000 and p["tiles_y"] * p["tiles_x"] > 1


WGRAD_CASES = [
    # n, c, h, w, k, L, dtype, planes or groups
    (2, 3, 16, 16, 5, 2, "f32", 2),
    (3, 2, 16, 24, 3, 3, "f32", 3),
    (2, 3, 9, 13, 5, 0, "f32", 2),
    (3, 2, 28, 28, 5, 2, "f16", 2),
    (2, 2, 56, 56, 5, 3, "f32", 2),
    (1, 2, 64, 96, 5, 4, "f16", 3),
    (2, 2, 14, 10, 7, 1, "f32", 2),   # staging groups of 2 rows, 2 columns
    (3, 2, 12, 12, 1, 2, "f16", 1),
    (2, 1, 24, 40, 3, 2, "f32", 2),   # odd border width
    (2, 2, 32, 48, 7, 3, "f32", 2),
    (2, 1, 32, 32, 1, 5, "f32", 2),
]


@pytest.mark.parametrize("case", WGRAD_CASES)
@pytest.mark.parametrize("tiled", [False, True])
def test_emulated_weight_gradients_match_oracle(orc, case, tiled):
    n, c, h, w, k, L, dt, g = case
    if not tiled and not emu.wgrad_plan(n, c, h, w, k, L, planes=g, dtype=dt)["ok"]:
        pytest.skip("plane too large for the whole-plane weight-gradient kernel")
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h + w + L)
    got = emu.wgrad(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L, dtype=dt,
                    planes=g, tiled=tiled)
    ref = orc.backward_weight(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    for gg, rr in zip(got, ref):
        if rr.size == 0:
            continue
        assert not np.isnan(gg).any()
        assert np.linalg.norm(gg - rr) / np.linalg.norm(rr) <= 2e-6


def test_weight_gradient_plans_refuse_pitches_past_the_descriptor_fields(orc):
    """Piece descriptors hold map pitches in 8 bits.  Without the base path
    the widest maps a piece reads are level 1's, so a plane whose level-1
    maps need a pitch above 255 (8 x 512, the nested call of a 64 x 4096
    layer three levels down) is refused, and the one just below the limit
    (8 x 480) computes the oracle's gradients."""
    inp = make_inputs(1, 1, 8, 512, 3, 3, seed=5)
    with pytest.raises(ValueError):
        emu.wgrad(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, 3, 3, nthreads=256,
                  budget_floats=40960, nobase=True)
    inp = make_inputs(1, 1, 8, 480, 3, 3, seed=6)
    got = emu.wgrad(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, 3, 3, nthreads=256,
                    budget_floats=40960, nobase=True)
    zero = np.zeros_like(inp.s_base)
    ref = orc.backward_weight(inp.x, inp.dy, inp.w_base, inp.bias, zero, inp.w_lvl, inp.s_lvl, 3, 3)
    for gg, rr in zip(got[3:], ref[3:]):
        assert np.linalg.norm(gg - rr) / np.linalg.norm(rr) <= 2e-6


def test_weight_gradient_piece_tails():
    """A one-set weight-gradient plan whose last wave would hold a few pieces
    runs those as four one-row pieces each on the lanes after the full waves,
    when they take at most two waves: 129 pieces at 28 x 28, L = 2 (one tail
    piece), 144 at 24 x 40, L = 2 (16).  None where the rest would take more
    (28 x 28, L = 1: 113 pieces, 49 past the first wave), where no wave is
    full (16 x 16, L = 2: 36 pieces), or where the plan has two sets (56 x 56,
    L = 3: 472 pieces on 256 threads)."""
    for shape, L, np_, tail in (((28, 28), 2, 129, 1), ((24, 40), 2, 144, 16), ((28, 28), 1, 113, 0),
                                ((16, 16), 2, 36, 0), ((56, 56), 3, 472, 0)):
        p = emu.wgrad_plan(2, 2, *shape, 5, L, nthreads=256, dtype="f16", budget_floats=1 << 16)
        assert p["ok"] and (p["npieces"], p["tail"]) == (np_, tail), (shape, L, p)


def _rounds_cost(n, c, slots, fixed, p):
    groups = -(-n // p)
    return -(-c * groups // slots) * (p + fixed)


@pytest.mark.parametrize("n,c,slots", [(64, 96, 512), (64, 192, 512), (64, 192, 1024), (16, 256, 512),
                                       (1, 7, 512), (5, 3, 512), (300, 2, 4)])
def test_choose_planes_minimises_rounds_cost(n, c, slots):
    """The planes chooser against brute force over every planes value."""
    for fixed in (0.0, 1.0, 3.0):
        got = emu.choose_planes(n, c, slots, fixed)
        assert 1 <= got <= n
        best = min(_rounds_cost(n, c, slots, fixed, p) for p in range(1, n + 1))
        assert _rounds_cost(n, c, slots, fixed, got) == best


def test_choose_planes_fills_one_round():
    # 96 channels x 64 images on 512 resident workgroups: 5 groups of 13 images run in one round
    assert emu.choose_planes(64, 96, 512, 1.0) == 13


@pytest.mark.parametrize("nthreads,planes,L", [(512, 2, 3), (128, 3, 3), (64, 2, 2)])
def test_emulated_whole_plane_thread_counts(orc, nthreads, planes, L):
    # 64 threads at L = 2: 144 pieces, the last 16 as one-row pieces
    n, c, h, w, k = 5, 2, 32, 32, 5
    inp = make_inputs(n, c, h, w, k, L, seed=nthreads + planes)
    y = emu.whole(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L, nthreads=nthreads,
                  planes=planes, budget_floats=1 << 16)
    ref = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    _check(y, ref)


@pytest.mark.parametrize("shape", [(1, 2, 56, 56, 5, 3, "f32", 512), (2, 2, 48, 16, 3, 4, "f32", 256),
                                   (1, 2, 16, 40, 7, 3, "f16", 256), (3, 1, 32, 32, 1, 5, "f32", 128)])
@pytest.mark.parametrize("rotate", [0, 1])
def test_emulated_whole_plane_level3_from_lane_quads(orc, shape, rotate):
    """L >= 3 with 4 x 4 staging groups: the four lanes of a quad stage a 2 x 2
    block of groups and build Haar level 3 from their level-2 sums (DPP in
    the kernel; here after every thread has staged)."""
    n, c, h, w, k, L, dt, nth = shape
    assert emu.whole_plan(n, c, h, w, k, L, nthreads=nth, dtype=dt, budget_floats=1 << 16)["stage_l3"] == 1
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h + 3 * w + rotate)
    y = emu.whole(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L, rotate=rotate, dtype=dt,
                  nthreads=nth, planes=2, budget_floats=1 << 16)
    if rotate == 0:
        ref = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    else:
        ref = orc.backward_data(inp.x, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    if dt == "f32":
        _check(y, ref)
    else:
        assert np.linalg.norm(y - ref) / np.linalg.norm(ref) <= 5e-3


@pytest.mark.parametrize("shape", [(2, 3, 16, 16, 5, 2), (1, 2, 28, 28, 5, 2), (1, 2, 24, 40, 3, 3), (1, 1, 32, 64, 7, 4)])
@pytest.mark.parametrize("rotate", [0, 1])
def test_emulated_whole_plane_fp16(orc, shape, rotate):
    """The whole-plane kernel with fp16 activations: staging segment width and
    output block width follow the dtype."""
    n, c, h, w, k, L = shape
    inp = make_inputs(n, c, h, w, k, L, dtype="f16", seed=h + w + rotate)
    y = emu.whole(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L, rotate=rotate, dtype="f16",
                  budget_floats=1 << 16)
    if rotate == 0:
        ref = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    else:
        ref = orc.backward_data(inp.x, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel <= 5e-3, rel


@pytest.mark.parametrize("shape", [(2, 3, 16, 16, 7, 0, "f32"), (1, 2, 14, 10, 3, 0, "f32"), (2, 2, 12, 20, 5, 0, "f16"),
                                   (1, 2, 28, 28, 5, 1, "f32"), (1, 2, 20, 12, 3, 1, "f16")])
@pytest.mark.parametrize("rotate", [0, 1])
def test_emulated_whole_plane_levels_0_and_1(orc, shape, rotate):
    """L = 0 (the plain depthwise convolution) and L = 1 through the whole-plane
    kernel, with 2- and 4-row staging groups."""
    n, c, h, w, k, L, dt = shape
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h * w + rotate)
    y = emu.whole(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L, rotate=rotate, dtype=dt,
                  budget_floats=1 << 16)
    if rotate == 0:
        ref = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    else:
        ref = orc.backward_data(inp.x, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    if dt == "f32":
        _check(y, ref)
    else:
        assert np.linalg.norm(y - ref) / np.linalg.norm(ref) <= 5e-3


def _lowpass(a):
    """Level-1 orthonormal low-pass band of (N, C, H, W): half the 2x2 block sums."""
    return 0.5 * (a[:, :, 0::2, 0::2] + a[:, :, 0::2, 1::2] + a[:, :, 1::2, 0::2] + a[:, :, 1::2, 1::2])


TILED = [
    # n, c, h, w, k, L, th, tw, dtype
    (2, 2, 64, 64, 7, 0, 32, 32, "f32"),
    (1, 3, 32, 64, 5, 0, 16, 32, "f16"),
    (2, 2, 64, 64, 5, 1, 32, 16, "f32"),
    (1, 2, 64, 96, 5, 3, 32, 32, "f32"),
    (2, 1, 48, 64, 3, 2, 16, 32, "f32"),
    (1, 2, 64, 64, 7, 4, 32, 32, "f32"),
    (1, 2, 64, 128, 5, 2, 32, 64, "f16"),
]


@pytest.mark.parametrize("case", TILED, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("rotate", [0, 1])
def test_emulated_tiled_pass_with_deeper_levels(orc, case, rotate):
    """Planes too large for one workgroup: the base and level-1 convolutions on
    tiles with halos, plus the deeper levels' contribution, which is the layer
    with L - 1 levels (weights and scales from level 2 on, base scale 0) on
    the level-1 low-pass map.  The deeper term is taken from the oracle here;
    the result must equal the oracle's full layer."""
    n, c, h, w, k, L, th, tw, dt = case
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h + w + L + rotate)
    src = inp.x
    low = None
    if L >= 2:
        zero = np.zeros_like(inp.s_base)
        ll = _lowpass(src)
        if rotate == 0:
            low = orc.forward(ll, inp.w_base, None, zero, inp.w_lvl[1:], inp.s_lvl[1:], k, L - 1)
        else:
            low = orc.backward_data(ll, inp.w_base, zero, inp.w_lvl[1:], inp.s_lvl[1:], k, L - 1)
    wl1, sl1 = (inp.w_lvl[:1], inp.s_lvl[:1]) if L else (None, None)
    y = emu.whole_tiled(src, low, inp.w_base, inp.bias, inp.s_base, wl1, sl1, k, th, tw,
                        rotate=rotate, dtype=dt, planes=3, budget_floats=1 << 16)
    if rotate == 0:
        ref = orc.forward(src, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    else:
        ref = orc.backward_data(src, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    if dt == "f32":
        _check(y, ref)
    else:
        assert np.linalg.norm(y - ref) / np.linalg.norm(ref) <= 5e-3


STACKED = [
    # n, c, h, w, k, L, nthreads, planes, dtype: odd batches leave the last
    # stack half empty
    (4, 3, 28, 28, 5, 2, 256, 2, "f16"),
    (3, 2, 28, 28, 5, 2, 256, 1, "f32"),
    (5, 2, 16, 16, 5, 2, 256, 2, "f32"),
    (2, 2, 16, 24, 3, 3, 512, 1, "f32"),
    (3, 2, 12, 20, 7, 1, 256, 3, "f32"),
    (2, 1, 8, 8, 1, 2, 256, 1, "f32"),
]


@pytest.mark.parametrize("k, L, gap", [(5, 2, 8), (5, 3, 16), (3, 1, 4), (7, 1, 8), (1, 2, 0), (3, 4, 16),
                                        (7, 2, 12)])
def test_stacked_plan_gap_and_units(k, L, gap):
    """The rows between stacked images: r rows at every level's resolution
    (r 2^L at full resolution), rounded up to whole 4-row staging groups and
    level-L cells; two images per unit, the last one half empty for odd
    batches."""
    r = k // 2
    assert gap == -(-(r << L) // max(4, 1 << L)) * max(4, 1 << L)
    p = emu.whole_plan(5, 2, 16, 16, k, L, nthreads=256, planes=1, stack=2, budget_floats=1 << 15)
    assert p["ok"] and p["gap"] == gap and p["rows"] == 2 * 16 + gap and p["units"] == 3


def test_stacked_plan_refused_where_it_would_not_be_exact():
    """No stacking for L = 0 (the caller's depthwise path) or when an image's
    rows are not whole staging groups and level-L cells."""
    assert not emu.whole_plan(2, 1, 16, 16, 5, 0, stack=2)["ok"]
    assert not emu.whole_plan(2, 1, 12, 16, 5, 3, stack=2)["ok"]  # 12 rows, 8-row level-3 cells
    assert not emu.whole_plan(2, 1, 18, 16, 3, 1, stack=2)["ok"]  # 18 rows, 4-row groups
    assert emu.whole_plan(2, 1, 16, 16, 5, 3, stack=2)["ok"]


@pytest.mark.parametrize("case", STACKED, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("rotate", [0, 1])
def test_emulated_stacked_small_planes(orc, case, rotate):
    """Small planes run two images per workgroup pass, stacked down one plane
    with zero rows between them (r rows at every level's resolution): the
    result must be each image's own layer, and the rows between images never
    stored (the output starts as NaN)."""
    n, c, h, w, k, L, nth, planes, dt = case
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=3 * h + w + L + rotate)
    src = inp.x if rotate == 0 else inp.dy
    y = emu.whole(src, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L, rotate=rotate, dtype=dt,
                  nthreads=nth, planes=planes, budget_floats=1 << 15, stack=2)
    if rotate == 0:
        ref = orc.forward(src, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    else:
        ref = orc.backward_data(src, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    assert not np.isnan(y).any()
    if dt == "f32":
        _check(y, ref)
    else:
        assert np.linalg.norm(y - ref) / np.linalg.norm(ref) <= 5e-3


NOBASE = [
    # n, c, h, w, k, L, nthreads, dtype
    (2, 3, 32, 32, 5, 1, 256, "f32"),
    (1, 2, 64, 64, 5, 1, 512, "f32"),
    (2, 2, 28, 28, 3, 2, 256, "f16"),
    (1, 2, 32, 48, 7, 3, 256, "f32"),
]


@pytest.mark.parametrize("case", NOBASE, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("rotate", [0, 1])
def test_emulated_whole_plane_without_the_base_path(orc, case, rotate):
    """The nested call for the deeper levels of a larger layer runs without
    the base path (its base scale is zero): no base pieces, no base output,
    base weights, bias and scale never read (NaN here).  It must equal the
    oracle's layer with a zero base scale and no bias."""
    n, c, h, w, k, L, nth, dt = case
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=7 * h + L + rotate)
    nan_w, nan_c = np.full_like(inp.w_base, np.nan), np.full_like(inp.s_base, np.nan)
    y = emu.whole(inp.x, nan_w, nan_c, nan_c, inp.w_lvl, inp.s_lvl, k, L, rotate=rotate, dtype=dt, nthreads=nth,
                  planes=2, budget_floats=1 << 15, nobase=True)
    zero = np.zeros_like(inp.s_base)
    if rotate == 0:
        ref = orc.forward(inp.x, inp.w_base, None, zero, inp.w_lvl, inp.s_lvl, k, L)
    else:
        ref = orc.backward_data(inp.x, inp.w_base, zero, inp.w_lvl, inp.s_lvl, k, L)
    if dt == "f32":
        _check(y, ref)
    else:
        assert np.linalg.norm(y - ref) / np.linalg.norm(ref) <= 5e-3


@pytest.mark.parametrize("rotate", [0, 1])
def test_emulated_tiled_pass_without_the_base_path(orc, rotate):
    """The same for the tiled pass of a nested call (levels 1..L of a layer
    whose base path is zero), with the deeper levels' low-pass term added."""
    n, c, h, w, k, L, th, tw = 2, 2, 64, 64, 5, 3, 32, 32
    inp = make_inputs(n, c, h, w, k, L, seed=99 + rotate)
    zero = np.zeros_like(inp.s_base)
    ll = _lowpass(inp.x)
    if rotate == 0:
        low = orc.forward(ll, inp.w_base, None, zero, inp.w_lvl[1:], inp.s_lvl[1:], k, L - 1)
        ref = orc.forward(inp.x, inp.w_base, None, zero, inp.w_lvl, inp.s_lvl, k, L)
    else:
        low = orc.backward_data(ll, inp.w_base, zero, inp.w_lvl[1:], inp.s_lvl[1:], k, L - 1)
        ref = orc.backward_data(inp.x, inp.w_base, zero, inp.w_lvl, inp.s_lvl, k, L)
    nan_w, nan_c = np.full_like(inp.w_base, np.nan), np.full_like(inp.s_base, np.nan)
    y = emu.whole_tiled(inp.x, low, nan_w, nan_c, nan_c, inp.w_lvl[:1], inp.s_lvl[:1], k, th, tw, rotate=rotate,
                        planes=3, budget_floats=1 << 16, nobase=True)
    _check(y, ref)


def test_emulated_tiled_pass_with_two_output_blocks_per_thread(orc):
    """Tiles with more output blocks than threads (64 x 64 tiles, 384 threads):
    a thread's second output block, with its own deeper-levels term."""
    n, c, h, w, k, L, th, tw = 1, 2, 128, 128, 5, 3, 64, 64
    inp = make_inputs(n, c, h, w, k, L, seed=321)
    zero = np.zeros_like(inp.s_base)
    low = orc.forward(_lowpass(inp.x), inp.w_base, None, zero, inp.w_lvl[1:], inp.s_lvl[1:], k, L - 1)
    y = emu.whole_tiled(inp.x, low, inp.w_base, inp.bias, inp.s_base, inp.w_lvl[:1], inp.s_lvl[:1], k, th, tw,
                        nthreads=384, planes=2, budget_floats=1 << 16)
    _check(y, orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L))


WGRAD_TILED = [
    # n, c, h, w, k, L (0 or 1), th, tw, dtype
    (2, 2, 64, 64, 5, 1, 32, 16, "f32"),
    (3, 1, 48, 64, 3, 1, 16, 32, "f32"),
    (1, 2, 64, 64, 7, 1, 32, 32, "f32"),
    (2, 2, 64, 128, 5, 1, 32, 64, "f16"),
    (2, 2, 64, 64, 7, 0, 32, 32, "f32"),
    (1, 3, 32, 64, 5, 0, 16, 32, "f16"),
]


@pytest.mark.parametrize("case", WGRAD_TILED, ids=lambda c: "x".join(map(str, c)))
def test_emulated_tiled_weight_gradients_levels_0_and_1(orc, case):
    """Planes too large for one workgroup: base and level-1 parameter gradients
    from correlations on tiles (x with halos, dy inside the tile); L = 0 is a
    plain depthwise convolution's gradients."""
    n, c, h, w, k, L, th, tw, dt = case
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h + w + k)
    wl, sl = (inp.w_lvl, inp.s_lvl) if L else (None, None)
    got = emu.wgrad_tiles(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, wl, sl, k, th, tw,
                          dtype=dt, planes=3, budget_floats=1 << 16)
    ref = orc.backward_weight(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, wl, sl, k, L)
    for gg, rr in zip(got, ref):
        assert not np.isnan(gg).any()
        assert np.linalg.norm(gg - rr) / np.linalg.norm(rr) <= 2e-6


@pytest.mark.parametrize("dt", ["f32", "f16"])
def test_emulated_tiled_weight_gradients_on_64x64_tiles_of_512_threads(orc, dt):
    """The tile shape the library tries first for the weight backward: 64 x 64
    tiles on 512 threads (one correlation piece per thread), on a plane of
    2 x 2 tiles, base and level 1, with the low-pass maps written too."""
    n, c, h, w, k, L = 2, 2, 128, 128, 5, 1
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=11)
    got, (llx, lld) = emu.wgrad_tiles(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k,
                                      64, 64, dtype=dt, nthreads=512, planes=3, budget_floats=40960, lowpass=True)
    ref = orc.backward_weight(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    for gg, rr in zip(got, ref):
        assert not np.isnan(gg).any()
        assert np.linalg.norm(gg - rr) / np.linalg.norm(rr) <= 2e-6
    assert np.abs(llx - _lowpass(inp.x)).max() <= 1e-6 and np.abs(lld - _lowpass(inp.dy)).max() <= 1e-6


@pytest.mark.parametrize("case", [c for c in WGRAD_TILED if c[5] == 1], ids=lambda c: "x".join(map(str, c)))
def test_emulated_tiled_weight_gradients_write_the_low_pass_maps(orc, case):
    """With L >= 2 the tiled weight-gradient pass also writes the level-1
    low-pass maps of x and dy (every tile its interior), which feed the nested
    call for the deeper levels: every element written once, equal to the
    oracle's Haar analysis, and the gradients unchanged."""
    n, c, h, w, k, L, th, tw, dt = case
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h + w + k)
    got, (llx, lld) = emu.wgrad_tiles(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k,
                                      th, tw, dtype=dt, planes=3, budget_floats=1 << 16, lowpass=True)
    plain = emu.wgrad_tiles(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, th, tw,
                            dtype=dt, planes=3, budget_floats=1 << 16)
    for gg, pp in zip(got, plain):
        assert np.array_equal(gg, pp)
    tol = 1e-6 if dt == "f32" else 1e-3
    for src, ll in ((inp.x, llx), (inp.dy, lld)):
        assert not np.isnan(ll).any()
        ref = np.stack([np.stack([orc.haar_analysis(src[i, j].astype(np.float64))[0] for j in range(c)])
                        for i in range(n)])
        assert np.abs(ll - ref).max() <= tol * (1 + np.abs(ref).max())


WGRAD_NOBASE = [
    # n, c, h, w, k, L, nthreads, dtype
    (2, 3, 32, 32, 5, 1, 256, "f32"),
    (3, 2, 28, 28, 3, 2, 256, "f16"),
    (1, 2, 64, 64, 5, 1, 256, "f32"),
    (2, 2, 32, 48, 7, 3, 512, "f32"),
]


@pytest.mark.parametrize("case", WGRAD_NOBASE, ids=lambda c: "x".join(map(str, c)))
def test_emulated_weight_gradients_without_the_base_path(orc, case):
    """The nested call for the deeper levels wants only the level gradients:
    the base map gets no pieces, its gradients come out as 0 (the scale
    gradient of the base is then s0 . 0 = 0), and every level gradient equals
    the oracle's."""
    n, c, h, w, k, L, nth, dt = case
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=11 * h + L)
    got = emu.wgrad(inp.x, inp.dy, inp.w_base, None, inp.s_base, inp.w_lvl, inp.s_lvl, k, L, dtype=dt,
                    nthreads=nth, planes=2, budget_floats=1 << 15, nobase=True)
    ref = orc.backward_weight(inp.x, inp.dy, inp.w_base, None, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    tol = 2e-6 if dt == "f32" else 5e-3
    for gg in got[:3]:
        assert np.array_equal(gg, np.zeros_like(gg))
    for gg, rr in zip(got[3:], ref[3:]):
        assert np.linalg.norm(gg - rr) / np.linalg.norm(rr) <= tol


def test_emulated_tiled_weight_gradients_without_the_base_path(orc):
    """The same for the tiled pass (the nested call on 128 x 128 maps of a
    256 x 256 layer): level-1 gradients equal the oracle's, base ones 0, and
    the low-pass maps still written."""
    n, c, h, w, k, th, tw = 2, 2, 64, 64, 5, 32, 16
    inp = make_inputs(n, c, h, w, k, 1, seed=5)
    got, (llx, lld) = emu.wgrad_tiles(inp.x, inp.dy, inp.w_base, None, inp.s_base, inp.w_lvl, inp.s_lvl, k, th, tw,
                                      planes=3, budget_floats=1 << 16, lowpass=True, nobase=True)
    ref = orc.backward_weight(inp.x, inp.dy, inp.w_base, None, inp.s_base, inp.w_lvl, inp.s_lvl, k, 1)
    for gg in got[:3]:
        assert np.array_equal(gg, np.zeros_like(gg))
    for gg, rr in zip(got[3:], ref[3:]):
        assert np.linalg.norm(gg - rr) / np.linalg.norm(rr) <= 2e-6
    assert np.abs(llx - _lowpass(inp.x.astype(np.float64))).max() <= 1e-6 * (1 + np.abs(llx).max())
    assert np.abs(lld - _lowpass(inp.dy.astype(np.float64))).max() <= 1e-6 * (1 + np.abs(lld).max())


@pytest.mark.parametrize("L", [2, 3, 4])
def test_deeper_level_gradients_are_the_layer_on_the_low_pass_maps(orc, L):
    """The decomposition the large-plane weight gradient relies on, checked on
    the oracle alone: the level-2..L gradients of the layer equal the level
    gradients of the (L-1)-level layer on the level-1 low-pass maps of x and dy
    (weights and scales from level 2 on)."""
    n, c, h, w, k = 2, 3, 32, 32, 5
    inp = make_inputs(n, c, h, w, k, L, seed=40 + L)
    full = orc.backward_weight(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    x64, dy64 = inp.x.astype(np.float64), inp.dy.astype(np.float64)
    sub = orc.backward_weight(_lowpass(x64), _lowpass(dy64), inp.w_base, None, inp.s_base, inp.w_lvl[1:],
                              inp.s_lvl[1:], k, L - 1)
    assert np.abs(full[3][1:] - sub[3]).max() <= 1e-12 * (1 + np.abs(full[3]).max())
    assert np.abs(full[4][1:] - sub[4]).max() <= 1e-12 * (1 + np.abs(full[4]).max())


LARGE = [
    # n, c, h, w, k, L, dtype, tile rows, tile cols, images per workgroup
    (2, 2, 32, 32, 5, 2, "f32", 16, 16, 1),
    (3, 1, 64, 64, 5, 3, "f32", 32, 64, 2),   # odd batch: a last workgroup with one image
    (2, 1, 64, 64, 3, 4, "f16", 32, 32, 2),
    (1, 2, 64, 128, 7, 5, "f32", 32, 64, 1),
    (2, 1, 32, 64, 1, 2, "f16", 16, 32, 2),
    (1, 1, 128, 128, 5, 3, "f32", 32, 64, 1),  # the level sweep's plane
    (1, 1, 128, 128, 7, 5, "f32", 32, 64, 1),  # ... with the other kernel sizes
    (1, 1, 128, 128, 3, 5, "f16", 32, 64, 1),
    (1, 1, 128, 128, 1, 4, "f16", 16, 128, 1),
]


@pytest.mark.parametrize("case", LARGE, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("rotate", [0, 1])
def test_emulated_large_plane_kernel_keeps_every_level_on_chip(orc, case, rotate):
    """The fused large-plane kernel: the deeper levels staged straight from x
    (8 x 8 blocks reduced to the level-1 low-pass map in registers), their
    output kept in an LDS map that the tiles' output pass reads, both plans'
    maps aliasing one LDS region.  The emulation poisons that region with NaN
    after the deeper levels and after every image, so the result also shows
    that the tiles' staging writes every element they read and that the
    deeper levels zero their own maps."""
    n, c, h, w, k, L, dt, th, tw, planes = case
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h + w + k + L)
    src = inp.x if rotate == 0 else inp.dy
    bias = inp.bias if rotate == 0 else None
    y, info = emu.large(src, inp.w_base, bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L, th, tw, rotate=rotate,
                        dtype=dt, planes=planes, budget_floats=160 * 256)
    assert info[0] == planes and info[3] == (h // th) * (w // tw)
    if rotate == 0:
        ref = orc.forward(inp.x, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    else:
        ref = orc.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    _check(y, ref, tol=1e-4 if dt == "f32" else 4 * 2.0 ** -11)


@pytest.mark.parametrize("case", [LARGE[0], LARGE[2], LARGE[5]], ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("rotate", [0, 1])
def test_emulated_large_plane_kernel_without_base_path(orc, case, rotate):
    """The fused large-plane kernel without the base path, as the nested
    deeper-levels call of a larger plane runs it: the base weights, bias and
    scale are NaN (never read), the tiles' output pass reads its base output
    from a zero row outside the aliased map region (which the emulation
    poisons), and the result is the layer with a zero base scale."""
    n, c, h, w, k, L, dt, th, tw, planes = case
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=3 * h + w + k + L)
    src = inp.x if rotate == 0 else inp.dy
    nan_c = np.full(c, np.nan, np.float32)
    nan_w = np.full_like(inp.w_base, np.nan)
    y, _ = emu.large(src, nan_w, nan_c if rotate == 0 else None, nan_c, inp.w_lvl, inp.s_lvl, k, L, th, tw,
                     rotate=rotate, dtype=dt, planes=planes, budget_floats=160 * 256, nobase=True)
    zero_c = np.zeros(c, np.float32)
    if rotate == 0:
        ref = orc.forward(inp.x, inp.w_base, zero_c, zero_c, inp.w_lvl, inp.s_lvl, k, L)
    else:
        ref = orc.backward_data(inp.dy, inp.w_base, zero_c, inp.w_lvl, inp.s_lvl, k, L)
    _check(y, ref, tol=1e-4 if dt == "f32" else 4 * 2.0 ** -11)


def test_large_plane_plan_sizes():
    """At the level sweep's 128 x 128 planes the fused plan (32 x 64 tiles, 256
    threads) fits two workgroups per compute unit for every L = 2..5 (at most
    80 KB of LDS each); it does not apply at L = 1 (no deeper levels) nor to a
    256 x 256 plane (its 128 x 128 level-1 map needs more staging groups than
    threads)."""
    for L in range(2, 6):
        for dt in ("f32", "f16"):
            info = emu.large_plan(32, 128, 128, 128, 32, 64, 5, L, dtype=dt, budget_floats=160 * 256)
            assert info is not None and info[1] * 4 <= 80 * 1024, (L, dt, info)
    assert emu.large_plan(32, 128, 128, 128, 32, 64, 5, 1) is None
    assert emu.large_plan(16, 256, 256, 256, 32, 64, 5, 4, budget_floats=160 * 256) is None
    # the nested deeper-levels call of the 256 x 256 layer: its fp32 level-1
    # map (128 x 128, L = 3) without the base path, 16 x 128 tiles
    info = emu.large_plan(16, 256, 128, 128, 16, 128, 5, 3, dtype="f32", budget_floats=160 * 256, nobase=True)
    assert info is not None and info[1] * 4 <= 80 * 1024, info
    # its tiles have 128 level-1 pieces for 256 threads: they run as 2-row halves
    assert info[6] == 128 and info[8] == 1, info


def test_convolution_piece_tails():
    """Pieces past the last full round of a workgroup's threads run as four
    one-row pieces each when those fit one round: the stacked 28 x 28 L = 2
    plan has 272 pieces on 256 threads, so 16 of them.  No tail where the
    pieces are one round (the 56 x 56 L = 3 plan: 472 pieces on 512 threads),
    where they are fewer than the threads, or where the rest would take more
    than a round (the 40 x 40 L = 1 plan on 128 threads: 200 pieces).  The
    large-plane kernel keeps its deeper-levels pieces whole (64, 80 and 84 past
    the first round at L = 3, 4, 5 of the level sweep's 128 x 128 planes); its
    tiles have one piece per thread."""
    for L, extra in ((2, 0), (3, 64), (4, 80), (5, 84)):
        info = emu.large_plan(32, 128, 128, 128, 32, 64, 5, L, dtype="f32", budget_floats=160 * 256)
        assert info[4:] == [256 + extra, 0, 256, 0, 0], (L, info)
    p = emu.whole_plan(64, 192, 28, 28, 5, 2, nthreads=256, dtype="f16", budget_floats=40960, stack=2)
    assert p["ok"] and (p["items"], p["tail"]) == (272, 16)
    p = emu.whole_plan(64, 96, 56, 56, 5, 3, nthreads=512, budget_floats=40960)
    assert p["ok"] and (p["items"], p["tail"]) == (472, 0)
    p = emu.whole_plan(4, 2, 16, 16, 5, 2, nthreads=256, budget_floats=40960)
    assert p["ok"] and (p["items"], p["tail"]) == (36, 0)
    p = emu.whole_plan(4, 2, 32, 32, 5, 2, nthreads=64, budget_floats=40960)
    assert p["ok"] and (p["items"], p["tail"]) == (64 + 64 + 16, 16)
    p = emu.whole_plan(4, 2, 40, 40, 5, 1, nthreads=128, budget_floats=40960)
    assert p["ok"] and (p["items"], p["tail"]) == (100 + 100, 0)


BWD = [
    # n, c, h, w, k, L, dtype, threads, images per workgroup
    (2, 2, 16, 16, 5, 2, "f32", 256, 2),
    (3, 2, 56, 56, 5, 3, "f32", 512, 2),   # odd batch: a last workgroup with one image
    (3, 2, 28, 28, 5, 2, "f16", 512, 2),
    (2, 1, 32, 32, 3, 5, "f32", 256, 1),
    (2, 2, 24, 40, 7, 1, "f32", 512, 2),
    (2, 2, 12, 20, 1, 2, "f16", 256, 2),
    (2, 2, 44, 44, 5, 1, "f32", 256, 1),   # 265 pieces on 256 threads: 9 run as one-row pieces
]


@pytest.mark.parametrize("case", BWD, ids=lambda c: "x".join(map(str, c)))
def test_emulated_fused_backward(orc, case):
    """The fused single-pass backward: one staging of x and dy serving the
    data backward's convolution and the weight backward's correlation; dx and
    every gradient against the oracle."""
    n, c, h, w, k, L, dt, nth, planes = case
    inp = make_inputs(n, c, h, w, k, L, dtype=dt, seed=h + w + L)
    dx, g = emu.bwd(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, dtype=dt,
                    nthreads=nth, planes=planes, budget_floats=160 * 256)
    ref = orc.backward_data(inp.dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    _check(dx, ref, tol=1e-4 if dt == "f32" else 4 * 2.0 ** -11)
    rg = orc.backward_weight(inp.x, inp.dy, inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    for a, b in zip(g, rg):
        assert np.linalg.norm(a - b) <= 1e-5 * np.linalg.norm(b)
