"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test checks the oracle against a worked example, a closed form, an
invariant, a library routine or brute force, chosen so that a plausible slip in
the oracle (a dropped term, a wrong sign or index, a transposed operand) fails at
least one of them.  Non-square maps are used wherever a height/width mix-up could
hide.
"""
import os

import numpy as np
import pytest
import torch

from level_haar_wavelet_amd.synthetic import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_params(rng, c, k, levels):
    w0 = rng.standard_normal((c, k, k))
    b0 = rng.standard_normal(c)
    s0 = rng.standard_normal(c)
    wl = rng.standard_normal((levels, 4 * c, k, k))
    sl = rng.standard_normal((levels, 4 * c))
    return w0, b0, s0, wl, sl


def _blockmean(x, f):
    """Mean over f x f blocks of the last two axes -> coarse map."""
    *lead, h, w = x.shape
    return x.reshape(*lead, h // f, f, w // f, f).mean(axis=(-3, -1))


def _up(x, f):
    return np.repeat(np.repeat(x, f, axis=-2), f, axis=-1)


# ---------------------------------------------------------------------------
# Haar steps
# ---------------------------------------------------------------------------

def test_haar_worked_blocks(orc):
    """Hand-worked 2x2 blocks (tests/golden/haar_blocks.txt)."""
    rows = []
    with open(os.path.join(GOLDEN, "haar_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("->")
            rows.append(([float(t) for t in lhs.split()], [float(t) for t in rhs.split()]))
    assert len(rows) >= 5
    for (a, b, c, d), expect in rows:
        bands = orc.haar_analysis(np.array([[a, b], [c, d]]))
        assert bands.shape == (4, 1, 1)
        np.testing.assert_array_equal(bands[:, 0, 0], expect)
        back = orc.haar_synthesis(bands)
        np.testing.assert_array_equal(back, [[a, b], [c, d]])


def test_haar_perfect_reconstruction_and_energy(orc):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((12, 20))
    bands = orc.haar_analysis(x)
    assert bands.shape == (4, 6, 10)
    np.testing.assert_allclose(orc.haar_synthesis(bands), x, rtol=0, atol=1e-14)
    # orthonormal: energy preserved, and analysis of a synthesis is the identity too
    assert abs((bands ** 2).sum() - (x ** 2).sum()) < 1e-12 * (x ** 2).sum()
    b = rng.standard_normal((4, 5, 3))
    np.testing.assert_allclose(orc.haar_analysis(orc.haar_synthesis(b)), b, rtol=0, atol=1e-14)


def test_haar_band_positions(orc):
    """Band b of block (i, j) reads exactly rows 2i..2i+1 and columns 2j..2j+1."""
    x = np.zeros((6, 8))
    x[2, 5] = 2.0  # block (1, 2), position b = top-right
    bands = orc.haar_analysis(x)
    nz = np.argwhere(bands != 0)
    assert {tuple(t[1:]) for t in nz} == {(1, 2)}
    np.testing.assert_array_equal(bands[:, 1, 2], [1.0, 1.0, -1.0, -1.0])


# ---------------------------------------------------------------------------
# Convolution orientation and the base path
# ---------------------------------------------------------------------------

def test_corr_same_matches_torch_conv2d(orc):
    rng = np.random.default_rng(3)
    for k in (1, 3, 5, 7):
        x = rng.standard_normal((9, 14))
        kern = rng.standard_normal((k, k))
        ref = torch.nn.functional.conv2d(torch.from_numpy(x)[None, None], torch.from_numpy(kern)[None, None],
                                         padding=(k - 1) // 2)[0, 0].numpy()
        np.testing.assert_allclose(orc.corr_same(x, kern), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("k", [1, 3, 5, 7])
def test_level0_is_scaled_depthwise_conv(orc, k):
    """With no levels the layer is s0 * (depthwise conv + bias) (torch on CPU, fp64)."""
    rng = np.random.default_rng(5 + k)
    n, c, h, w = 2, 3, 10, 13
    x = rng.standard_normal((n, c, h, w))
    w0, b0, s0, _, _ = _rand_params(rng, c, k, 0)
    y = orc.forward(x, w0, b0, s0, None, None, k, 0)
    ref = torch.nn.functional.conv2d(torch.from_numpy(x), torch.from_numpy(w0)[:, None], torch.from_numpy(b0),
                                     padding=(k - 1) // 2, groups=c).numpy() * s0[None, :, None, None]
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)
    # bias may be absent
    y0 = orc.forward(x, w0, None, s0, None, None, k, 0)
    np.testing.assert_allclose(y - y0, (b0 * s0)[None, :, None, None] * np.ones_like(y), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms of the cascade
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("levels", [1, 2, 3, 4])
def test_identity_kernels_give_block_means(orc, levels):
    """k=1, unit level weights, per-level scale a_l on all four bands, no base path:
    level l reconstructs exactly its input map LL_{l-1}, i.e. the mean over
    2^(l-1) blocks, so y = sum_l a_l * blockmean_{2^(l-1)}(x)."""
    rng = np.random.default_rng(20 + levels)
    n, c, h, w = 1, 2, 16, 32
    x = rng.standard_normal((n, c, h, w))
    a = rng.uniform(0.5, 2.0, size=levels)
    wl = np.ones((levels, 4 * c, 1, 1))
    sl = np.repeat(a[:, None], 4 * c, axis=1)
    y = orc.forward(x, np.ones((c, 1, 1)), None, np.zeros(c), wl, sl, 1, levels)
    ref = sum(a[l - 1] * _up(_blockmean(x, 2 ** (l - 1)), 2 ** (l - 1)) for l in range(1, levels + 1))
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("levels", [1, 2, 3])
def test_lowpass_only_gives_coarser_block_means(orc, levels):
    """Same, but only the low-pass band of each level carries a scale: level l
    then keeps only LL_l, so y = sum_l a_l * blockmean_{2^l}(x)."""
    rng = np.random.default_rng(30 + levels)
    n, c, h, w = 2, 1, 32, 16
    x = rng.standard_normal((n, c, h, w))
    a = rng.uniform(0.5, 2.0, size=levels)
    wl = np.ones((levels, 4 * c, 1, 1))
    sl = np.zeros((levels, 4 * c))
    sl[:, 0::4] = a[:, None]
    y = orc.forward(x, np.ones((c, 1, 1)), None, np.zeros(c), wl, sl, 1, levels)
    ref = sum(a[l - 1] * _up(_blockmean(x, 2 ** l), 2 ** l) for l in range(1, levels + 1))
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("level,du,dv", [(1, 1, -1), (2, -1, 2), (3, 2, 0), (2, 0, -2)])
def test_shifted_delta_kernel_per_level(orc, level, du, dv):
    """A level whose four kernels are one unit tap at offset (du, dv) from the
    centre (k=5) and all other levels off: the band maps are shifted by whole
    level-l pixels, so the output is LL_{l-1} shifted by 2*(du, dv) level-(l-1)
    pixels with zero fill, brought back up: the 2^(l-1) block mean, shifted by
    2^l * (du, dv) full-resolution pixels.  Pins the orientation of the
    per-level cross-correlation and the level alignment."""
    rng = np.random.default_rng(40 + level)
    L, k, r = 3, 5, 2
    n, c, h, w = 1, 1, 32, 48
    x = rng.standard_normal((n, c, h, w))
    wl = np.zeros((L, 4 * c, k, k))
    wl[level - 1, :, r + du, r + dv] = 1.0
    sl = np.zeros((L, 4 * c))
    sl[level - 1] = 1.0
    y = orc.forward(x, np.zeros((c, k, k)), None, np.zeros(c), wl, sl, k, L)
    f = 2 ** (level - 1)
    bm = _blockmean(x, f)[0, 0]
    sh = np.zeros_like(bm)
    ci, cj = bm.shape
    si, sj = 2 * du, 2 * dv  # y(i) = bm(i + shift) with cross-correlation
    for i in range(ci):
        for j in range(cj):
            ii, jj = i + si, j + sj
            if 0 <= ii < ci and 0 <= jj < cj:
                sh[i, j] = bm[ii, jj]
    np.testing.assert_allclose(y[0, 0], _up(sh, f), rtol=0, atol=1e-13)


def test_band_identity(orc):
    """Band 1 is the row difference and band 2 the column difference: an input
    constant along each column (varying only with w) has no band-1 or band-3
    content at any level, one constant along each row has no band-2 or band-3
    content."""
    rng = np.random.default_rng(50)
    L, k, c, h, w = 3, 3, 1, 16, 24
    vary_w = np.broadcast_to(rng.standard_normal(w)[None, :], (h, w)).copy()[None, None]
    vary_h = np.broadcast_to(rng.standard_normal(h)[:, None], (h, w)).copy()[None, None]
    wl = rng.standard_normal((L, 4 * c, k, k))
    zero_base = (np.zeros((c, k, k)), None, np.zeros(c))

    def only(band):
        sl = np.zeros((L, 4 * c))
        sl[:, band] = 1.0
        return sl

    for band, x, vanishes in [(1, vary_w, True), (3, vary_w, True), (2, vary_w, False),
                              (2, vary_h, True), (3, vary_h, True), (1, vary_h, False)]:
        y = orc.forward(x, *zero_base, wl, only(band), k, L)
        if vanishes:  # zero up to the rounding of (a + b) - c - d with a = c, b = d
            assert np.abs(y).max() < 1e-13, band
        else:
            assert np.abs(y).max() > 1e-3, band


def test_closed_form_synthesis_matches_cascade(orc):
    """The bit-indexed closed form of the synthesis (method reformulation 2):
    y_levels[h, w] = sum_l 2^-l sum_b sign_b(p_l, q_l) Z_l^b[h >> l, w >> l],
    p_l = bit (l-1) of h, q_l = bit (l-1) of w, signs +1, (-1)^p, (-1)^q,
    (-1)^(p+q), evaluated on the oracle's own band outputs, equals the oracle's
    cascaded reconstruction."""
    rng = np.random.default_rng(60)
    L, k, c, h, w = 4, 5, 1, 32, 48
    x = rng.standard_normal((1, c, h, w))
    _, _, _, wl, sl = _rand_params(rng, c, k, L)
    y = orc.forward(x, np.zeros((c, k, k)), None, np.zeros(c), wl, sl, k, L)[0, 0]
    z = orc.level_outputs(x[0, 0], wl[:, 0:4], sl[:, 0:4], k, L)
    hh, ww = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    ref = np.zeros((h, w))
    for l in range(1, L + 1):
        p = (hh >> (l - 1)) & 1
        q = (ww >> (l - 1)) & 1
        zl = z[l - 1]
        i, j = hh >> l, ww >> l
        ref += 2.0 ** -l * (zl[0][i, j] + (-1.0) ** p * zl[1][i, j] + (-1.0) ** q * zl[2][i, j]
                            + (-1.0) ** (p + q) * zl[3][i, j])
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Structure: linearity, equivariance, determinism
# ---------------------------------------------------------------------------

def test_linearity_and_bilinearity(orc):
    rng = np.random.default_rng(70)
    n, c, h, w, k, L = 2, 2, 16, 8, 3, 3
    w0, b0, s0, wl, sl = _rand_params(rng, c, k, L)
    x1, x2 = rng.standard_normal((2, n, c, h, w))
    f = lambda x, **kw: orc.forward(x, kw.get("w0", w0), b0, s0, kw.get("wl", wl), kw.get("sl", sl), k, L)
    y0 = f(np.zeros_like(x1))
    np.testing.assert_allclose(f(2.0 * x1 - 3.0 * x2) - y0, 2.0 * (f(x1) - y0) - 3.0 * (f(x2) - y0),
                               rtol=0, atol=1e-11)
    # scale and level weight enter as a product
    np.testing.assert_allclose(f(x1, wl=wl * 4.0, sl=sl * 0.25), f(x1), rtol=0, atol=1e-12)
    # the level part is linear in the level weights for fixed scales
    yb = orc.forward(x1, w0, b0, s0, wl * 0.0, sl, k, L)
    np.testing.assert_allclose(f(x1, wl=3.0 * wl) - yb, 3.0 * (f(x1) - yb), rtol=0, atol=1e-11)


def test_translation_equivariance_by_2_to_L(orc):
    """Away from the borders the layer commutes with shifts by multiples of 2^L
    (the Haar grid is preserved) but not with a shift by one pixel."""
    rng = np.random.default_rng(80)
    L, k, c, h, w = 3, 3, 1, 64, 64
    w0, b0, s0, wl, sl = _rand_params(rng, c, k, L)
    x = np.zeros((1, c, h, w))
    x[..., 24:40, 24:40] = rng.standard_normal((16, 16))
    f = lambda t: orc.forward(t, w0, None, s0, wl, sl, k, L)
    y = f(x)
    y_s = f(np.roll(x, (8, -16), axis=(2, 3)))
    np.testing.assert_allclose(y_s, np.roll(y, (8, -16), axis=(2, 3)), rtol=0, atol=1e-12)
    y_1 = f(np.roll(x, (1, 0), axis=(2, 3)))
    assert np.abs(y_1 - np.roll(y, (1, 0), axis=(2, 3))).max() > 1e-3


def test_thread_count_does_not_change_results(orc):
    inp = make_inputs(3, 4, 16, 24, 5, 3, seed=5)
    args = (inp.w_base, inp.bias, inp.s_base, inp.w_lvl, inp.s_lvl, 5, 3)
    np.testing.assert_array_equal(orc.forward(inp.x, *args, nthreads=1), orc.forward(inp.x, *args, nthreads=7))
    g1 = orc.backward_weight(inp.x, inp.dy, *args, nthreads=1)
    g7 = orc.backward_weight(inp.x, inp.dy, *args, nthreads=5)
    for a, b in zip(g1, g7):
        np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# Backward: brute-force matrix, adjoint identity, finite differences
# ---------------------------------------------------------------------------

def _dense_matrix(orc, h, w, k, L, w0, s0, wl, sl):
    """Matrix of the (bias-free) one-channel layer built by probing unit impulses."""
    cols = []
    for idx in range(h * w):
        e = np.zeros((1, 1, h, w))
        e.flat[idx] = 1.0
        cols.append(orc.forward(e, w0, None, s0, wl, sl, k, L).reshape(-1))
    return np.stack(cols, axis=1)


@pytest.mark.parametrize("k,L,h,w", [(3, 2, 8, 12), (5, 3, 16, 8)])
def test_dense_matrix_forward_and_backward_data(orc, k, L, h, w):
    rng = np.random.default_rng(90 + k)
    w0, b0, s0, wl, sl = _rand_params(rng, 1, k, L)
    M = _dense_matrix(orc, h, w, k, L, w0, s0, wl, sl)
    x = rng.standard_normal((1, 1, h, w))
    dy = rng.standard_normal((1, 1, h, w))
    y = orc.forward(x, w0, b0, s0, wl, sl, k, L)
    np.testing.assert_allclose(y.reshape(-1), M @ x.reshape(-1) + s0[0] * b0[0], rtol=0, atol=1e-12)
    dx = orc.backward_data(dy, w0, s0, wl, sl, k, L)
    np.testing.assert_allclose(dx.reshape(-1), M.T @ dy.reshape(-1), rtol=0, atol=1e-12)
    # the transpose is the same layer with every kernel turned by 180 degrees and no bias
    Mt = _dense_matrix(orc, h, w, k, L, w0[:, ::-1, ::-1], s0, wl[:, :, ::-1, ::-1], sl)
    np.testing.assert_allclose(Mt, M.T, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", [(2, 96, 56, 56, 5, 3), (1, 2, 256, 256, 5, 4), (1, 3, 128, 128, 5, 5)])
def test_adjoint_identity_at_workload_shapes(orc, shape):
    """<y(x) - y(0), dy> = <x, dx(dy)> at the workloads' plane shapes."""
    n, c, h, w, k, L = shape
    inp = make_inputs(n, c, h, w, k, L, seed=7)
    x, dy = inp.x.astype(np.float64), inp.dy.astype(np.float64)
    y = orc.forward(x, inp.w_base, None, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    dx = orc.backward_data(dy, inp.w_base, inp.s_base, inp.w_lvl, inp.s_lvl, k, L)
    lhs, rhs = float((y * dy).sum()), float((x * dx).sum())
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + np.sqrt((y * y).sum() * (dy * dy).sum()))


def test_parameter_gradients_by_finite_differences(orc):
    """The loss <dy, y> is affine in each single parameter, so a central
    difference is exact up to rounding: pins every entry of dW0, db0, ds0,
    dW_l and ds_l (including the chain rule through the scales)."""
    rng = np.random.default_rng(100)
    n, c, h, w, k, L = 2, 2, 8, 16, 3, 2
    x = rng.standard_normal((n, c, h, w))
    dy = rng.standard_normal((n, c, h, w))
    params = list(_rand_params(rng, c, k, L))
    grads = orc.backward_weight(x, dy, *params, k, L)

    def loss(p):
        return float((orc.forward(x, *p, k, L) * dy).sum())

    for pi, g in enumerate(grads):
        flat = params[pi].reshape(-1)
        fd = np.empty(flat.size)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + 0.5
            lp = loss(params)
            flat[i] = old - 0.5
            lm = loss(params)
            flat[i] = old
            fd[i] = lp - lm
        np.testing.assert_allclose(np.asarray(g).reshape(-1), fd, rtol=0, atol=1e-10 * (1 + np.abs(fd).max()))


def test_backward_data_by_finite_differences(orc):
    rng = np.random.default_rng(110)
    n, c, h, w, k, L = 1, 2, 8, 8, 5, 3
    x = rng.standard_normal((n, c, h, w))
    dy = rng.standard_normal((n, c, h, w))
    w0, b0, s0, wl, sl = _rand_params(rng, c, k, L)
    dx = orc.backward_data(dy, w0, s0, wl, sl, k, L)
    for idx in rng.choice(x.size, 12, replace=False):
        xp, xm = x.copy(), x.copy()
        xp.flat[idx] += 0.5
        xm.flat[idx] -= 0.5
        fd = float(((orc.forward(xp, w0, b0, s0, wl, sl, k, L) - orc.forward(xm, w0, b0, s0, wl, sl, k, L))
                    * dy).sum())
        assert abs(fd - dx.flat[idx]) < 1e-11 * (1 + abs(fd))


def test_rejects_bad_shapes(orc):
    x = np.zeros((1, 1, 12, 12))
    with pytest.raises(ValueError):  # even kernel side
        orc.forward(x, np.zeros((1, 4, 4)), None, np.ones(1), None, None, 4, 0)
    with pytest.raises(ValueError):  # more levels than the oracle keeps
        orc.forward(x, np.zeros((1, 3, 3)), None, np.ones(1), np.zeros((16, 4, 3, 3)), np.ones((16, 4)), 3, 16)


# ---------------------------------------------------------------------------
# Sides not divisible by 2^L: each odd map is padded with one zero row at the
# bottom / one zero column at the right before its analysis, and that level's
# synthesis is cropped back (level l is ceil(H / 2^l) x ceil(W / 2^l))
# ---------------------------------------------------------------------------

def _padded_blockmean_up(x, f):
    """Mean over the f x f blocks of x zero-padded at the bottom and right to
    multiples of f (a block that sticks out still divides by f^2), spread back
    over its pixels and cropped to x's size."""
    *lead, h, w = x.shape
    hp, wp = -(-h // f) * f, -(-w // f) * f
    xp = np.zeros((*lead, hp, wp))
    xp[..., :h, :w] = x
    return _up(_blockmean(xp, f), f)[..., :h, :w]


@pytest.mark.parametrize("levels,h,w", [(1, 7, 10), (2, 13, 22), (3, 9, 17), (4, 21, 6), (3, 3, 5)])
def test_ragged_identity_kernels_give_zero_padded_block_means(orc, levels, h, w):
    """k = 1, unit level weights, scale a_l on all four bands, no base path: level
    l reconstructs its (cropped) input map exactly, so y = sum_l a_l times the
    2^(l-1) block means of x with zeros past the bottom and right edges."""
    rng = np.random.default_rng(200 + levels + h)
    n, c = 2, 2
    x = rng.standard_normal((n, c, h, w))
    a = rng.uniform(0.5, 2.0, size=levels)
    wl = np.ones((levels, 4 * c, 1, 1))
    sl = np.repeat(a[:, None], 4 * c, axis=1)
    y = orc.forward(x, np.ones((c, 1, 1)), None, np.zeros(c), wl, sl, 1, levels)
    ref = sum(a[l - 1] * _padded_blockmean_up(x, 2 ** (l - 1)) for l in range(1, levels + 1))
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("levels,h,w", [(1, 7, 10), (2, 13, 22), (3, 9, 17), (3, 5, 3)])
def test_ragged_lowpass_only_gives_zero_padded_block_means(orc, levels, h, w):
    """Only the low-pass band scaled: y = sum_l a_l times the 2^l block means of
    the zero-padded x (the padding of every level is where the closed form puts
    it: bottom and right, blocks anchored at the top-left corner)."""
    rng = np.random.default_rng(210 + levels + w)
    n, c = 1, 3
    x = rng.standard_normal((n, c, h, w))
    a = rng.uniform(0.5, 2.0, size=levels)
    wl = np.ones((levels, 4 * c, 1, 1))
    sl = np.zeros((levels, 4 * c))
    sl[:, 0::4] = a[:, None]
    y = orc.forward(x, np.ones((c, 1, 1)), None, np.zeros(c), wl, sl, 1, levels)
    ref = sum(a[l - 1] * _padded_blockmean_up(x, 2 ** l) for l in range(1, levels + 1))
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("k,L,h,w", [(3, 2, 7, 10), (5, 3, 9, 5), (3, 3, 3, 6)])
def test_ragged_dense_matrix_forward_and_backward_data(orc, k, L, h, w):
    """Brute force on ragged planes: dx is the transpose of the probed forward
    matrix, and that transpose is the layer with 180-degree kernels."""
    rng = np.random.default_rng(220 + k + h)
    w0, b0, s0, wl, sl = _rand_params(rng, 1, k, L)
    M = _dense_matrix(orc, h, w, k, L, w0, s0, wl, sl)
    x = rng.standard_normal((1, 1, h, w))
    dy = rng.standard_normal((1, 1, h, w))
    y = orc.forward(x, w0, b0, s0, wl, sl, k, L)
    np.testing.assert_allclose(y.reshape(-1), M @ x.reshape(-1) + s0[0] * b0[0], rtol=0, atol=1e-12)
    dx = orc.backward_data(dy, w0, s0, wl, sl, k, L)
    np.testing.assert_allclose(dx.reshape(-1), M.T @ dy.reshape(-1), rtol=0, atol=1e-12)
    Mt = _dense_matrix(orc, h, w, k, L, w0[:, ::-1, ::-1], s0, wl[:, :, ::-1, ::-1], sl)
    np.testing.assert_allclose(Mt, M.T, rtol=0, atol=1e-12)


def test_ragged_parameter_gradients_by_finite_differences(orc):
    """Every parameter gradient on a ragged plane against exact central
    differences of the (parameter-wise affine) loss <dy, y>."""
    rng = np.random.default_rng(230)
    n, c, h, w, k, L = 2, 2, 7, 11, 3, 2
    x = rng.standard_normal((n, c, h, w))
    dy = rng.standard_normal((n, c, h, w))
    params = list(_rand_params(rng, c, k, L))
    grads = orc.backward_weight(x, dy, *params, k, L)

    def loss(p):
        return float((orc.forward(x, *p, k, L) * dy).sum())

    for pi, g in enumerate(grads):
        flat = params[pi].reshape(-1)
        fd = np.empty(flat.size)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + 0.5
            lp = loss(params)
            flat[i] = old - 0.5
            lm = loss(params)
            flat[i] = old
            fd[i] = lp - lm
        np.testing.assert_allclose(np.asarray(g).reshape(-1), fd, rtol=0, atol=1e-10 * (1 + np.abs(fd).max()))


@pytest.mark.parametrize("k,L,h,w,extra", [(5, 2, 13, 22, 0), (3, 3, 9, 17, 0), (5, 3, 10, 7, 8), (7, 1, 5, 9, 2)])
def test_ragged_equals_layer_on_zero_padded_input(orc, k, L, h, w, extra):
    """Padding every odd level map by one zero row / column is the same as
    padding x once with zeros at the bottom and right to a multiple of 2^L (or
    further) and cropping: the padded pixels only ever feed outputs that are
    cropped away, and every level's zero 'same' padding sees zeros either way.
    So the ragged layer equals the (already pinned) divisible layer on the
    zero-padded input, cropped; its data backward equals the divisible one on
    the zero-padded dy, cropped; its parameter gradients are those of the
    padded pair (x, dy)."""
    rng = np.random.default_rng(240 + h + w + extra)
    n, c = 2, 2
    x = rng.standard_normal((n, c, h, w))
    dy = rng.standard_normal((n, c, h, w))
    params = _rand_params(rng, c, k, L)
    f = 2 ** L
    hp, wp = -(-h // f) * f + extra, -(-w // f) * f + extra
    pad = lambda a: np.pad(a, ((0, 0), (0, 0), (0, hp - h), (0, wp - w)))
    y = orc.forward(x, *params, k, L)
    np.testing.assert_allclose(y, orc.forward(pad(x), *params, k, L)[:, :, :h, :w], rtol=0, atol=1e-12)
    w0, _, s0, wl, sl = params
    dx = orc.backward_data(dy, w0, s0, wl, sl, k, L)
    np.testing.assert_allclose(dx, orc.backward_data(pad(dy), w0, s0, wl, sl, k, L)[:, :, :h, :w], rtol=0,
                               atol=1e-12)
    for g, gp in zip(orc.backward_weight(x, dy, *params, k, L), orc.backward_weight(pad(x), pad(dy), *params, k, L)):
        np.testing.assert_allclose(g, gp, rtol=1e-12, atol=1e-10)
