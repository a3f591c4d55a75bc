/*
 * wtconv_oracle.c -- plain, slow CPU definition of the WTConv layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite (tests/), the smoke check in
 * __graft_entry__.py and the cpu_baseline leg of bench.py may load or call this
 * library.  The GPU library (level_haar_wavelet_amd/csrc) shares no code, header,
 * table or helper with this file, and this file includes nothing from it.
 *
 * Everything is computed in double precision with the layer written out in its
 * unfused form, one step after another, so that it can be checked against the
 * pages by eye:
 *   base depthwise conv + bias, times the base scale;
 *   an L-level orthonormal 2D Haar analysis of the input;
 *   a k x k depthwise conv of each of the 4 subbands at every level, times a
 *   learned per-(channel, band) scale;
 *   the cascaded Haar synthesis from the deepest level upward, adding the
 *   reconstruction of the level below into the (convolved, scaled) low-pass band;
 *   and the backward pass by explicit reverse mode through that same graph.
 *
 * Sources.  The pages are five renderings of "Fast and Memory-Efficient Wavelet
 * Convolutions via I/O-Aware Reformulation" (Aflalo, Finder, Amoyal, Treister,
 * Freifeld; arXiv 2608.10805): the arxivdaily.com page (English abstract) and the
 * gist.science explainers (German, French, Spanish, Japanese) with a technical
 * summary.  Citations below name the section of that summary:
 *   [abstract]        English abstract: WTConv is a drop-in replacement for a
 *                     depthwise conv whose receptive field grows with the number
 *                     of decomposition levels while parameters grow linearly.
 *   [problem]         technical summary, problem statement: the reference
 *                     materialises wavelet coefficients and reconstructions at
 *                     every stage.
 *   [method 1]        technical summary, methodology, reformulation 1: the Haar
 *                     analysis uses only signed additions and fixed power-of-two
 *                     scalings; it produces the coefficient tensor Y^(l).
 *   [method 2]        technical summary, methodology, reformulation 2: the
 *                     reference reconstruction is a sequential L-step loop; each
 *                     step adds the previous reconstruction to the low-pass
 *                     subband and applies a transposed convolution.
 *   [method 3]        technical summary, methodology, reformulation 3: learned
 *                     per-channel scales are a separate elementwise pass after
 *                     the convolution; the base path has a bias.
 *   [contributions]   technical summary, key contributions: the fused form keeps
 *                     the operator up to floating-point evaluation order; forward
 *                     outputs and all parameter gradients were validated.
 *
 * Readings taken where the pages are silent (each is listed with its reason in
 * the design notes of the repository):
 *   - orthonormal Haar: 2x2 taps of +-1/2 (power-of-two scaling, [method 1]);
 *   - band order inside the 4C subbands: b = 0 low-pass, 1 row difference
 *     (top row minus bottom row), 2 column difference (left minus right),
 *     3 diagonal; channel index of band b of channel c is 4c+b;
 *   - the input of level l+1 is the raw (unconvolved) low-pass band of level l;
 *   - the cascade adds the reconstruction of level l+1 to the convolved and
 *     scaled low-pass band of level l ([method 2]);
 *   - base path: y0 = s0 * (W0 (*) x + b0); per-level convs have no bias
 *     ([method 3]);
 *   - every convolution is a cross-correlation with zero 'same' padding and
 *     stride 1 at the resolution of its own level; k is odd;
 *   - a map with an odd side is padded with one zero row at the bottom and/or
 *     one zero column at the right before its Haar analysis, and the synthesis
 *     of that level is cropped back to the map's size, so level l is
 *     ceil(H / 2^l) x ceil(W / 2^l) (when 2^L divides H and W nothing is
 *     padded).
 *
 * Parameter layout (all double here):
 *   w_base [C][k][k], bias [C] (may be NULL = zero), s_base [C],
 *   w_lvl  [L][4C][k][k] (band b of channel c at index 4c+b), s_lvl [L][4C].
 * Activations are NCHW contiguous.
 *
 * Return value of every exported function: 0 on success, -1 on a bad argument,
 * -2 when memory could not be allocated.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Building blocks on one (h x w) map                                         */
/* ------------------------------------------------------------------------ */

/* Side of a level-l map of an h-pixel side: ceil(h / 2^l) (an odd side is
 * padded by one zero before each analysis). */
static int64_t lvl_dim(int64_t h, int l) { return (h + ((int64_t)1 << l) - 1) >> l; }

/* Pixel (i, j) of an h x w map, zero outside it (the zero padding of an odd
 * side). */
static double px(const double *in, int64_t h, int64_t w, int64_t i, int64_t j)
{
    return (i < h && j < w) ? in[i * w + j] : 0.0;
}

/* One level of the 2D Haar analysis [method 1].  in is h x w; each 2x2 block
 * (a b / c d) gives one coefficient in each of the four bands:
 *   band 0 = (a+b+c+d)/2, band 1 = (a+b-c-d)/2, band 2 = (a-b+c-d)/2,
 *   band 3 = (a-b-c+d)/2.
 * out holds the 4 bands one after another, each ceil(h/2) x ceil(w/2); pixels
 * past an odd side count as zero. */
static void haar_analysis(const double *in, int64_t h, int64_t w, double *out)
{
    int64_t h2 = lvl_dim(h, 1), w2 = lvl_dim(w, 1), m = h2 * w2;
    for (int64_t i = 0; i < h2; i++) {
        for (int64_t j = 0; j < w2; j++) {
            double a = px(in, h, w, 2 * i, 2 * j);
            double b = px(in, h, w, 2 * i, 2 * j + 1);
            double c = px(in, h, w, 2 * i + 1, 2 * j);
            double d = px(in, h, w, 2 * i + 1, 2 * j + 1);
            out[0 * m + i * w2 + j] = 0.5 * (a + b + c + d);
            out[1 * m + i * w2 + j] = 0.5 * (a + b - c - d);
            out[2 * m + i * w2 + j] = 0.5 * (a - b + c - d);
            out[3 * m + i * w2 + j] = 0.5 * (a - b - c + d);
        }
    }
}

/* Adjoint of haar_analysis: each band coefficient is scattered back onto its
 * 2x2 block with the same +-1/2 weights it was gathered with; what falls on the
 * zero padding is dropped (the adjoint of padding is cropping).  out is h x w
 * and is overwritten. */
static void haar_analysis_adjoint(const double *bands, int64_t h, int64_t w, double *out)
{
    int64_t h2 = lvl_dim(h, 1), w2 = lvl_dim(w, 1), m = h2 * w2;
    memset(out, 0, (size_t)(h * w) * sizeof(double));
    for (int64_t i = 0; i < h2; i++) {
        for (int64_t j = 0; j < w2; j++) {
            double g0 = bands[0 * m + i * w2 + j];
            double g1 = bands[1 * m + i * w2 + j];
            double g2 = bands[2 * m + i * w2 + j];
            double g3 = bands[3 * m + i * w2 + j];
            int row1 = 2 * i + 1 < h, col1 = 2 * j + 1 < w;
            /* a: coefficient +1/2 in all four bands */
            out[(2 * i) * w + 2 * j] += 0.5 * g0 + 0.5 * g1 + 0.5 * g2 + 0.5 * g3;
            /* b: +, +, -, - */
            if (col1) out[(2 * i) * w + 2 * j + 1] += 0.5 * g0 + 0.5 * g1 - 0.5 * g2 - 0.5 * g3;
            /* c: +, -, +, - */
            if (row1) out[(2 * i + 1) * w + 2 * j] += 0.5 * g0 - 0.5 * g1 + 0.5 * g2 - 0.5 * g3;
            /* d: +, -, -, + */
            if (row1 && col1) out[(2 * i + 1) * w + 2 * j + 1] += 0.5 * g0 - 0.5 * g1 - 0.5 * g2 + 0.5 * g3;
        }
    }
}

/* One level of the Haar synthesis (the inverse of haar_analysis, which is an
 * orthogonal map, so the synthesis is the transposed analysis) [method 2].
 * bands: 4 maps of h2 x w2, the analysis of an h x w map (h2 = ceil(h/2),
 * w2 = ceil(w/2)); out: h x w, overwritten, i.e. the (2 h2) x (2 w2)
 * reconstruction cropped back to the analysed map.  The pixel at row parity p
 * and column parity q of block (i, j) is
 *   (band0 + (-1)^p band1 + (-1)^q band2 + (-1)^(p+q) band3) / 2. */
static void haar_synthesis(const double *bands, int64_t h2, int64_t w2, int64_t h, int64_t w, double *out)
{
    int64_t m = h2 * w2;
    for (int64_t i = 0; i < h2; i++) {
        for (int64_t j = 0; j < w2; j++) {
            double b0 = bands[0 * m + i * w2 + j];
            double b1 = bands[1 * m + i * w2 + j];
            double b2 = bands[2 * m + i * w2 + j];
            double b3 = bands[3 * m + i * w2 + j];
            int row1 = 2 * i + 1 < h, col1 = 2 * j + 1 < w;
            out[(2 * i) * w + 2 * j] = 0.5 * (b0 + b1 + b2 + b3);
            if (col1) out[(2 * i) * w + 2 * j + 1] = 0.5 * (b0 + b1 - b2 - b3);
            if (row1) out[(2 * i + 1) * w + 2 * j] = 0.5 * (b0 - b1 + b2 - b3);
            if (row1 && col1) out[(2 * i + 1) * w + 2 * j + 1] = 0.5 * (b0 - b1 - b2 + b3);
        }
    }
}

/* Adjoint of haar_synthesis: gathers the gradient of the four pixels of each
 * block back into the four band coefficients with the synthesis weights; g is
 * h x w, and the pixels the crop removed contribute zero. */
static void haar_synthesis_adjoint(const double *g, int64_t h2, int64_t w2, int64_t h, int64_t w, double *bands)
{
    int64_t m = h2 * w2;
    for (int64_t i = 0; i < h2; i++) {
        for (int64_t j = 0; j < w2; j++) {
            double ga = px(g, h, w, 2 * i, 2 * j);         /* p=0, q=0 */
            double gb = px(g, h, w, 2 * i, 2 * j + 1);     /* p=0, q=1 */
            double gc = px(g, h, w, 2 * i + 1, 2 * j);     /* p=1, q=0 */
            double gd = px(g, h, w, 2 * i + 1, 2 * j + 1); /* p=1, q=1 */
            bands[0 * m + i * w2 + j] = 0.5 * (ga + gb + gc + gd);
            bands[1 * m + i * w2 + j] = 0.5 * (ga + gb - gc - gd);
            bands[2 * m + i * w2 + j] = 0.5 * (ga - gb + gc - gd);
            bands[3 * m + i * w2 + j] = 0.5 * (ga - gb - gc + gd);
        }
    }
}

/* Depthwise k x k cross-correlation of one map with zero 'same' padding:
 *   out[i][j] = sum_{u,v} kern[u][v] * in[i+u-r][j+v-r],  r = (k-1)/2,
 * with in = 0 outside [0,h) x [0,w).  out is overwritten. */
static void corr_same(const double *in, int64_t h, int64_t w, const double *kern, int k, double *out)
{
    int r = (k - 1) / 2;
    for (int64_t i = 0; i < h; i++) {
        for (int64_t j = 0; j < w; j++) {
            double acc = 0.0;
            for (int u = 0; u < k; u++) {
                int64_t ii = i + u - r;
                if (ii < 0 || ii >= h) continue;
                for (int v = 0; v < k; v++) {
                    int64_t jj = j + v - r;
                    if (jj < 0 || jj >= w) continue;
                    acc += kern[u * k + v] * in[ii * w + jj];
                }
            }
            out[i * w + j] = acc;
        }
    }
}

/* Adjoint of corr_same with respect to its input: every output gradient g[i][j]
 * is scattered back onto the input positions it was computed from.  out is
 * overwritten. */
static void corr_same_adjoint(const double *g, int64_t h, int64_t w, const double *kern, int k, double *out)
{
    int r = (k - 1) / 2;
    memset(out, 0, (size_t)(h * w) * sizeof(double));
    for (int64_t i = 0; i < h; i++) {
        for (int64_t j = 0; j < w; j++) {
            double gij = g[i * w + j];
            for (int u = 0; u < k; u++) {
                int64_t ii = i + u - r;
                if (ii < 0 || ii >= h) continue;
                for (int v = 0; v < k; v++) {
                    int64_t jj = j + v - r;
                    if (jj < 0 || jj >= w) continue;
                    out[ii * w + jj] += kern[u * k + v] * gij;
                }
            }
        }
    }
}

/* Gradient of corr_same with respect to its kernel, added into gk:
 *   gk[u][v] += sum_{i,j} g[i][j] * in[i+u-r][j+v-r]   (zero outside). */
static void corr_same_kernel_grad(const double *g, const double *in, int64_t h, int64_t w, int k, double *gk)
{
    int r = (k - 1) / 2;
    for (int u = 0; u < k; u++) {
        for (int v = 0; v < k; v++) {
            double acc = 0.0;
            for (int64_t i = 0; i < h; i++) {
                int64_t ii = i + u - r;
                if (ii < 0 || ii >= h) continue;
                for (int64_t j = 0; j < w; j++) {
                    int64_t jj = j + v - r;
                    if (jj < 0 || jj >= w) continue;
                    acc += g[i * w + j] * in[ii * w + jj];
                }
            }
            gk[u * k + v] += acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Per-plane layer: the unfused graph of one (n, c) plane                     */
/* ------------------------------------------------------------------------ */

/* Parameters of one channel gathered from the packed tensors. */
typedef struct {
    int k, levels;
    const double *w0;   /* [k][k] */
    double b0, s0;
    const double *wl[16]; /* per level, 4 consecutive [k][k] kernels (bands 0..3) */
    double sl[16][4];
} chan_params;

static void gather_params(chan_params *p, int64_t C, int64_t c, int k, int levels,
                          const double *w_base, const double *bias, const double *s_base,
                          const double *w_lvl, const double *s_lvl)
{
    int64_t kk = (int64_t)k * k;
    p->k = k;
    p->levels = levels;
    p->w0 = w_base + c * kk;
    p->b0 = bias ? bias[c] : 0.0;
    p->s0 = s_base[c];
    for (int l = 0; l < levels; l++) {
        p->wl[l] = w_lvl + ((int64_t)l * 4 * C + 4 * c) * kk;
        for (int b = 0; b < 4; b++) p->sl[l][b] = s_lvl[(int64_t)l * 4 * C + 4 * c + b];
    }
}

/* Sizes of the level maps: level l is ceil(h / 2^l) x ceil(w / 2^l). */
static int64_t map_elems(int64_t h, int64_t w, int l) { return lvl_dim(h, l) * lvl_dim(w, l); }

/* Offsets into one buffer holding, for l = 1..L, the 4 band maps of level l. */
static int64_t level_offset(int64_t h, int64_t w, int l)
{
    int64_t off = 0;
    for (int m = 1; m < l; m++) off += 4 * map_elems(h, w, m);
    return off;
}

static int64_t pyramid_elems(int64_t h, int64_t w, int levels) { return level_offset(h, w, levels + 1); }

/* Forward analysis of one plane: for every level the 4 subbands A_l (raw
 * analysis coefficients) and, if zc is not NULL, the unscaled convolution of
 * each band Zc_l^b = W_l^b (*) A_l^b.  Level l+1 analyses the raw low-pass band
 * of level l.  a and zc are pyramid buffers laid out by level_offset. */
static void plane_analysis(const chan_params *p, int64_t h, int64_t w, const double *x, double *a, double *zc)
{
    int k = p->k;
    int64_t kk = (int64_t)k * k;
    const double *ll = x;
    for (int l = 1; l <= p->levels; l++) {
        int64_t hp = lvl_dim(h, l - 1), wp = lvl_dim(w, l - 1);
        int64_t hl = lvl_dim(h, l), wl = lvl_dim(w, l), m = hl * wl;
        double *al = a + level_offset(h, w, l);
        haar_analysis(ll, hp, wp, al);
        if (zc) {
            double *zl = zc + level_offset(h, w, l);
            for (int b = 0; b < 4; b++) corr_same(al + b * m, hl, wl, p->wl[l - 1] + b * kk, k, zl + b * m);
        }
        ll = al; /* band 0 of level l */
    }
}

/* Forward of one plane.  scratch must hold 2 * pyramid + 2 * h * w doubles. */
static void plane_forward(const chan_params *p, int64_t h, int64_t w, const double *x, double *y, double *scratch)
{
    int L = p->levels;
    int64_t hw = h * w, pyr = pyramid_elems(h, w, L);
    double *a = scratch, *zc = scratch + pyr, *r = scratch + 2 * pyr, *t = r + hw;

    /* base path: y0 = s0 * (W0 (*) x + b0) */
    corr_same(x, h, w, p->w0, p->k, y);
    for (int64_t i = 0; i < hw; i++) y[i] = p->s0 * (y[i] + p->b0);
    if (L == 0) return;

    /* analysis and per-level scaled convs: Z_l^b = s_l^b * (W_l^b (*) A_l^b) */
    plane_analysis(p, h, w, x, a, zc);
    for (int l = 1; l <= L; l++) {
        int64_t m = map_elems(h, w, l);
        double *zl = zc + level_offset(h, w, l);
        for (int b = 0; b < 4; b++)
            for (int64_t i = 0; i < m; i++) zl[b * m + i] *= p->sl[l - 1][b];
    }

    /* cascade, deepest level first: R_{L+1} = 0;
     * R_l = synthesis(Z_l^0 + R_{l+1}, Z_l^1, Z_l^2, Z_l^3). */
    memset(r, 0, (size_t)map_elems(h, w, L) * sizeof(double));
    for (int l = L; l >= 1; l--) {
        int64_t hl = lvl_dim(h, l), wl = lvl_dim(w, l), m = hl * wl;
        int64_t hp = lvl_dim(h, l - 1), wp = lvl_dim(w, l - 1);
        double *zl = zc + level_offset(h, w, l);
        for (int64_t i = 0; i < m; i++) zl[i] += r[i]; /* into the low-pass band */
        haar_synthesis(zl, hl, wl, hp, wp, t);          /* cropped to level l-1 */
        memcpy(r, t, (size_t)(hp * wp) * sizeof(double));
    }
    for (int64_t i = 0; i < hw; i++) y[i] += r[i];
}

/* Reverse mode, data part, of one plane: dx = d<dy, y>/dx.
 * scratch must hold 3 * pyramid + 3 * h * w doubles. */
static void plane_backward_data(const chan_params *p, int64_t h, int64_t w, const double *dy, double *dx, double *scratch)
{
    int L = p->levels, k = p->k;
    int64_t hw = h * w, kk = (int64_t)k * k, pyr = pyramid_elems(h, w, L);
    double *dz = scratch;               /* gradient at each level's band outputs Z_l */
    double *da = scratch + pyr;         /* gradient at each level's analysis outputs A_l */
    double *t = scratch + 2 * pyr;      /* h*w */
    double *dll = t + hw;               /* h*w : gradient flowing into LL_{l} */
    double *tmp = dll + hw;             /* h*w */

    /* base path: y0 = s0 * (W0 (*) x + b0)  ->  dx = s0 * adjoint(W0)(dy) */
    corr_same_adjoint(dy, h, w, p->w0, k, dx);
    for (int64_t i = 0; i < hw; i++) dx[i] *= p->s0;
    if (L == 0) return;

    /* cascade in reverse: dR_1 = dy; for l = 1..L the synthesis adjoint gives
     * the gradient of its four inputs; the low-pass one is also dR_{l+1}. */
    const double *dr = dy;
    for (int l = 1; l <= L; l++) {
        int64_t hl = lvl_dim(h, l), wl = lvl_dim(w, l);
        double *dzl = dz + level_offset(h, w, l);
        haar_synthesis_adjoint(dr, hl, wl, lvl_dim(h, l - 1), lvl_dim(w, l - 1), dzl);
        dr = dzl; /* band 0 map = gradient of R_{l+1} */
    }

    /* scaled convs: Z = s * Zc, Zc = W (*) A  ->  dA = adjoint(W)(s * dZ) */
    for (int l = 1; l <= L; l++) {
        int64_t hl = lvl_dim(h, l), wl = lvl_dim(w, l), m = hl * wl;
        double *dzl = dz + level_offset(h, w, l);
        double *dal = da + level_offset(h, w, l);
        for (int b = 0; b < 4; b++) {
            for (int64_t i = 0; i < m; i++) tmp[i] = p->sl[l - 1][b] * dzl[b * m + i];
            corr_same_adjoint(tmp, hl, wl, p->wl[l - 1] + b * kk, k, dal + b * m);
        }
    }

    /* analysis chain in reverse: A_l = analysis(LL_{l-1}), LL_l = A_l^0.
     * dLL_L = 0; dLL_{l-1} = analysis_adjoint(dA_l with dLL_l added to band 0). */
    memset(dll, 0, (size_t)map_elems(h, w, L) * sizeof(double));
    for (int l = L; l >= 1; l--) {
        int64_t hp = lvl_dim(h, l - 1), wp = lvl_dim(w, l - 1), m = map_elems(h, w, l);
        double *dal = da + level_offset(h, w, l);
        for (int64_t i = 0; i < m; i++) dal[i] += dll[i];
        haar_analysis_adjoint(dal, hp, wp, t);
        memcpy(dll, t, (size_t)(hp * wp) * sizeof(double));
    }
    for (int64_t i = 0; i < hw; i++) dx[i] += dll[i];
}

/* Reverse mode, parameter part, of one plane.  Adds this plane's gradient
 * contributions into g (length k*k + 2 + L*4*(k*k+1)):
 *   g[0 .. kk)         dW0,  g[kk] db0,  g[kk+1] ds0,
 *   then per level l, per band b: kk entries of dW_l^b, then per level the 4 ds_l^b
 *   (layout: [kk+2 + (l*4+b)*kk ...] for dW, [kk+2 + L*4*kk + l*4 + b] for ds).
 * scratch must hold 3 * pyramid + 2 * h * w doubles. */
static void plane_backward_weight(const chan_params *p, int64_t h, int64_t w, const double *x, const double *dy,
                                  double *g, double *scratch)
{
    int L = p->levels, k = p->k;
    int64_t hw = h * w, kk = (int64_t)k * k, pyr = pyramid_elems(h, w, L);
    double *a = scratch, *zc = scratch + pyr, *dz = scratch + 2 * pyr;
    double *zc0 = dz + pyr, *tmp = zc0 + hw;

    /* base path: y0 = s0 * (Zc0 + b0), Zc0 = W0 (*) x */
    corr_same(x, h, w, p->w0, k, zc0);
    double sdy = 0.0, sdyz = 0.0;
    for (int64_t i = 0; i < hw; i++) {
        sdy += dy[i];
        sdyz += dy[i] * (zc0[i] + p->b0);
    }
    for (int64_t i = 0; i < hw; i++) tmp[i] = p->s0 * dy[i];
    corr_same_kernel_grad(tmp, x, h, w, k, g);   /* dW0 = s0 * sum dy * x(shift) */
    g[kk] += p->s0 * sdy;                        /* db0 */
    g[kk + 1] += sdyz;                           /* ds0 */
    if (L == 0) return;

    /* forward quantities the level parameters multiply */
    plane_analysis(p, h, w, x, a, zc);

    /* gradient at every Z_l (same reverse cascade as the data part) */
    const double *dr = dy;
    for (int l = 1; l <= L; l++) {
        int64_t hl = lvl_dim(h, l), wl = lvl_dim(w, l);
        double *dzl = dz + level_offset(h, w, l);
        haar_synthesis_adjoint(dr, hl, wl, lvl_dim(h, l - 1), lvl_dim(w, l - 1), dzl);
        dr = dzl;
    }

    /* Z = s * Zc:  ds = sum dZ * Zc;  dW = sum (s dZ) * A(shift) */
    double *gw = g + kk + 2, *gs = g + kk + 2 + (int64_t)L * 4 * kk;
    for (int l = 1; l <= L; l++) {
        int64_t hl = lvl_dim(h, l), wl = lvl_dim(w, l), m = hl * wl;
        double *al = a + level_offset(h, w, l);
        double *zl = zc + level_offset(h, w, l);
        double *dzl = dz + level_offset(h, w, l);
        for (int b = 0; b < 4; b++) {
            double s = p->sl[l - 1][b], acc = 0.0;
            for (int64_t i = 0; i < m; i++) {
                acc += dzl[b * m + i] * zl[b * m + i];
                tmp[i] = s * dzl[b * m + i];
            }
            gs[(l - 1) * 4 + b] += acc;
            corr_same_kernel_grad(tmp, al + b * m, hl, wl, k, gw + ((int64_t)(l - 1) * 4 + b) * kk);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Drivers over N x C planes, with plain threads over planes                  */
/* ------------------------------------------------------------------------ */

typedef struct {
    int op; /* 0 forward, 1 backward data, 2 backward weight */
    int64_t n, c, h, w;
    int k, levels;
    const double *x, *dy, *w_base, *bias, *s_base, *w_lvl, *s_lvl;
    double *out;      /* y or dx */
    double *partial;  /* per-plane parameter gradients [N*C][P] */
    int64_t plen;
    int tid, nthreads;
    int failed;
} job_t;

static void *run_planes(void *arg)
{
    job_t *j = (job_t *)arg;
    int64_t hw = j->h * j->w, pyr = pyramid_elems(j->h, j->w, j->levels);
    double *scratch = (double *)malloc((size_t)(3 * pyr + 3 * hw + 16) * sizeof(double));
    if (!scratch) {
        j->failed = 1;
        return NULL;
    }
    for (int64_t pl = j->tid; pl < j->n * j->c; pl += j->nthreads) {
        int64_t c = pl % j->c;
        chan_params p;
        gather_params(&p, j->c, c, j->k, j->levels, j->w_base, j->bias, j->s_base, j->w_lvl, j->s_lvl);
        if (j->op == 0) {
            plane_forward(&p, j->h, j->w, j->x + pl * hw, j->out + pl * hw, scratch);
        } else if (j->op == 1) {
            plane_backward_data(&p, j->h, j->w, j->dy + pl * hw, j->out + pl * hw, scratch);
        } else {
            double *g = j->partial + pl * j->plen;
            memset(g, 0, (size_t)j->plen * sizeof(double));
            plane_backward_weight(&p, j->h, j->w, j->x + pl * hw, j->dy + pl * hw, g, scratch);
        }
    }
    free(scratch);
    return NULL;
}

static int check_args(int64_t n, int64_t c, int64_t h, int64_t w, int k, int levels)
{
    if (n < 0 || c < 0 || h < 0 || w < 0) return -1;
    if (k < 1 || (k % 2) == 0 || levels < 0 || levels > 15) return -1;
    return 0;
}

static int run_all(job_t *proto, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    job_t jobs[256];
    pthread_t th[256];
    int started[256] = {0};
    for (int t = 0; t < nthreads; t++) {
        jobs[t] = *proto;
        jobs[t].tid = t;
        jobs[t].nthreads = nthreads;
        jobs[t].failed = 0;
    }
    if (nthreads == 1) {
        run_planes(&jobs[0]);
        return jobs[0].failed ? -2 : 0;
    }
    for (int t = 0; t < nthreads; t++) started[t] = pthread_create(&th[t], NULL, run_planes, &jobs[t]) == 0;
    int failed = 0;
    for (int t = 0; t < nthreads; t++) {
        if (started[t])
            pthread_join(th[t], NULL);
        else
            run_planes(&jobs[t]); /* could not start a thread: do its share here */
        failed |= jobs[t].failed;
    }
    return failed ? -2 : 0;
}

/* y = WTConv(x).  All arrays double, NCHW. */
int oracle_wtconv_forward(int64_t n, int64_t c, int64_t h, int64_t w, int k, int levels, const double *x,
                          const double *w_base, const double *bias, const double *s_base, const double *w_lvl,
                          const double *s_lvl, double *y, int nthreads)
{
    if (check_args(n, c, h, w, k, levels) || !x || !w_base || !s_base || !y) return -1;
    if (levels > 0 && (!w_lvl || !s_lvl)) return -1;
    job_t j = {0};
    j.op = 0; j.n = n; j.c = c; j.h = h; j.w = w; j.k = k; j.levels = levels;
    j.x = x; j.w_base = w_base; j.bias = bias; j.s_base = s_base; j.w_lvl = w_lvl; j.s_lvl = s_lvl;
    j.out = y;
    return run_all(&j, nthreads);
}

/* dx = gradient of <dy, WTConv(x)> with respect to x. */
int oracle_wtconv_backward_data(int64_t n, int64_t c, int64_t h, int64_t w, int k, int levels, const double *dy,
                                const double *w_base, const double *s_base, const double *w_lvl,
                                const double *s_lvl, double *dx, int nthreads)
{
    if (check_args(n, c, h, w, k, levels) || !dy || !w_base || !s_base || !dx) return -1;
    if (levels > 0 && (!w_lvl || !s_lvl)) return -1;
    job_t j = {0};
    j.op = 1; j.n = n; j.c = c; j.h = h; j.w = w; j.k = k; j.levels = levels;
    j.dy = dy; j.w_base = w_base; j.s_base = s_base; j.w_lvl = w_lvl; j.s_lvl = s_lvl;
    j.out = dx;
    return run_all(&j, nthreads);
}

/* Gradients of <dy, WTConv(x)> with respect to every parameter.  Outputs are
 * overwritten: dw_base [C][k][k], dbias [C], ds_base [C], dw_lvl [L][4C][k][k],
 * ds_lvl [L][4C].  Per channel, the plane contributions are summed over n in
 * ascending order, so the result does not depend on the thread count. */
int oracle_wtconv_backward_weight(int64_t n, int64_t c, int64_t h, int64_t w, int k, int levels, const double *x,
                                  const double *dy, const double *w_base, const double *bias, const double *s_base,
                                  const double *w_lvl, const double *s_lvl, double *dw_base, double *dbias,
                                  double *ds_base, double *dw_lvl, double *ds_lvl, int nthreads)
{
    if (check_args(n, c, h, w, k, levels) || !x || !dy || !w_base || !s_base) return -1;
    if (!dw_base || !dbias || !ds_base) return -1;
    if (levels > 0 && (!w_lvl || !s_lvl || !dw_lvl || !ds_lvl)) return -1;
    int64_t kk = (int64_t)k * k, plen = kk + 2 + (int64_t)levels * 4 * (kk + 1);
    double *partial = (double *)malloc((size_t)(n * c * plen + 1) * sizeof(double));
    if (!partial) return -2;
    job_t j = {0};
    j.op = 2; j.n = n; j.c = c; j.h = h; j.w = w; j.k = k; j.levels = levels;
    j.x = x; j.dy = dy; j.w_base = w_base; j.bias = bias; j.s_base = s_base; j.w_lvl = w_lvl; j.s_lvl = s_lvl;
    j.partial = partial; j.plen = plen;
    int rc = run_all(&j, nthreads);
    if (rc == 0) {
        for (int64_t ch = 0; ch < c; ch++) {
            double *gsum = (double *)calloc((size_t)plen, sizeof(double));
            if (!gsum) { rc = -2; break; }
            for (int64_t nn = 0; nn < n; nn++) {
                const double *g = partial + (nn * c + ch) * plen;
                for (int64_t i = 0; i < plen; i++) gsum[i] += g[i];
            }
            for (int64_t i = 0; i < kk; i++) dw_base[ch * kk + i] = gsum[i];
            dbias[ch] = gsum[kk];
            ds_base[ch] = gsum[kk + 1];
            for (int l = 0; l < levels; l++) {
                for (int b = 0; b < 4; b++) {
                    const double *gw = gsum + kk + 2 + ((int64_t)l * 4 + b) * kk;
                    double *dst = dw_lvl + ((int64_t)l * 4 * c + 4 * ch + b) * kk;
                    for (int64_t i = 0; i < kk; i++) dst[i] = gw[i];
                    ds_lvl[(int64_t)l * 4 * c + 4 * ch + b] = gsum[kk + 2 + (int64_t)levels * 4 * kk + l * 4 + b];
                }
            }
            free(gsum);
        }
    }
    free(partial);
    return rc;
}

/* The scaled per-level band outputs Z_l^b = s_l^b * (W_l^b (*) A_l^b) of one
 * plane, for l = 1..L and b = 0..3, written one after another (level 1 band 0
 * first; each map ceil(h/2^l) x ceil(w/2^l)).  wl: [L][4][k][k] and sl: [L][4] of this
 * channel.  Lets a test evaluate the closed-form synthesis on the oracle's own
 * band outputs. */
int oracle_wtconv_level_outputs(int64_t h, int64_t w, int k, int levels, const double *x, const double *wl,
                                const double *sl, double *z)
{
    if (check_args(1, 1, h, w, k, levels) || levels < 1 || !x || !wl || !sl || !z) return -1;
    chan_params p;
    double w0dummy = 0.0;
    memset(&p, 0, sizeof(p));
    p.k = k;
    p.levels = levels;
    p.w0 = &w0dummy;
    for (int l = 0; l < levels; l++) {
        p.wl[l] = wl + (int64_t)l * 4 * k * k;
        for (int b = 0; b < 4; b++) p.sl[l][b] = sl[l * 4 + b];
    }
    int64_t pyr = pyramid_elems(h, w, levels);
    double *a = (double *)malloc((size_t)(pyr + 1) * sizeof(double));
    if (!a) return -2;
    plane_analysis(&p, h, w, x, a, z);
    for (int l = 1; l <= levels; l++) {
        int64_t m = map_elems(h, w, l);
        double *zl = z + level_offset(h, w, l);
        for (int b = 0; b < 4; b++)
            for (int64_t i = 0; i < m; i++) zl[b * m + i] *= p.sl[l - 1][b];
    }
    free(a);
    return 0;
}

/* Exported single-level Haar steps (for the perfect-reconstruction checks). */
int oracle_haar_analysis(const double *in, int64_t h, int64_t w, double *bands)
{
    if (!in || !bands || h < 2 || w < 2 || (h % 2) || (w % 2)) return -1;
    haar_analysis(in, h, w, bands);
    return 0;
}

int oracle_haar_synthesis(const double *bands, int64_t h2, int64_t w2, double *out)
{
    if (!bands || !out || h2 < 1 || w2 < 1) return -1;
    haar_synthesis(bands, h2, w2, 2 * h2, 2 * w2, out);
    return 0;
}

/* Exported single-map depthwise cross-correlation (zero 'same' padding). */
int oracle_corr_same(const double *in, int64_t h, int64_t w, const double *kern, int k, double *out)
{
    if (!in || !kern || !out || h < 1 || w < 1 || k < 1 || (k % 2) == 0) return -1;
    corr_same(in, h, w, kern, k, out);
    return 0;
}
