// wtconv_large_body.h -- the fused forward / data backward for planes too
// large for one workgroup whose level-1 low-pass map still fits one ("large
// planes": the 128 x 128 maps of the level sweep).  Every level stays on chip:
// nothing but the input is read and nothing but the output is written.
//
// Source: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation" (arXiv 2608.10805), technical summary, Methodology: the Haar
// analysis is recomputed on chip instead of storing the subbands
// (reformulation 1), and the multi-level synthesis is one closed-form pass
// (reformulation 2), which removes the stored intermediate low-pass tensors.
//
// The orthonormal Haar pyramid splits the layer exactly: levels 2..L of the
// layer on x are the layer with L - 1 levels, without base path, on the
// level-1 low-pass map LL_1(x) = (a + b + c + d) / 2, and their output enters
// level 1's synthesis as the low-pass input.  A workgroup owns one channel and
// P images of it; per image it runs two plans that share its LDS:
//   D ("deeper levels"): the whole-plane plan on the (h/2) x (w/2) map with
//     L - 1 levels and no base path, staged straight from x -- each thread
//     loads the 8 x 8 input block under its 4 x 4 group of LL_1 and reduces it
//     in registers -- whose output pass writes the deeper levels' term to an
//     fp32 map in LDS instead of storing it;
//   T ("tiles"): the tiled plan of the base and level-1 convolutions on
//     th x tw tiles with halos, which re-reads x (the lines D just brought into
//     the L2 cache) and adds the term from LDS before level 1's butterfly.
// The two plans' maps alias one LDS region (D's are zeroed again before every
// image; T's staging writes every element T reads); the folded weights and
// piece tables of both plans and the term map live outside it.
// Without the base path (nobase: the nested deeper-levels call of a plane too
// large even for this kernel) T has no base pieces and its output pass reads
// the base output from one zero row, which lives outside the aliased region
// too (D's maps overwrite that region every image).
#ifndef WTCONV_LARGE_BODY_H
#define WTCONV_LARGE_BODY_H

#include "wtconv_whole_body.h"

struct WtcLargePlan {
    WtcWholePlan d;     // deeper levels: (h/2) x (w/2), L - 1 levels, no base path
    WtcWholePlan t;     // base and level 1 on th x tw tiles of h x w
    int32_t n, c, h, w, k, levels, rotate, nthreads;
    int32_t planes;     // images per workgroup
    int32_t nobase;     // no base path (w_base, bias, s_base not read)
    int32_t maps_off;   // the aliased map region [maps_off, maps_off + maps_floats)
    int32_t dmaps_floats, maps_floats;
    int32_t lds_floats;
};

// Moves a plan's maps to start at `maps_to` and its folded weights and piece
// table to `wf_to` and `tab_to` (the layout puts the weights first, then the
// maps, then the table).
static inline void wtc_relocate(WtcWholePlan *p, int32_t maps_to, int32_t wf_to, int32_t tab_to)
{
    const int32_t first = (1 + 4 * p->levels) * p->ws;
    const int32_t delta = maps_to - first;
    p->x.off += delta;
    for (int32_t m = 0; m <= WTC_MAXL; ++m) {
        p->u[m].off += delta;
        p->z[m].off += delta;
    }
    p->wf_off = wf_to;
    p->tab_off = tab_to;
}

static inline int32_t wtc_maps_floats(const WtcWholePlan *p) { return p->tab_off - (1 + 4 * p->levels) * p->ws; }

// Plan of the fused large-plane pass on th x tw tiles, or -1 when it does not
// apply or fit: L >= 2, the level-1 map fits one 256-thread workgroup as 4 x 4
// staging groups, both plans use 4-wide output blocks, and the LDS holds both
// plans' tables and weights, the term map and the larger plan's maps.
static inline int wtc_make_large_plan(WtcLargePlan *lp, int32_t n, int32_t c, int32_t h, int32_t w, int32_t th,
                                      int32_t tw, int32_t k, int32_t levels, int32_t rotate, int32_t nthreads,
                                      int32_t planes, int32_t elem_bytes, int32_t budget_floats,
                                      int32_t nobase = 0)
{
    if (levels < 2 || h % 8 || w % 8 || (th >= h && tw >= w)) return -1;
    if (h % th || w % tw) return -1;
    const int32_t tiles = (h / th) * (w / tw);
    lp->n = n;
    lp->c = c;
    lp->h = h;
    lp->w = w;
    lp->k = k;
    lp->levels = levels;
    lp->rotate = rotate;
    lp->nthreads = nthreads;
    lp->planes = planes < 1 ? 1 : (planes > n ? n : planes);
    lp->nobase = nobase ? 1 : 0;
    WtcWholePlan &d = lp->d, &t = lp->t;
    // the deeper levels: staged from registers in 4 x 4 groups of the
    // level-1 map (fp32 values, whatever the activation type)
    if (wtc_make_whole_plan(&d, n, c, h / 2, w / 2, k, levels - 1, rotate, nthreads, lp->planes, 4, 1 << 30, 1))
        return -1;
    if (d.gr != 4 || d.vec != 4 || d.groups != (h / 8) * (w / 8) || d.out_bw != 4) return -1;
    // its pieces past the first round stay whole: one-row pieces there (the
    // second workgroup on the compute unit keeps the SIMDs busy meanwhile)
    // measured no faster at L = 3 and slower at L = 4 and 5
    d.tail = 0;
    if (wtc_make_whole_tile_plan(&t, n, c, h, w, th, tw, k, 1, rotate, nthreads, lp->planes * tiles, elem_bytes,
                                 1 << 30, lp->nobase))
        return -1;
    if (t.out_bw != 4 || t.planes != lp->planes * tiles) return -1;
    // persistent: D weights, T weights, D table, T table, the term map; then
    // the aliased maps
    int32_t off = 0;
    const int32_t dwf = off;
    off += (1 + 4 * d.levels) * d.ws;
    const int32_t twf = off;
    off += (1 + 4 * t.levels) * t.ws;
    const int32_t dtab = off;
    off += 4 * d.items;
    const int32_t ttab = off;
    off += 4 * t.items;
    off = wtc_roundup(off, 4);
    const int32_t deep = off, dpitch = w / 2;
    off += (h / 2) * dpitch;
    off = wtc_roundup(off, 4);
    // without the base path: the zero row T's output pass reads as its base
    // output (as wide as the row the tile plan reserved for it)
    const int32_t zrow = off;
    if (lp->nobase) off += wtc_roundup(wtc_pitch16(wtc_roundup(tw, WTC_WP)), 4);
    lp->maps_off = off;
    lp->dmaps_floats = wtc_roundup(wtc_maps_floats(&d), 4);
    lp->maps_floats = wtc_max(lp->dmaps_floats, wtc_roundup(wtc_maps_floats(&t), 4));
    wtc_relocate(&d, off, dwf, dtab);
    wtc_relocate(&t, off, twf, ttab);
    if (lp->nobase) t.z[0].off = zrow;
    d.deep_off = t.deep_off = deep;
    d.deep_pitch = t.deep_pitch = dpitch;
    lp->lds_floats = wtc_roundup(off + lp->maps_floats, 4);
    d.lds_floats = t.lds_floats = lp->lds_floats;
    return lp->lds_floats <= budget_floats ? 0 : -1;
}

// Kernel arguments: the two plans' views of the layer's arguments, built on
// the host and passed whole, so that the kernel reads plan fields (indexed by
// level at run time) from the argument segment rather than from a private
// copy.  The deeper levels take the level weights and scales from level 2 on
// (no base path, no output), the tiles the base and level 1.
template <typename T>
struct WtcLargeArgs {
    WtcWholeArgs<T> d, t;
    int32_t n, c, h, w;
    int32_t planes, maps_off, dmaps_floats, maps_floats, lds_floats;
};

template <typename T>
static inline WtcLargeArgs<T> wtc_large_args(const WtcLargePlan &lp, const T *in, T *out, const float *w_base,
                                            const float *bias, const float *s_base, const float *w_lvl,
                                            const float *s_lvl)
{
    const int64_t kk = (int64_t)lp.k * lp.k;
    WtcLargeArgs<T> a;
    a.d = WtcWholeArgs<T>{in, nullptr, nullptr, nullptr, nullptr, w_lvl ? w_lvl + 4 * lp.c * kk : nullptr,
                          s_lvl ? s_lvl + 4 * lp.c : nullptr, lp.d};
    a.t = WtcWholeArgs<T>{in, out, w_base, bias, s_base, w_lvl, s_lvl, lp.t};
    a.n = lp.n;
    a.c = lp.c;
    a.h = lp.h;
    a.w = lp.w;
    a.planes = lp.planes;
    a.maps_off = lp.maps_off;
    a.dmaps_floats = lp.dmaps_floats;
    a.maps_floats = lp.maps_floats;
    a.lds_floats = lp.lds_floats;
    return a;
}

// Zero the deeper-levels plan's maps (their zero borders are the
// convolutions' padding; the tiles wrote over them).
template <typename T>
WTC_HD WTC_INLINE void wtc_large_zero_d(const WtcLargeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    for (int i = 4 * ctx.tid; i < a.dmaps_floats; i += 4 * ctx.nth) {
        const float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        wtc_lds_put<4, 4>(ctx, a.maps_off + i, z);
    }
}

// The deeper levels' staging input of image `img` of the workgroup, in two
// steps so that the loads can be issued a phase ahead: wtc_large_fetch_d loads
// this thread's 8 x 8 block of x (the 4 x 4 group of the level-1 map it
// stages) as it is stored, wtc_large_reduce_d turns it into the orthonormal
// low-pass values (a + b + c + d) / 2.
template <typename T>
struct WtcLargeRaw {
    T v[8][8];
};

template <typename T>
WTC_HD WTC_INLINE void wtc_large_fetch_d(const WtcLargeArgs<T> &a, const WtcWholeCtx<T> &ctx, int img,
                                         WtcLargeRaw<T> &raw)
{
    const int64_t plane = (int64_t)(ctx.n0 + img) * a.c + ctx.c;
    const T *src = a.d.in + plane * ((int64_t)a.h * a.w);
    const int row0 = 8 * ctx.grow, col0 = 8 * ctx.gcol;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int64_t e = (int64_t)(row0 + r) * a.w + col0;
#ifdef WTC_EMULATE
        const int64_t base = src - a.d.in, all = (int64_t)a.n * a.c * a.h * a.w;
        for (int t = 0; t < 8; ++t) raw.v[r][t] = wtc_chk(a.d.in, base + e + t, all, __LINE__);
#else
        constexpr int PER = 16 / sizeof(T);  // elements per 16-byte load
#pragma unroll
        for (int s = 0; s < 8 / PER; ++s) {
            typedef float v4 __attribute__((ext_vector_type(4)));
            const v4 d = *(const v4 *)(src + e + s * PER);
            __builtin_memcpy(&raw.v[r][s * PER], &d, 16);
        }
#endif
    }
}

template <typename T>
WTC_HD WTC_INLINE void wtc_large_reduce_d(const WtcLargeRaw<T> &raw, float (&ll)[4][4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            ll[i][j] = 0.5f * ((wtc_to_float(raw.v[2 * i][2 * j]) + wtc_to_float(raw.v[2 * i][2 * j + 1])) +
                               (wtc_to_float(raw.v[2 * i + 1][2 * j]) + wtc_to_float(raw.v[2 * i + 1][2 * j + 1])));
}

#endif  // WTCONV_LARGE_BODY_H
