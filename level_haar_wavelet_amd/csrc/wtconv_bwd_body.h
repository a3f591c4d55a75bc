// wtconv_bwd_body.h -- the fused single-pass backward of the WTConv layer for
// planes that fit one workgroup: one pass reads x and dy once and writes dx and
// the parameter-gradient partials (5 E e bytes instead of the 6 E e of a data
// backward plus a weight backward).
//
// Source: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation" (arXiv 2608.10805), technical summary, Key Contributions:
// forward outputs and all parameter gradients of the layer; Methodology,
// reformulations 1-3 (on-chip Haar analysis, closed-form synthesis, scales
// folded into the weights).  Both halves of the backward analyse dy: the data
// backward convolves dy's pyramid with the kernels turned by 180 degrees
// (wtconv_whole_body.h, rotate = 1), the weight backward correlates it with
// x's pyramid (wtconv_wgrad_body.h).  A workgroup owns one channel and P images
// and runs both plans on one staging of every image:
//   * each thread loads its 4 x 4 group of x and of dy once; the weight plan's
//     staging writes x's bordered pyramid and dy's interior pyramid, the data
//     plan's staging writes dy's bordered pyramid (its convolution's input);
//   * the correlation (persistent per-thread accumulators) and the
//     convolution run in the same barrier interval, the output pass writes dx
//     while the next image is staged;
//   * after the last image the accumulators are reduced in a fixed order into
//     the workgroup's partial row (the weight backward's second pass applies
//     the chain rule).
// The two plans' LDS layouts are placed one after the other.
#ifndef WTCONV_BWD_BODY_H
#define WTCONV_BWD_BODY_H

#include "wtconv_wgrad_body.h"
#include "wtconv_whole_body.h"

struct WtcBwdPlan {
    WtcWholePlan d;  // data backward (rotate = 1): dy's bordered pyramid, convolution outputs, output pass
    WtcWgradPlan g;  // weight backward: x's bordered pyramid, dy's interior pyramid, correlation, reduction
    int32_t lds_floats;
};

static inline void wtc_wgrad_relocate(WtcWgradPlan *p, int32_t delta)
{
    p->x.off += delta;
    p->dy.off += delta;
    for (int32_t m = 0; m <= WTC_MAXL; ++m) {
        p->u[m].off += delta;
        p->d[m].off += delta;
    }
    p->tab_off += delta;
    p->red_off += delta;
    p->csum_off += delta;
    p->res_off += delta;
    p->ctab_off += delta;
}

// Plan of the fused backward, or -1: both plans whole-plane (untiled,
// unstacked), staging the same 4 x 4 groups (so one load of x and dy serves
// both), and both layouts within the budget.
static inline int wtc_make_bwd_plan(WtcBwdPlan *bp, int32_t n, int32_t c, int32_t h, int32_t w, int32_t k,
                                    int32_t levels, int32_t nthreads, int32_t planes, int32_t elem_bytes,
                                    int32_t budget_floats)
{
    WtcWholePlan &d = bp->d;
    WtcWgradPlan &g = bp->g;
    if (levels < 1) return -1;
    if (wtc_make_whole_plan(&d, n, c, h, w, k, levels, 1, nthreads, planes, elem_bytes, 1 << 30)) return -1;
    if (wtc_make_wgrad_plan(&g, n, c, h, w, k, levels, nthreads, planes, elem_bytes, 1 << 30)) return -1;
    if (d.tiled || d.stack != 1 || d.gr != 4 || d.vec != 4 || g.gr != 4 || g.vec != 4) return -1;
    if (d.groups != g.sgroups || d.planes != g.planes || d.out_bw != 4) return -1;
    // 16-byte aligned start of the weight plan's region
    const int32_t base = wtc_roundup(d.lds_floats, 4);
    if (g.lds_floats > 65535 - base) return -1;  // piece descriptors hold 16-bit LDS indexes
    wtc_wgrad_relocate(&g, base);
    bp->lds_floats = wtc_roundup(base + g.lds_floats, 4);
    g.lds_floats = d.lds_floats = bp->lds_floats;
    return bp->lds_floats <= budget_floats ? 0 : -1;
}

template <typename T>
struct WtcBwdArgs {
    WtcWholeArgs<T> d;  // in = dy, out = dx, the layer's weights (turned on chip), no bias
    WtcWgradArgs<T> g;  // x, dy, the partial rows
    int32_t lds_floats;
};

template <typename T>
static inline WtcBwdArgs<T> wtc_bwd_args(const WtcBwdPlan &bp, const T *x, const T *dy, T *dx, const float *w_base,
                                        const float *s_base, const float *w_lvl, const float *s_lvl, float *partial)
{
    WtcBwdArgs<T> a;
    a.d = WtcWholeArgs<T>{dy, dx, w_base, nullptr, s_base, w_lvl, s_lvl, bp.d};
    a.g = WtcWgradArgs<T>{x, dy, partial, bp.g};
    a.lds_floats = bp.lds_floats;
    return a;
}

// The data plan's staging of the group the weight plan's thread holds (its
// prefetched dy rows): dy's bordered map and bands, from the same registers.
template <typename T, int K, int BW>
WTC_HD WTC_INLINE void wtc_bwd_stage_dy(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &cw,
                                       const WtcWgradCtx<T, 4> &cg)
{
    float v[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < 4; ++t) v[q][t] = wtc_to_float(cg.prey[q][t]);
    wtc_whole_stage_vals<T, K, BW, false, false, true>(a, cw, v);  // the plan has 4-row groups
}

#endif  // WTCONV_BWD_BODY_H
