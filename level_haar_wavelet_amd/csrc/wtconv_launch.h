// wtconv_launch.h -- host-side launch entry points of the kernel files, used by
// the C ABI in wtconv_api.hip.
#ifndef WTCONV_LAUNCH_H
#define WTCONV_LAUNCH_H

#include <hip/hip_runtime.h>

#include "wtconv_bwd_body.h"
#include "wtconv_large_body.h"
#include "wtconv_plan.h"
#include "wtconv_whole_body.h"
#include "wtconv_wgrad_body.h"
#include "wtconv_wgrad_tile_body.h"

// Fused forward (rotate = 0) or data backward (rotate = 1), per plan p.
hipError_t wtc_launch_fused(int dtype, const WtcFusedPlan &p, const void *in, void *out, const float *w_base,
                            const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
                            hipStream_t stream);

// Whole-plane fused forward / data backward, per plan p; for a tiled plan,
// `low` is the deeper levels' low-pass term at level-1 resolution, fp32 (or
// null).
hipError_t wtc_launch_whole(int dtype, const WtcWholePlan &p, const void *in, void *out, const float *w_base,
                            const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
                            hipStream_t stream, const void *low = nullptr);

// Fused large-plane forward / data backward (every level on chip), per plan p.
hipError_t wtc_launch_large(int dtype, const WtcLargePlan &p, const void *in, void *out, const float *w_base,
                            const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
                            hipStream_t stream);

// Fused single-pass backward (dx and the weight-gradient partial rows), per
// plan p; the weight backward's finalize pass reduces the partials.
hipError_t wtc_launch_bwd(int dtype, const WtcBwdPlan &p, const void *x, const void *dy, void *dx,
                          const float *w_base, const float *s_base, const float *w_lvl, const float *s_lvl,
                          float *partial, hipStream_t stream);

// Level-1 low-pass band (orthonormal, (a + b + c + d) / 2 of every 2x2 block)
// of `planes` planes of h x w (multiples of 4) of the input dtype, into fp32
// planes of (h/2) x (w/2).
hipError_t wtc_launch_lowpass(int dtype, const void *in, float *out, int64_t planes, int h, int w,
                              hipStream_t stream);

// n floats set to v (a kernel, so that callers may capture it in a graph).
hipError_t wtc_launch_fill(float *p, int64_t n, float v, hipStream_t stream);

// The hout x wout window of each of `planes` planes of hin x win: zero-padded
// (at the bottom and right) or cropped copy.
hipError_t wtc_launch_repack(int dtype, const void *in, void *out, int64_t planes, int hin, int win, int hout,
                             int wout, hipStream_t stream);

// Fused parameter-gradient correlations (partials per workgroup) and the
// fixed-order reduction with the chain rule.  Tiled plans may also write the
// level-1 low-pass maps of x and dy (llx, lld: (N, C, ih/2, iw/2) fp32, both or
// neither).
hipError_t wtc_launch_wgrad(int dtype, const WtcWgradPlan &p, const void *x, const void *dy, float *partial,
                            hipStream_t stream, void *llx = nullptr, void *lld = nullptr);
hipError_t wtc_launch_wgrad_finalize(int C, int k, int levels, int groups, int plen, const float *partial,
                                     const float *w_base, const float *bias, const float *s_base,
                                     const float *w_lvl, const float *s_lvl, float *dw_base, float *dbias,
                                     float *ds_base, float *dw_lvl, float *ds_lvl, hipStream_t stream);

// Several partial-row sets finalized by one launch (a tiled weight backward
// and its nested calls: every set is the chain rule of its own levels into its
// own outputs).
#define WTC_FIN_MAX 8
struct WtcFinalizeSet {
    int levels, groups, plen;
    const float *partial, *w_base, *bias, *s_base, *w_lvl, *s_lvl;
    float *dw_base, *dbias, *ds_base, *dw_lvl, *ds_lvl;
};
struct WtcFinalizeSets {
    int C, k, n;
    WtcFinalizeSet s[WTC_FIN_MAX];
};
hipError_t wtc_launch_wgrad_finalize_sets(const WtcFinalizeSets &f, hipStream_t stream);

// Step `p.step` of the level-by-level tiled parameter gradient (input dtype:
// 0 fp32, 1 fp16; steps after the first read the fp32 maps of the previous).
hipError_t wtc_launch_wgrad_tile(int in_dtype, const WtcWtilePlan &p, const void *x, const void *dy, float *ux,
                                 float *ud, float *partial, hipStream_t stream);

// Workgroups of a kernel (nthreads threads, lds bytes of dynamic LDS) that
// the current device holds at once: resident per compute unit x compute
// units; 0 when HIP cannot tell.  Cached per device and configuration.
int wtc_resident_blocks(const void *fn, int nthreads, size_t lds);

// Resident workgroups of the whole-plane and weight-gradient kernels for a plan.
int wtc_whole_resident(int dtype, const WtcWholePlan &p);
int wtc_large_resident(int dtype, const WtcLargePlan &p);
int wtc_bwd_resident(int dtype, const WtcBwdPlan &p);
int wtc_wgrad_resident(int dtype, const WtcWgradPlan &p);

#endif  // WTCONV_LAUNCH_H
