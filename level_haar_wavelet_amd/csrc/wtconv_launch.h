// wtconv_launch.h -- host-side launch entry points of the kernel files, used by
// the C ABI in wtconv_api.hip.
#ifndef WTCONV_LAUNCH_H
#define WTCONV_LAUNCH_H

#include <hip/hip_runtime.h>

#include "wtconv_plan.h"
#include "wtconv_whole_body.h"

// Fused forward (rotate = 0) or data backward (rotate = 1), per plan p.
hipError_t wtc_launch_fused(int dtype, const WtcFusedPlan &p, const void *in, void *out, const float *w_base,
                            const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
                            hipStream_t stream);

// Whole-plane fused forward / data backward, per plan p.
hipError_t wtc_launch_whole(int dtype, const WtcWholePlan &p, const void *in, void *out, const float *w_base,
                            const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
                            hipStream_t stream);

#endif  // WTCONV_LAUNCH_H
