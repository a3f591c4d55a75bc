// wtconv_fused.hip -- the fused WTConv forward / data-backward kernel for gfx950.
//
// One workgroup per (plane, tile).  The phases and the arithmetic are in
// wtconv_fused_body.h; this file strings them together with workgroup barriers
// and instantiates them for the supported (activation type, kernel size,
// output block width) triples.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wtconv_fused_body.h"
#include "wtconv_launch.h"

template <typename T, int K, int BW>
__global__ __launch_bounds__(256) void wtconv_fused_kernel(WtcFusedArgs<T> a)
{
    extern __shared__ float wtc_lds[];
    WtcCtx<T> ctx;
    ctx.lds = wtc_lds;
    ctx.tid = threadIdx.x;
    ctx.nth = blockDim.x;
    wtc_fused_setup<T>(a, ctx, blockIdx.x, gridDim.x);

    wtc_phase_fold<T, K>(a, ctx);
    wtc_phase_coarse<T, K>(a, ctx);
    __syncthreads();
    for (int m = 2; m <= a.p.levels; ++m) {
        wtc_phase_deep_level<T, K>(a, ctx, m);
        __syncthreads();
    }
    // The deep convolution outputs are first read by the output phase of the
    // first strip, two barriers later; the strip staging writes other maps.
    wtc_phase_deep_conv<T, K>(a, ctx);
    for (int s0 = ctx.ty0; s0 < ctx.ty0 + a.p.tile_h; s0 += a.p.strip_h) {
        wtc_phase_stage<T, K>(a, ctx, s0);
        __syncthreads();
        wtc_phase_strip_bands<T, K>(a, ctx, s0);
        __syncthreads();
        wtc_phase_strip_conv1<T, K>(a, ctx, s0);
        __syncthreads();
        wtc_phase_strip_out<T, K, BW>(a, ctx, s0);
        __syncthreads();
    }
}

template <typename T, int K, int BW>
static hipError_t launch_fused_bw(const WtcFusedArgs<T> &a, hipStream_t stream)
{
    const size_t lds = (size_t)a.p.lds_floats * sizeof(float);
    const void *fn = (const void *)&wtconv_fused_kernel<T, K, BW>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const unsigned blocks = (unsigned)((int64_t)a.p.n * a.p.c * a.p.tiles_y * a.p.tiles_x);
    hipLaunchKernelGGL((wtconv_fused_kernel<T, K, BW>), dim3(blocks), dim3(a.p.nthreads), lds, stream, a);
    return hipGetLastError();
}

template <typename T, int K>
static hipError_t launch_fused_k(const WtcFusedArgs<T> &a, hipStream_t stream)
{
    switch (a.p.out_bw) {
    case 8: return launch_fused_bw<T, K, 8>(a, stream);
    case 4: return launch_fused_bw<T, K, 4>(a, stream);
    default: return launch_fused_bw<T, K, 2>(a, stream);
    }
}

template <typename T>
static hipError_t launch_fused_t(const WtcFusedArgs<T> &a, hipStream_t stream)
{
    switch (a.p.k) {
    case 1: return launch_fused_k<T, 1>(a, stream);
    case 3: return launch_fused_k<T, 3>(a, stream);
    case 5: return launch_fused_k<T, 5>(a, stream);
    case 7: return launch_fused_k<T, 7>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t wtc_launch_fused(int dtype, const WtcFusedPlan &p, const void *in, void *out, const float *w_base,
                            const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
                            hipStream_t stream)
{
    if (dtype == 0) {
        WtcFusedArgs<float> a{(const float *)in, (float *)out, w_base, bias, s_base, w_lvl, s_lvl, p};
        return launch_fused_t<float>(a, stream);
    }
    WtcFusedArgs<_Float16> a{(const _Float16 *)in, (_Float16 *)out, w_base, bias, s_base, w_lvl, s_lvl, p};
    return launch_fused_t<_Float16>(a, stream);
}
