// wtconv_bwd.hip -- the fused single-pass backward kernel for gfx950 (plans
// and phases in wtconv_bwd_body.h, wtconv_whole_body.h, wtconv_wgrad_body.h).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wtconv_bwd_body.h"
#include "wtconv_launch.h"

static __device__ __forceinline__ void wtc_lds_barrier_bw() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename T, int K, int BW, int Q>
__global__ __launch_bounds__(512) void wtconv_bwd_kernel(WtcBwdArgs<T> A)
{
    extern __shared__ float wtc_lds[];
    const WtcWholeArgs<T> &ad = A.d;
    const WtcWgradArgs<T> &ag = A.g;
    WtcWholeCtx<T> cw;
    WtcWgradCtx<T, 4> cg;
    cw.lds = cg.lds = wtc_lds;
    cw.tid = cg.tid = threadIdx.x;
    cw.nth = cg.nth = blockDim.x;
    wtc_whole_setup<T>(ad, cw, blockIdx.x);
    wtc_wgrad_setup<T, 4>(ag, cg, blockIdx.x);
    // one staging group per thread for both plans: the data plan's (lane
    // quads hold 2 x 2 blocks of groups where it builds level 3 by DPP)
    cg.grow = cw.grow;
    cg.gcol = cw.gcol;
    cg.gvalid = cw.gvalid;
    wtc_wgrad_load<T, 4, false>(ag, cg, 0);
    for (int i = cw.tid; i < A.lds_floats; i += cw.nth) wtc_lds[i] = 0.0f;
    wtc_lds_barrier_bw();
    wtc_whole_fold<T, K>(ad, cw);
    wtc_whole_table<T, K, BW>(ad, cw);
    wtc_wgrad_table<T, K, 4>(ag, cg);
    float acc[Q][K * K + 1];
#pragma unroll
    for (int s = 0; s < Q; ++s)
#pragma unroll
        for (int e = 0; e < K * K + 1; ++e) acc[s][e] = 0.0f;
    wtc_wgrad_stage<T, K, 4, false>(ag, cg);
    wtc_bwd_stage_dy<T, K, BW>(ad, cw, cg);
    wtc_lds_barrier_bw();
    if (cw.nimg > 1) wtc_wgrad_load<T, 4, false>(ag, cg, 1);
    for (int img = 0; img < cw.nimg; ++img) {
        for (int m = ag.p.first_deep; m <= ag.p.levels; ++m) {
            wtc_wgrad_analysis<T, K, 4>(ag, cg, m);
            wtc_lds_barrier_bw();
        }
        for (int m = wtc_whole_first_deep(ad.p); m <= ad.p.levels; ++m) {
            wtc_whole_analysis<T, K>(ad, cw, m);
            wtc_lds_barrier_bw();
        }
        // the correlation and the convolution only read the pyramids: one
        // barrier interval for both, at the low wave priority
        __builtin_amdgcn_s_setprio(0);
        wtc_wgrad_correlate<T, K, 4, Q>(ag, cg, acc);
        wtc_whole_conv<T, K, BW>(ad, cw);
        wtc_lds_barrier_bw();
        __builtin_amdgcn_s_setprio(2);
        // the next image is staged while this one's dx is written (the output
        // pass reads only the convolution outputs)
        if (img + 1 < cw.nimg) {
            wtc_wgrad_stage<T, K, 4, false>(ag, cg);
            wtc_bwd_stage_dy<T, K, BW>(ad, cw, cg);
        }
        if (img + 2 < cw.nimg) wtc_wgrad_load<T, 4, false>(ag, cg, img + 2);
        wtc_whole_select<T, false>(ad, cw, img);
        wtc_whole_out<T, K, BW, false, false>(ad, cw);
        wtc_lds_barrier_bw();
    }
#pragma unroll
    for (int s = 0; s < Q; ++s) {
        if (s < ag.p.q) {
            wtc_wgrad_park<T, K, 4>(ag, cg, acc[s]);
            wtc_lds_barrier_bw();
            wtc_wgrad_chunks<T, K, 4>(ag, cg, s);
            wtc_lds_barrier_bw();
            wtc_wgrad_combine<T, K, 4>(ag, cg, s);
            wtc_lds_barrier_bw();
        }
    }
    wtc_wgrad_write<T, K, 4>(ag, cg);
}

template <typename T, int K, int Q>
static hipError_t launch_q(const WtcBwdArgs<T> &a, hipStream_t stream, int *resident)
{
    const size_t lds = (size_t)a.lds_floats * sizeof(float);
    const void *fn = (const void *)&wtconv_bwd_kernel<T, K, 4, Q>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (resident) {
        *resident = wtc_resident_blocks(fn, a.d.p.nthreads, lds);
        return hipSuccess;
    }
    const unsigned blocks = (unsigned)(a.g.p.groups * a.g.p.c);
    hipLaunchKernelGGL((wtconv_bwd_kernel<T, K, 4, Q>), dim3(blocks), dim3(a.d.p.nthreads), lds, stream, a);
    return hipGetLastError();
}

template <typename T, int K>
static hipError_t launch_k(const WtcBwdArgs<T> &a, hipStream_t stream, int *resident)
{
    if (a.d.p.out_bw != 4 || a.g.p.vec != 4) return hipErrorInvalidValue;
    return a.g.p.q == 1 ? launch_q<T, K, 1>(a, stream, resident)
                        : launch_q<T, K, WTC_WG_QMAX>(a, stream, resident);
}

template <typename T>
static hipError_t launch_t(const WtcBwdArgs<T> &a, hipStream_t stream, int *resident = nullptr)
{
    switch (a.d.p.k) {
    case 1: return launch_k<T, 1>(a, stream, resident);
    case 3: return launch_k<T, 3>(a, stream, resident);
    case 5: return launch_k<T, 5>(a, stream, resident);
    case 7: return launch_k<T, 7>(a, stream, resident);
    default: return hipErrorInvalidValue;
    }
}

hipError_t wtc_launch_bwd(int dtype, const WtcBwdPlan &p, const void *x, const void *dy, void *dx,
                          const float *w_base, const float *s_base, const float *w_lvl, const float *s_lvl,
                          float *partial, hipStream_t stream)
{
    if (dtype == 0)
        return launch_t<float>(wtc_bwd_args<float>(p, (const float *)x, (const float *)dy, (float *)dx, w_base, s_base,
                                                    w_lvl, s_lvl, partial),
                               stream);
    return launch_t<_Float16>(wtc_bwd_args<_Float16>(p, (const _Float16 *)x, (const _Float16 *)dy, (_Float16 *)dx,
                                                     w_base, s_base, w_lvl, s_lvl, partial),
                              stream);
}

int wtc_bwd_resident(int dtype, const WtcBwdPlan &p)
{
    int r = 0;
    hipError_t e;
    if (dtype == 0)
        e = launch_t<float>(
            wtc_bwd_args<float>(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), nullptr,
            &r);
    else
        e = launch_t<_Float16>(
            wtc_bwd_args<_Float16>(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), nullptr,
            &r);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return r;
}
