// wtconv_wgrad_tile.hip -- level-by-level tiled parameter-gradient kernel for
// planes too large for the whole-plane kernel (phases in
// wtconv_wgrad_tile_body.h).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wtconv_launch.h"
#include "wtconv_wgrad_tile_body.h"

static __device__ __forceinline__ void wtc_lds_barrier_wt() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <typename TI, int K>
__global__ __launch_bounds__(256) void wtconv_wgrad_tile_kernel(WtcWtileArgs<TI> a)
{
    extern __shared__ float wtc_lds[];
    WtcWtileCtx ctx;
    ctx.lds = wtc_lds;
    ctx.tid = threadIdx.x;
    ctx.nth = blockDim.x;
    ctx.c = blockIdx.x % a.p.c;
    ctx.group = blockIdx.x / a.p.c;
    const int units = a.p.n * a.p.tiles_y * a.p.tiles_x;
    const int u0 = ctx.group * a.p.units_per_wg, u1 = min(units, u0 + a.p.units_per_wg);
    const bool next = a.p.step < a.p.levels;
    wtc_wtile_zero<TI>(a, ctx);
    wtc_lds_barrier_wt();
    wtc_wtile_table<TI, K>(a, ctx);
    float acc[WTC_WT_QMAX][K * K + 1];
#pragma unroll
    for (int s = 0; s < WTC_WT_QMAX; ++s)
#pragma unroll
        for (int e = 0; e < K * K + 1; ++e) acc[s][e] = 0.0f;
    for (int u = u0; u < u1; ++u) {
        wtc_wtile_stage<TI, K>(a, ctx, u);
        wtc_lds_barrier_wt();
        if (next) {
            wtc_wtile_analysis<TI, K>(a, ctx, u);
            wtc_lds_barrier_wt();
        }
        wtc_wtile_correlate<TI, K>(a, ctx, acc);
        wtc_lds_barrier_wt();
    }
#pragma unroll
    for (int s = 0; s < WTC_WT_QMAX; ++s) {
        if (s < a.p.q) {
            wtc_wtile_park<TI, K>(a, ctx, acc[s]);
            wtc_lds_barrier_wt();
            wtc_wtile_gather<TI, K>(a, ctx, s);
            wtc_lds_barrier_wt();
        }
    }
    wtc_wtile_write<TI, K>(a, ctx);
}

template <typename TI, int K>
static hipError_t launch_wtile(const WtcWtileArgs<TI> &a, hipStream_t stream)
{
    const size_t lds = (size_t)a.p.lds_floats * sizeof(float);
    const void *fn = (const void *)&wtconv_wgrad_tile_kernel<TI, K>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const unsigned blocks = (unsigned)(a.p.groups * a.p.c);
    hipLaunchKernelGGL((wtconv_wgrad_tile_kernel<TI, K>), dim3(blocks), dim3(a.p.nthreads), lds, stream, a);
    return hipGetLastError();
}

template <typename TI>
static hipError_t launch_wtile_t(const WtcWtileArgs<TI> &a, hipStream_t stream)
{
    switch (a.p.k) {
    case 1: return launch_wtile<TI, 1>(a, stream);
    case 3: return launch_wtile<TI, 3>(a, stream);
    case 5: return launch_wtile<TI, 5>(a, stream);
    case 7: return launch_wtile<TI, 7>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t wtc_launch_wgrad_tile(int in_dtype, const WtcWtilePlan &p, const void *x, const void *dy, float *ux,
                                 float *ud, float *partial, hipStream_t stream)
{
    if (in_dtype == 0) {
        WtcWtileArgs<float> a{(const float *)x, (const float *)dy, ux, ud, partial, p};
        return launch_wtile_t<float>(a, stream);
    }
    WtcWtileArgs<_Float16> a{(const _Float16 *)x, (const _Float16 *)dy, ux, ud, partial, p};
    return launch_wtile_t<_Float16>(a, stream);
}
