// wtconv_whole.hip -- the whole-plane fused WTConv forward / data-backward
// kernel for gfx950 (phases in wtconv_whole_body.h).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wtconv_launch.h"
#include "wtconv_whole_body.h"

// Workgroup barrier that waits only for this wave's LDS operations: global
// loads issued before it (the next image's input) stay in flight.  The memory
// clobber keeps the compiler from moving LDS accesses across it.
static __device__ __forceinline__ void wtc_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ST: stacked small planes (two images per pass); a kernel instance of its
// own, so that the other plans carry none of its row checks.  G4: 4-row
// staging groups, which tiled and stacked plans always have (an instance of
// its own for whole planes whose height 4 divides measured no faster).  LV:
// the plan's level count where an instance knows it (tiles of L >= 1 layers
// carry level 1), so that the output pass reads level 1's bands without a
// run-time test of the count.  LV = 0: read from the plan.
template <typename T, int K, int BW, bool TL, bool ST, bool G4 = TL || ST, int LV = 0>
__global__ __launch_bounds__(512) void wtconv_whole_kernel(WtcWholeArgs<T> a)
{
    extern __shared__ float wtc_lds[];
    WtcWholeCtx<T> ctx;
    ctx.lds = wtc_lds;
    ctx.tid = threadIdx.x;
    ctx.nth = blockDim.x;
    wtc_whole_setup<T>(a, ctx, blockIdx.x);
    wtc_whole_load<T, K, BW, TL, ST, G4>(a, ctx, 0);
    wtc_whole_init<T, K>(a, ctx);
    wtc_lds_barrier();
    wtc_whole_fold<T, K>(a, ctx);
    wtc_whole_table<T, K, BW>(a, ctx);
    // Software pipeline over the images: image i+1 is staged (its input map
    // and first Haar levels written) in the same barrier interval as image i's
    // output pass, and the input of image i+2 is requested between the two,
    // so the wait for a prefetched input never waits for output stores issued
    // just before it (loads and stores share one counter) and the loads do
    // not queue behind the stores.
    wtc_whole_stage<T, K, BW, TL, ST, G4>(a, ctx);
    wtc_lds_barrier();
    if (ctx.nimg > 1) wtc_whole_load<T, K, BW, TL, ST, G4>(a, ctx, 1);
    for (int img = 0; img < ctx.nimg; ++img) {
        for (int m = wtc_whole_first_deep(a.p); !TL && m <= a.p.levels; ++m) {
            wtc_whole_analysis<T, K>(a, ctx, m);
            wtc_lds_barrier();
        }
        // The convolution phase issues FMAs back to back; the staging, load
        // and output phases wait on memory and LDS.  Lowering this wave's
        // priority for the convolution lets the other workgroup's latency-
        // bound waves issue first when both want the SIMD (measured: stage1
        // forward 64.5 -> 60.0 us, the 256 x 256 layer's step -10 %).
        __builtin_amdgcn_s_setprio(0);
        wtc_whole_conv<T, K, BW, !TL>(a, ctx);
        wtc_lds_barrier();
        __builtin_amdgcn_s_setprio(2);
        // the convolutions above have finished reading the input and analysis
        // maps, which the staging of the next image overwrites; the output
        // pass reads only the convolution outputs
        if (img + 1 < ctx.nimg) wtc_whole_stage<T, K, BW, TL, ST, G4>(a, ctx);
        if (img + 2 < ctx.nimg) wtc_whole_load<T, K, BW, TL, ST, G4>(a, ctx, img + 2);
        wtc_whole_select<T, ST>(a, ctx, img);
        wtc_whole_out<T, K, BW, TL, ST, 0, LV>(a, ctx);
        wtc_lds_barrier();
    }
}

template <typename T, int K, int BW, bool TL, bool ST, bool G4 = TL || ST, int LV = 0>
static hipError_t launch_tl(const WtcWholeArgs<T> &a, hipStream_t stream, int *resident)
{
    if (TL && a.p.tail) return hipErrorInvalidValue;  // the tiled instances carry no tail loop
    if (LV && a.p.levels != LV) return hipErrorInvalidValue;
    const size_t lds = (size_t)a.p.lds_floats * sizeof(float);
    const void *fn = (const void *)&wtconv_whole_kernel<T, K, BW, TL, ST, G4, LV>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (resident) {
        *resident = wtc_resident_blocks(fn, a.p.nthreads, lds);
        return hipSuccess;
    }
    const unsigned groups = (unsigned)((a.p.units + a.p.planes - 1) / a.p.planes);
    const unsigned blocks = groups * (unsigned)a.p.c;
    hipLaunchKernelGGL((wtconv_whole_kernel<T, K, BW, TL, ST, G4, LV>), dim3(blocks), dim3(a.p.nthreads), lds, stream,
                       a);
    return hipGetLastError();
}

template <typename T, int K, int BW>
static hipError_t launch_bw(const WtcWholeArgs<T> &a, hipStream_t stream, int *resident)
{
    if (a.p.tiled) {
        // level-1 tiles with 4-wide output blocks (every tile shape the
        // planner tries) know their level count; L = 0 tiles (a plain
        // depthwise convolution) and wider blocks read it from the plan
        if constexpr (BW == 4) {
            if (a.p.levels == 1) return launch_tl<T, K, BW, true, false, true, 1>(a, stream, resident);
        }
        return launch_tl<T, K, BW, true, false>(a, stream, resident);
    }
    return a.p.stack > 1 ? launch_tl<T, K, BW, false, true>(a, stream, resident)
                         : launch_tl<T, K, BW, false, false>(a, stream, resident);
}

template <typename T, int K>
static hipError_t launch_k(const WtcWholeArgs<T> &a, hipStream_t stream, int *resident)
{
    switch (a.p.out_bw) {
    case 8: return launch_bw<T, K, 8>(a, stream, resident);
    case 4: return launch_bw<T, K, 4>(a, stream, resident);
    default: return launch_bw<T, K, 2>(a, stream, resident);
    }
}

template <typename T>
static hipError_t launch_t(const WtcWholeArgs<T> &a, hipStream_t stream, int *resident = nullptr)
{
    switch (a.p.k) {
    case 1: return launch_k<T, 1>(a, stream, resident);
    case 3: return launch_k<T, 3>(a, stream, resident);
    case 5: return launch_k<T, 5>(a, stream, resident);
    case 7: return launch_k<T, 7>(a, stream, resident);
    default: return hipErrorInvalidValue;
    }
}

hipError_t wtc_launch_whole(int dtype, const WtcWholePlan &p, const void *in, void *out, const float *w_base,
                            const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
                            hipStream_t stream, const void *low)
{
    if (dtype == 0) {
        WtcWholeArgs<float> a{(const float *)in, (float *)out, w_base, bias, s_base, w_lvl, s_lvl, p,
                              (const float *)low};
        return launch_t<float>(a, stream);
    }
    WtcWholeArgs<_Float16> a{(const _Float16 *)in, (_Float16 *)out, w_base, bias, s_base, w_lvl, s_lvl, p,
                             (const float *)low};
    return launch_t<_Float16>(a, stream);
}

int wtc_whole_resident(int dtype, const WtcWholePlan &p)
{
    int r = 0;
    hipError_t e;
    if (dtype == 0) {
        WtcWholeArgs<float> a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, p};
        e = launch_t<float>(a, nullptr, &r);
    } else {
        WtcWholeArgs<_Float16> a{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, p};
        e = launch_t<_Float16>(a, nullptr, &r);
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return r;
}
