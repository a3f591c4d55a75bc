// wtconv_wgrad.hip -- parameter-gradient kernels of the WTConv layer for
// gfx950: the fused per-channel correlation kernel (phases in
// wtconv_wgrad_body.h) and the second pass that sums the workgroup partials in
// a fixed order and applies the chain rule through the scales.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wtconv_launch.h"
#include "wtconv_wgrad_body.h"

static __device__ __forceinline__ void wtc_lds_barrier_wg() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Q: accumulator sets per thread the kernel holds (1, 2 for whole planes, or
// WTC_WG_QMAX for q = 2..3 on tiles and q = 3).
// With one set (fp32, k <= 5) the whole-plane kernel is held to 128 VGPRs: two
// 512-thread workgroups (four waves per SIMD) share a compute unit.  The tiled
// instance is held to three waves per SIMD (168 VGPRs), the occupancy its LDS
// allows anyway (three 256-thread workgroups of 42-45 KB per compute unit), and
// so is the two-set whole-plane instance (160 VGPRs at k = 5 fp32: three
// workgroups fit where its LDS allows, e.g. the 64 x 64 maps of the nested
// weight backward at L = 3; the three-set instance holds 188).
template <int Q, int TB, int K, bool TL>
struct WtcWgradWaves {
    static constexpr int v = (Q == 1 && TB == 4 && K <= 5) ? (TL ? 3 : 4) : (Q == 2 && TB == 4 && K <= 5) ? 3 : 1;
};

template <typename T, int K, int VEC, int Q, bool TL>
__global__ __launch_bounds__(512, (WtcWgradWaves<Q, (int)sizeof(T), K, TL>::v)) void wtconv_wgrad_kernel(WtcWgradArgs<T> a)
{
    extern __shared__ float wtc_lds[];
    WtcWgradCtx<T, VEC> ctx;
    ctx.lds = wtc_lds;
    ctx.tid = threadIdx.x;
    ctx.nth = blockDim.x;
    wtc_wgrad_setup<T, VEC>(a, ctx, blockIdx.x);
    wtc_wgrad_load<T, VEC, TL>(a, ctx, 0);
    wtc_wgrad_zero<T, VEC>(a, ctx);
    wtc_lds_barrier_wg();
    wtc_wgrad_table<T, K, VEC>(a, ctx);
    float acc[Q][K * K + 1];
#pragma unroll
    for (int s = 0; s < Q; ++s)
#pragma unroll
        for (int e = 0; e < K * K + 1; ++e) acc[s][e] = 0.0f;
    for (int img = 0; img < ctx.nimg; ++img) {
        wtc_wgrad_stage<T, K, VEC, TL>(a, ctx);
        wtc_lds_barrier_wg();
        if (img + 1 < ctx.nimg) wtc_wgrad_load<T, VEC, TL>(a, ctx, img + 1);
        for (int m = a.p.first_deep; !TL && m <= a.p.levels; ++m) {
            wtc_wgrad_analysis<T, K, VEC>(a, ctx, m);
            wtc_lds_barrier_wg();
        }
        // low wave priority for the FMA-bound correlation, high for the
        // latency-bound staging and analysis (as in the whole-plane kernel)
        __builtin_amdgcn_s_setprio(0);
        wtc_wgrad_correlate<T, K, VEC, Q, !TL && Q == 1>(a, ctx, acc);
        wtc_lds_barrier_wg();
        __builtin_amdgcn_s_setprio(2);
    }
#pragma unroll
    for (int s = 0; s < Q; ++s) {
        if (s < a.p.q) {
            wtc_wgrad_park<T, K, VEC>(a, ctx, acc[s]);
            wtc_lds_barrier_wg();
            wtc_wgrad_chunks<T, K, VEC>(a, ctx, s);
            wtc_lds_barrier_wg();
            wtc_wgrad_combine<T, K, VEC>(a, ctx, s);
            wtc_lds_barrier_wg();
        }
    }
    wtc_wgrad_write<T, K, VEC>(a, ctx);
}

// One wave per (channel, map): lane t < k*k sums tap t over the workgroup
// partials in group order (consecutive lanes read consecutive floats), lane
// k*k does the same for the sum of dy; the scale gradient <W, G> (+ b0 Gb) is
// a fixed butterfly reduction across the wave, so the result is bitwise
// reproducible.
__global__ __launch_bounds__(256) void wtconv_wgrad_finalize_kernel(int C, int k, int levels, int groups, int plen,
                                                                    const float *__restrict__ partial,
                                                                    const float *__restrict__ w_base,
                                                                    const float *__restrict__ bias,
                                                                    const float *__restrict__ s_base,
                                                                    const float *__restrict__ w_lvl,
                                                                    const float *__restrict__ s_lvl, float *dw_base,
                                                                    float *dbias, float *ds_base, float *dw_lvl,
                                                                    float *ds_lvl)
{
    const int nmaps = 1 + 4 * levels;
    const int lane = threadIdx.x & 63;
    const int pair = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (pair >= C * nmaps) return;  // whole waves leave together
    const int c = pair / nmaps, g = pair - c * nmaps;
    float term = wtc_wgrad_finalize_lane(lane, c, g, C, k, groups, plen, partial, w_base, bias, s_base, w_lvl,
                                         s_lvl, dw_base, dbias, dw_lvl);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) term += __shfl_xor(term, d, 64);
    if (lane == 0) wtc_wgrad_finalize_store(c, g, C, term, ds_base, ds_lvl);
}

template <typename T, int K, int VEC, int Q, bool TL>
static hipError_t launch_wgrad_q(const WtcWgradArgs<T> &a, hipStream_t stream, int *resident)
{
    if ((TL || Q != 1) && a.p.tail) return hipErrorInvalidValue;  // these instances carry no tail pieces
    const size_t lds = (size_t)a.p.lds_floats * sizeof(float);
    const void *fn = (const void *)&wtconv_wgrad_kernel<T, K, VEC, Q, TL>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (resident) {
        *resident = wtc_resident_blocks(fn, a.p.nthreads, lds);
        return hipSuccess;
    }
    const unsigned blocks = (unsigned)(a.p.groups * a.p.c);
    hipLaunchKernelGGL((wtconv_wgrad_kernel<T, K, VEC, Q, TL>), dim3(blocks), dim3(a.p.nthreads), lds, stream, a);
    return hipGetLastError();
}

template <typename T, int K, int VEC, bool TL = false>
static hipError_t launch_wgrad(const WtcWgradArgs<T> &a, hipStream_t stream, int *resident)
{
    if (a.p.q == 1) return launch_wgrad_q<T, K, VEC, 1, TL>(a, stream, resident);
    if (a.p.q == 2 && !TL) return launch_wgrad_q<T, K, VEC, 2, false>(a, stream, resident);
    return launch_wgrad_q<T, K, VEC, WTC_WG_QMAX, TL>(a, stream, resident);
}

template <typename T, int K>
static hipError_t launch_wgrad_k(const WtcWgradArgs<T> &a, hipStream_t stream, int *resident)
{
    switch (a.p.vec) {
    // tiled plans always stage 4-element segments
    case 4: return a.p.tiled ? launch_wgrad<T, K, 4, true>(a, stream, resident)
                             : launch_wgrad<T, K, 4>(a, stream, resident);
    case 2: return launch_wgrad<T, K, 2>(a, stream, resident);
    default: return launch_wgrad<T, K, 1>(a, stream, resident);
    }
}

template <typename T>
static hipError_t launch_wgrad_t(const WtcWgradArgs<T> &a, hipStream_t stream, int *resident = nullptr)
{
    switch (a.p.k) {
    case 1: return launch_wgrad_k<T, 1>(a, stream, resident);
    case 3: return launch_wgrad_k<T, 3>(a, stream, resident);
    case 5: return launch_wgrad_k<T, 5>(a, stream, resident);
    case 7: return launch_wgrad_k<T, 7>(a, stream, resident);
    default: return hipErrorInvalidValue;
    }
}

int wtc_wgrad_resident(int dtype, const WtcWgradPlan &p)
{
    int r = 0;
    hipError_t e;
    if (dtype == 0) {
        WtcWgradArgs<float> a{nullptr, nullptr, nullptr, p};
        e = launch_wgrad_t<float>(a, nullptr, &r);
    } else {
        WtcWgradArgs<_Float16> a{nullptr, nullptr, nullptr, p};
        e = launch_wgrad_t<_Float16>(a, nullptr, &r);
    }
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return r;
}

hipError_t wtc_launch_wgrad(int dtype, const WtcWgradPlan &p, const void *x, const void *dy, float *partial,
                            hipStream_t stream, void *llx, void *lld)
{
    if ((llx != nullptr) != (lld != nullptr) || (llx && !p.tiled)) return hipErrorInvalidValue;
    if (dtype == 0) {
        WtcWgradArgs<float> a{(const float *)x, (const float *)dy, partial, p, (float *)llx, (float *)lld};
        return launch_wgrad_t<float>(a, stream);
    }
    WtcWgradArgs<_Float16> a{(const _Float16 *)x, (const _Float16 *)dy, partial, p, (float *)llx,
                             (float *)lld};
    return launch_wgrad_t<_Float16>(a, stream);
}

// The same over several partial-row sets: waves are numbered across the sets
// (set i holds C (1 + 4 L_i) of them, in set order).
__global__ __launch_bounds__(256) void wtconv_wgrad_finalize_sets_kernel(WtcFinalizeSets F)
{
    const int lane = threadIdx.x & 63;
    int pair = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    int i = 0;
    for (; i < F.n; ++i) {
        const int n = F.C * (1 + 4 * F.s[i].levels);
        if (pair < n) break;
        pair -= n;
    }
    if (i >= F.n) return;  // whole waves leave together
    const WtcFinalizeSet &f = F.s[i];
    const int nmaps = 1 + 4 * f.levels;
    const int c = pair / nmaps, g = pair - c * nmaps;
    float term = wtc_wgrad_finalize_lane(lane, c, g, F.C, F.k, f.groups, f.plen, f.partial, f.w_base, f.bias,
                                         f.s_base, f.w_lvl, f.s_lvl, f.dw_base, f.dbias, f.dw_lvl);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) term += __shfl_xor(term, d, 64);
    if (lane == 0) wtc_wgrad_finalize_store(c, g, F.C, term, f.ds_base, f.ds_lvl);
}

hipError_t wtc_launch_wgrad_finalize_sets(const WtcFinalizeSets &f, hipStream_t stream)
{
    if (f.n < 1 || f.n > WTC_FIN_MAX) return hipErrorInvalidValue;
    int pairs = 0;
    for (int i = 0; i < f.n; ++i) pairs += f.C * (1 + 4 * f.s[i].levels);  // one wave each, four per workgroup
    hipLaunchKernelGGL(wtconv_wgrad_finalize_sets_kernel, dim3((pairs + 3) / 4), dim3(256), 0, stream, f);
    return hipGetLastError();
}

hipError_t wtc_launch_wgrad_finalize(int C, int k, int levels, int groups, int plen, const float *partial,
                                     const float *w_base, const float *bias, const float *s_base,
                                     const float *w_lvl, const float *s_lvl, float *dw_base, float *dbias,
                                     float *ds_base, float *dw_lvl, float *ds_lvl, hipStream_t stream)
{
    const int pairs = C * (1 + 4 * levels);  // one wave each, four per workgroup
    hipLaunchKernelGGL(wtconv_wgrad_finalize_kernel, dim3((pairs + 3) / 4), dim3(256), 0, stream, C, k, levels,
                       groups, plen, partial, w_base, bias, s_base, w_lvl, s_lvl, dw_base, dbias, ds_base, dw_lvl,
                       ds_lvl);
    return hipGetLastError();
}
