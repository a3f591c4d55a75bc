// wtconv_large.hip -- the fused large-plane forward / data-backward kernel for
// gfx950 (plans and phases in wtconv_large_body.h and wtconv_whole_body.h).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wtconv_large_body.h"
#include "wtconv_launch.h"

// Workgroup barrier that waits only for this wave's LDS operations: global
// loads issued before it (the next tile's input) stay in flight.
static __device__ __forceinline__ void wtc_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Two workgroups per compute unit (their LDS allows no more): at most 256
// registers per lane.  DL: the deeper-levels plan's level count (L - 1) for
// DL = 1..3, a kernel instance each, so that its staging, analysis and output
// passes take no branch on it; DL = 0: read from the plan (L >= 5, where the
// unrolled instances measured no faster).  HALF: tiles whose pieces run as
// 2-row halves (without the base path: the nested call of a larger plane).
template <typename T, int K, int BW, int DL, bool HALF = false>
__global__ __launch_bounds__(256, 2) void wtconv_large_kernel(WtcLargeArgs<T> A)
{
    extern __shared__ float wtc_lds[];
    const WtcWholeArgs<T> &ad = A.d, &at = A.t;
    WtcWholeCtx<T> cd, ct;
    cd.lds = ct.lds = wtc_lds;
    cd.tid = ct.tid = threadIdx.x;
    cd.nth = ct.nth = blockDim.x;
    wtc_whole_setup<T>(ad, cd, blockIdx.x);
    wtc_whole_setup<T>(at, ct, blockIdx.x);
    const int tiles = at.p.tiles_x * at.p.tiles_y;
    // the first image's deeper-levels input is requested before the set-up
    WtcLargeRaw<T> raw;
    wtc_large_fetch_d<T>(A, cd, 0, raw);
    for (int i = ct.tid; i < A.lds_floats; i += ct.nth) wtc_lds[i] = 0.0f;
    wtc_lds_barrier();
    wtc_whole_fold<T, K>(ad, cd);
    wtc_whole_fold<T, K>(at, ct);
    wtc_whole_table<T, K, BW>(ad, cd);
    wtc_whole_table<T, K, BW>(at, ct);
    for (int img = 0; img < cd.nimg; ++img) {
        // deeper levels, staged from x through registers
        float ll[4][4];
        wtc_large_reduce_d<T>(raw, ll);
        if (img > 0) {
            wtc_large_zero_d<T>(A, cd);
            wtc_lds_barrier();
        }
        wtc_whole_stage_vals<T, K, BW, false, false, true, DL>(ad, cd, ll);  // the plan has 4-row groups
        // the first tile's input is requested now and lands while the deeper
        // levels are computed
        const int u0 = img * tiles;
        wtc_whole_load<T, K, BW, true, false>(at, ct, u0);
        wtc_lds_barrier();
        // the staging computed levels 1, 2 (two or more) and 3 (three or more)
#pragma unroll
        for (int m = DL ? (DL >= 3 ? 4 : (DL >= 2 ? 3 : 2)) : wtc_whole_first_deep(ad.p); m <= (DL ? DL : ad.p.levels);
             ++m) {
            wtc_whole_analysis<T, K>(ad, cd, m);
            wtc_lds_barrier();
        }
        __builtin_amdgcn_s_setprio(0);
        wtc_whole_conv<T, K, BW, false>(ad, cd);
        wtc_lds_barrier();
        __builtin_amdgcn_s_setprio(2);
        wtc_whole_out<T, K, BW, false, false, 2, DL>(ad, cd);
        wtc_lds_barrier();
        // base and level 1 on the tiles of the image, the deeper levels' term
        // from LDS; the same software pipeline as the tiled whole-plane kernel
        wtc_whole_stage<T, K, BW, true, false>(at, ct);
        wtc_lds_barrier();
        if (tiles > 1) wtc_whole_load<T, K, BW, true, false>(at, ct, u0 + 1);
        for (int t = 0; t < tiles; ++t) {
            // the next image's deeper-levels input lands during the last tile
            if (t == tiles - 1 && img + 1 < cd.nimg) wtc_large_fetch_d<T>(A, cd, img + 1, raw);
            __builtin_amdgcn_s_setprio(0);
            wtc_whole_conv<T, K, BW, false, HALF>(at, ct);
            wtc_lds_barrier();
            __builtin_amdgcn_s_setprio(2);
            if (t + 1 < tiles) wtc_whole_stage<T, K, BW, true, false>(at, ct);
            if (t + 2 < tiles) wtc_whole_load<T, K, BW, true, false>(at, ct, u0 + t + 2);
            wtc_whole_select<T, false>(at, ct, u0 + t);
            wtc_whole_out<T, K, BW, true, false, 1, 1>(at, ct);  // the tile plan has level 1
            wtc_lds_barrier();
        }
    }
}

template <typename T, int K, int DL, bool HALF = false>
static hipError_t launch_dl(const WtcLargeArgs<T> &a, hipStream_t stream, int *resident)
{
    // (other instances run such plans' pieces whole)
    if (HALF && !a.t.p.halves) return hipErrorInvalidValue;
    // the instance's analysis starts where the plan's staging stops
    const WtcWholePlan &d = a.d.p;
    const int first = d.stage_l3 ? 4 : (d.gr == 4 && d.vec >= 4 && d.levels >= 2 ? 3 : 2);
    if (DL && (d.levels != DL || first != (DL >= 3 ? 4 : (DL >= 2 ? 3 : 2)))) return hipErrorInvalidValue;
    if (d.tail || a.t.p.tail) return hipErrorInvalidValue;  // no tail loop in this kernel
    if (a.t.p.levels != 1) return hipErrorInvalidValue;     // the tiles' output pass assumes level 1
    const size_t lds = (size_t)a.lds_floats * sizeof(float);
    const void *fn = (const void *)&wtconv_large_kernel<T, K, 4, DL, HALF>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (resident) {
        *resident = wtc_resident_blocks(fn, a.t.p.nthreads, lds);
        return hipSuccess;
    }
    const unsigned groups = (unsigned)((a.n + a.planes - 1) / a.planes);
    hipLaunchKernelGGL((wtconv_large_kernel<T, K, 4, DL, HALF>), dim3(groups * (unsigned)a.c), dim3(a.t.p.nthreads),
                       lds, stream, a);
    return hipGetLastError();
}

template <typename T, int K>
static hipError_t launch_k(const WtcLargeArgs<T> &a, hipStream_t stream, int *resident)
{
    if (a.d.p.out_bw != 4 || a.t.p.out_bw != 4 || a.d.p.gr != 4) return hipErrorInvalidValue;
    if constexpr (sizeof(T) == 4 && K == 5) {
        // the nested call of a larger plane runs on its fp32 level-1 map
        if (a.t.p.halves) {
            switch (a.d.p.levels) {
            case 1: return launch_dl<T, K, 1, true>(a, stream, resident);
            case 2: return launch_dl<T, K, 2, true>(a, stream, resident);
            case 3: return launch_dl<T, K, 3, true>(a, stream, resident);
            default: return launch_dl<T, K, 0, true>(a, stream, resident);
            }
        }
    }
    switch (a.d.p.levels) {
    case 1: return launch_dl<T, K, 1>(a, stream, resident);
    case 2: return launch_dl<T, K, 2>(a, stream, resident);
    case 3: return launch_dl<T, K, 3>(a, stream, resident);
    default: return launch_dl<T, K, 0>(a, stream, resident);
    }
}

template <typename T>
static hipError_t launch_t(const WtcLargeArgs<T> &a, hipStream_t stream, int *resident = nullptr)
{
    if (a.t.p.nthreads != 256 || a.d.p.nthreads != 256) return hipErrorInvalidValue;
    switch (a.t.p.k) {
    case 1: return launch_k<T, 1>(a, stream, resident);
    case 3: return launch_k<T, 3>(a, stream, resident);
    case 5: return launch_k<T, 5>(a, stream, resident);
    case 7: return launch_k<T, 7>(a, stream, resident);
    default: return hipErrorInvalidValue;
    }
}

hipError_t wtc_launch_large(int dtype, const WtcLargePlan &p, const void *in, void *out, const float *w_base,
                            const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
                            hipStream_t stream)
{
    if (dtype == 0)
        return launch_t<float>(wtc_large_args<float>(p, (const float *)in, (float *)out, w_base, bias, s_base, w_lvl,
                                                     s_lvl),
                               stream);
    return launch_t<_Float16>(wtc_large_args<_Float16>(p, (const _Float16 *)in, (_Float16 *)out, w_base, bias, s_base,
                                                       w_lvl, s_lvl),
                              stream);
}

int wtc_large_resident(int dtype, const WtcLargePlan &p)
{
    int r = 0;
    hipError_t e;
    if (dtype == 0)
        e = launch_t<float>(wtc_large_args<float>(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
                            nullptr, &r);
    else
        e = launch_t<_Float16>(
            wtc_large_args<_Float16>(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), nullptr, &r);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return r;
}
