// wtconv_lowpass.hip -- the level-1 low-pass band of a plane, written to HBM
// for planes too large for one workgroup: the deeper levels of the layer are
// then computed from it (technical summary, Methodology: the Haar analysis
// feeds each level from the low-pass band of the level above), and a fill
// kernel for small parameter buffers.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wtconv_launch.h"

namespace {

constexpr int kThreads = 256;

// One thread per 2 x 2 output block: reads a 4 x 4 input block as four
// 16-byte (fp32) rows, writes two 8-byte rows.  The output is fp32 whatever
// the input type: it is an intermediate of the layer, and the layer's outputs
// are rounded once, at their own store.
template <typename T>
__global__ __launch_bounds__(kThreads) void lowpass_kernel(const T *__restrict__ in, float *__restrict__ out,
                                                           int64_t planes, int h, int w)
{
    const int h2 = h / 2, w2 = w / 2, bw = w2 / 2, bh = h2 / 2;
    const int64_t per = (int64_t)bh * bw, total = planes * per;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = t / per;
        const int r = (int)(t - p * per);
        const int bi = r / bw, bj = r - (r / bw) * bw;
        const T *src = in + p * ((int64_t)h * w) + (int64_t)(4 * bi) * w + 4 * bj;
        float v[4][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) v[q][e] = (float)src[(int64_t)q * w + e];
        float *dst = out + p * ((int64_t)h2 * w2) + (int64_t)(2 * bi) * w2 + 2 * bj;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                dst[(int64_t)a * w2 + b] =
                    0.5f * (v[2 * a][2 * b] + v[2 * a][2 * b + 1] + v[2 * a + 1][2 * b] + v[2 * a + 1][2 * b + 1]);
    }
}

__global__ void fill_kernel(float *p, int64_t n, float v)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

unsigned grid_for(int64_t n)
{
    const int64_t g = (n + kThreads - 1) / kThreads;
    return (unsigned)(g < 1 ? 1 : (g > 262144 ? 262144 : g));
}

}  // namespace

hipError_t wtc_launch_lowpass(int dtype, const void *in, float *out, int64_t planes, int h, int w,
                              hipStream_t stream)
{
    if (h % 4 || w % 4) return hipErrorInvalidValue;  // whole 2 x 2 output blocks
    const unsigned g = grid_for(planes * (h / 4) * (w / 4));
    if (dtype == 0)
        hipLaunchKernelGGL(lowpass_kernel<float>, dim3(g), dim3(kThreads), 0, stream, (const float *)in, out, planes,
                           h, w);
    else
        hipLaunchKernelGGL(lowpass_kernel<_Float16>, dim3(g), dim3(kThreads), 0, stream, (const _Float16 *)in, out,
                           planes, h, w);
    return hipGetLastError();
}

hipError_t wtc_launch_fill(float *p, int64_t n, float v, hipStream_t stream)
{
    hipLaunchKernelGGL(fill_kernel, dim3(grid_for(n) < 64 ? grid_for(n) : 64), dim3(kThreads), 0, stream, p, n, v);
    return hipGetLastError();
}
