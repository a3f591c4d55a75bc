// wtconv_dwconv.hip -- the layer with no Haar levels (L = 0): a plain scaled
// k x k depthwise cross-correlation with bias, y = s0 * (W0 (*) x + b0), and its
// data backward (kernel turned by 180 degrees, no bias).
//
// One workgroup per (plane, band of 16 output rows); the rows plus the halo
// are staged in LDS as fp32 and every thread computes 4 adjacent outputs.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wtconv_launch.h"

namespace {

constexpr int kRows = 16;
constexpr int kThreads = 256;

template <typename T, int K>
__global__ __launch_bounds__(kThreads) void dwconv_kernel(const T *__restrict__ in, T *__restrict__ out,
                                                          const float *__restrict__ w_base,
                                                          const float *__restrict__ bias,
                                                          const float *__restrict__ s_base, int C, int H, int W,
                                                          int rotate, int pitch)
{
    constexpr int R = K / 2, kk = K * K;
    extern __shared__ float lds[];
    float *wf = lds;          // kk folded weights
    float *tile = lds + 64;   // (kRows + 2R) x pitch
    const int bands = (H + kRows - 1) / kRows;
    const int plane = blockIdx.x / bands, band = blockIdx.x % bands;
    const int c = plane % C;
    const int h0 = band * kRows;
    const int64_t hw = (int64_t)H * W;
    const T *xin = in + (int64_t)plane * hw;
    T *yout = out + (int64_t)plane * hw;
    const float s0 = s_base[c];
    for (int e = threadIdx.x; e < kk; e += blockDim.x) wf[e] = s0 * w_base[c * kk + (rotate ? kk - 1 - e : e)];
    const float b0 = (!rotate && bias) ? s0 * bias[c] : 0.0f;
    const int rows = kRows + 2 * R, cols = W + 2 * R;
    for (int idx = threadIdx.x; idx < rows * cols; idx += blockDim.x) {
        const int ri = idx / cols, ci = idx - ri * cols;
        const int hh = h0 - R + ri, ww = ci - R;
        float v = 0.0f;
        if (hh >= 0 && hh < H && ww >= 0 && ww < W) v = (float)xin[(int64_t)hh * W + ww];
        tile[ri * pitch + ci] = v;
    }
    __syncthreads();
    const int nbx = (W + 3) / 4;
    for (int idx = threadIdx.x; idx < kRows * nbx; idx += blockDim.x) {
        const int ri = idx / nbx, bx = idx - ri * nbx;
        const int h = h0 + ri;
        if (h >= H) continue;
        float acc[4] = {b0, b0, b0, b0};
#pragma unroll
        for (int u = 0; u < K; ++u) {
            float row[4 + K - 1];
#pragma unroll
            for (int e = 0; e < 4 + K - 1; ++e) row[e] = tile[(ri + u) * pitch + 4 * bx + e];
#pragma unroll
            for (int v = 0; v < K; ++v)
#pragma unroll
                for (int d = 0; d < 4; ++d) acc[d] = __builtin_fmaf(wf[u * K + v], row[d + v], acc[d]);
        }
#pragma unroll
        for (int d = 0; d < 4; ++d)
            if (4 * bx + d < W) yout[(int64_t)h * W + 4 * bx + d] = (T)acc[d];
    }
}

template <typename T, int K>
hipError_t launch(const void *in, void *out, const float *w_base, const float *bias, const float *s_base, int N,
                  int C, int H, int W, int rotate, hipStream_t stream)
{
    constexpr int R = K / 2;
    // tile columns cover the ragged last group of 4 outputs as well
    const int pitch = ((W + 3) / 4) * 4 + 2 * R + 4;
    const size_t lds = (64 + (size_t)(kRows + 2 * R) * pitch) * sizeof(float);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    const void *fn = (const void *)&dwconv_kernel<T, K>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const unsigned blocks = (unsigned)((int64_t)N * C * ((H + kRows - 1) / kRows));
    hipLaunchKernelGGL((dwconv_kernel<T, K>), dim3(blocks), dim3(kThreads), lds, stream, (const T *)in, (T *)out,
                       w_base, bias, s_base, C, H, W, rotate, pitch);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(int k, const void *in, void *out, const float *w_base, const float *bias, const float *s_base,
                    int N, int C, int H, int W, int rotate, hipStream_t stream)
{
    switch (k) {
    case 1: return launch<T, 1>(in, out, w_base, bias, s_base, N, C, H, W, rotate, stream);
    case 3: return launch<T, 3>(in, out, w_base, bias, s_base, N, C, H, W, rotate, stream);
    case 5: return launch<T, 5>(in, out, w_base, bias, s_base, N, C, H, W, rotate, stream);
    case 7: return launch<T, 7>(in, out, w_base, bias, s_base, N, C, H, W, rotate, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Maximum plane width the L = 0 kernel stages (its LDS band must fit).
int wtc_dwconv_max_width(int k) { return (160 * 1024 / 4 - 64) / (kRows + k) - k - 8; }

hipError_t wtc_launch_dwconv(int dtype, int k, const void *in, void *out, const float *w_base, const float *bias,
                             const float *s_base, int N, int C, int H, int W, int rotate, hipStream_t stream)
{
    if (dtype == 0) return launch_t<float>(k, in, out, w_base, bias, s_base, N, C, H, W, rotate, stream);
    return launch_t<_Float16>(k, in, out, w_base, bias, s_base, N, C, H, W, rotate, stream);
}
