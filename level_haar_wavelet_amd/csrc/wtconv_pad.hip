// wtconv_pad.hip -- window copies between NCHW activations of different
// sides, for layers whose sides 2^L does not divide.  Padding every odd level
// map with one zero row / column at the bottom / right before its Haar
// analysis and cropping that level's synthesis back is the same operator as
// zero-padding the input once, at the bottom and right, to multiples of 2^L and
// cropping the result: the padded pixels only feed outputs the crop removes,
// and every level's zero "same" padding sees zeros either way.  (The pages
// describe the layer on the Haar pyramid, technical summary, Methodology; they
// do not treat odd sides.)
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wtconv_launch.h"

namespace {

constexpr int kThreads = 256;

// out[p][i][j] = in[p][i][j] for i < hin, j < win, else 0, over the hout x wout
// output window of each plane: a zero-padded copy when hout >= hin and
// wout >= win, a crop when hout <= hin and wout <= win.  One workgroup per
// output row (grid-stride), its threads across the row.
template <typename T>
__global__ __launch_bounds__(kThreads) void repack_kernel(const T *__restrict__ in, T *__restrict__ out, int64_t rows,
                                                          int hin, int win, int hout, int wout)
{
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const int64_t plane = r / hout;
        const int i = (int)(r - plane * hout);
        T *dst = out + r * wout;
        if (i < hin) {
            const T *src = in + (plane * hin + i) * win;
            for (int j = threadIdx.x; j < wout; j += kThreads) dst[j] = j < win ? src[j] : (T)0;
        } else {
            for (int j = threadIdx.x; j < wout; j += kThreads) dst[j] = (T)0;
        }
    }
}

}  // namespace

hipError_t wtc_launch_repack(int dtype, const void *in, void *out, int64_t planes, int hin, int win, int hout,
                             int wout, hipStream_t stream)
{
    if (planes < 1 || hin < 1 || win < 1 || hout < 1 || wout < 1) return hipErrorInvalidValue;
    const int64_t rows = planes * hout;
    const unsigned g = (unsigned)(rows < 65536 ? rows : 65536);
    if (dtype == 0)
        hipLaunchKernelGGL(repack_kernel<float>, dim3(g), dim3(kThreads), 0, stream, (const float *)in, (float *)out,
                           rows, hin, win, hout, wout);
    else
        hipLaunchKernelGGL(repack_kernel<_Float16>, dim3(g), dim3(kThreads), 0, stream, (const _Float16 *)in,
                           (_Float16 *)out, rows, hin, win, hout, wout);
    return hipGetLastError();
}
