// wtconv_unfused.hip -- the unfused WTConv layer, a test/bench-only baseline:
// the layer composed of separate kernels with every intermediate in HBM, the
// way the layer is written in a framework (the composition the pages measure
// their fused kernel against).
//
// Source: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation" (arXiv 2608.10805), technical summary, Problem Statement and
// Methodology (the reference implementation's per-level wavelet transform,
// convolution, scale, concatenation and inverse transform, each a separate
// pass over HBM), and its analysis of the element moves of that composition.
//
// Forward, per level l = 1..L (orthonormal Haar, factor 1/2 per step):
//   Y_l   = analysis(LL_{l-1})            (4 bands; LL_0 = x, LL_l = band 0 of Y_l)
//   Zc_l  = W_l (*) Y_l                   (depthwise over the 4C band channels)
//   Zs_l  = s_l * Zc_l
// then from the deepest level up, with N_{L} = 0:
//   A_l   = Zs_l[band 0] + N_l,   N_{l-1} = synthesis(A_l, Zs_l[bands 1..3])
// and y = s0 * (W0 (*) x + b0) + N_0 (base conv Bc, scaled Bs, final add).
// The backward passes are the adjoints, step by step, as reverse-mode
// differentiation of that composition produces them (analysis and synthesis
// are each other's adjoints; a convolution's data adjoint is the convolution
// with the kernel turned by 180 degrees; its weight gradient a correlation).
//
// Everything here is plain and separate on purpose: one kernel per step, one
// HBM round trip per intermediate, intermediates stored in the activation
// type.  The workspace holds the forward's intermediates for the backward
// calls (the caller passes the same workspace to all three calls).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/wtconv.h"

namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float ld(const T *p, int64_t i) { return (float)p[i]; }
template <typename T>
__device__ __forceinline__ void st(T *p, int64_t i, float v) { p[i] = (T)v; }

unsigned grid_for(int64_t n)
{
    int64_t g = (n + kThreads - 1) / kThreads;
    return (unsigned)(g < 65536 * 4 ? (g < 1 ? 1 : g) : 65536 * 4);
}

// Haar analysis of P planes of h x w (even) into 4 bands of (h/2) x (w/2):
// out[p][b] at out + p * ostride + b * (h/2)(w/2); input plane p at in + p * istride.
template <typename T>
__global__ void k_analysis(const T *in, int64_t istride, T *out, int64_t ostride, int64_t P, int h, int w)
{
    const int h2 = h / 2, w2 = w / 2;
    const uint32_t per = (uint32_t)(h2 * w2), total = (uint32_t)(P * per);
    for (uint32_t t = blockIdx.x * blockDim.x + threadIdx.x; t < total; t += gridDim.x * blockDim.x) {
        const uint32_t p = t / per, r = t - p * per;
        const uint32_t i = r / (uint32_t)w2, j = r - i * (uint32_t)w2;
        const T *s = in + p * istride + (int64_t)(2 * i) * w + 2 * j;
        const float a = ld(s, 0), b = ld(s, 1), c = ld(s, w), d = ld(s, w + 1);
        T *o = out + p * ostride + (int64_t)i * w2 + j;
        st(o, 0, 0.5f * (a + b + c + d));
        st(o, per, 0.5f * (a + b - c - d));
        st(o, 2 * per, 0.5f * (a - b + c - d));
        st(o, 3 * per, 0.5f * (a - b - c + d));
    }
}

// Haar synthesis: the low-pass band from `ll` (plane stride lstride) and the
// three detail bands from `bands` (bands 1..3 of a 4-band block of stride
// bstride), into P planes of (2h) x (2w).
template <typename T>
__global__ void k_synthesis(const T *ll, int64_t lstride, const T *bands, int64_t bstride, T *out, int64_t P, int h,
                            int w)
{
    const uint32_t per = (uint32_t)(h * w), total = (uint32_t)(P * per);
    for (uint32_t t = blockIdx.x * blockDim.x + threadIdx.x; t < total; t += gridDim.x * blockDim.x) {
        const uint32_t p = t / per, r = t - p * per;
        const uint32_t i = r / (uint32_t)w, j = r - i * (uint32_t)w;
        const float a0 = ld(ll, p * lstride + r);
        const T *bb = bands + p * bstride + r;
        const float a1 = ld(bb, per), a2 = ld(bb, 2 * per), a3 = ld(bb, 3 * per);
        T *o = out + (int64_t)p * (4 * per) + (int64_t)(2 * i) * (2 * w) + 2 * j;
        st(o, 0, 0.5f * (a0 + a1 + a2 + a3));
        st(o, 1, 0.5f * (a0 + a1 - a2 - a3));
        st(o, 2 * w, 0.5f * (a0 - a1 + a2 - a3));
        st(o, 2 * w + 1, 0.5f * (a0 - a1 - a2 + a3));
    }
}

// Depthwise k x k cross-correlation with zero padding over P planes, channel
// of plane p = p % C; weights [C][k][k] (turned by 180 degrees if rotate),
// optional bias [C].
template <typename T, int K>
__global__ void k_dwconv(const T *in, T *out, const float *wt, const float *bias, int C, int64_t P, int h, int w,
                         int rotate)
{
    constexpr int R = K / 2, KK = K * K;
    const int64_t per = (int64_t)h * w, total = P * per;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = t / per;
        const int r = (int)(t - p * per);
        const int i = r / w, j = r - (r / w) * w;
        const int c = (int)(p % C);
        const T *src = in + p * per;
        const float *wc = wt + (int64_t)c * KK;
        float acc = bias ? bias[c] : 0.0f;
        for (int u = 0; u < K; ++u) {
            const int ii = i + u - R;
            if (ii < 0 || ii >= h) continue;
            for (int v = 0; v < K; ++v) {
                const int jj = j + v - R;
                if (jj < 0 || jj >= w) continue;
                const int e = u * K + v;
                acc += wc[rotate ? KK - 1 - e : e] * ld(src, (int64_t)ii * w + jj);
            }
        }
        st(out, t, acc);
    }
}

// out = s[channel] * in (+ add, elementwise, if given); channel of plane p = p % C.
template <typename T>
__global__ void k_scale_add(const T *in, const float *s, const T *add, T *out, int C, int64_t P, int64_t per)
{
    const uint32_t total = (uint32_t)(P * per), per32 = (uint32_t)per;
    for (uint32_t t = blockIdx.x * blockDim.x + threadIdx.x; t < total; t += gridDim.x * blockDim.x) {
        const uint32_t c = (t / per32) % (uint32_t)C;
        float v = (s ? s[c] : 1.0f) * ld(in, t);
        if (add) v += ld(add, t);
        st(out, t, v);
    }
}

// out[p] = a[p * astride + r] + b[p * bstride + r], r < per.
template <typename T>
__global__ void k_add_strided(const T *a, int64_t astride, const T *b, int64_t bstride, T *out, int64_t P, int64_t per)
{
    const uint32_t total = (uint32_t)(P * per), per32 = (uint32_t)per;
    for (uint32_t t = blockIdx.x * blockDim.x + threadIdx.x; t < total; t += gridDim.x * blockDim.x) {
        const uint32_t p = t / per32, r = t - p * per32;
        st(out, t, ld(a, p * astride + r) + ld(b, p * bstride + r));
    }
}

// Per-(channel, group) partial correlations of (scale[c] * dz) with a:
//   part[g][c][u*K+v] = sum over the group's planes of channel c of
//                       sum_ij s dz[i][j] a[i+u-R][j+v-R],  part[g][c][K*K] = sum s dz.
// Plane index = n * C + c; group g takes images g, g + G, ...
template <typename T, int K>
__global__ __launch_bounds__(kThreads) void k_corr(const T *dz, const float *scale, const T *a, float *part, int C,
                                                   int N, int G, int h, int w)
{
    constexpr int R = K / 2, KK = K * K, L1 = KK + 1;
    __shared__ float red[kThreads];
    const int c = blockIdx.x % C, g = blockIdx.x / C;
    const int64_t per = (int64_t)h * w;
    const float s = scale ? scale[c] : 1.0f;
    float acc[L1];
    for (int e = 0; e < L1; ++e) acc[e] = 0.0f;
    for (int n = g; n < N; n += G) {
        const T *dp = dz + ((int64_t)n * C + c) * per;
        const T *ap = a + ((int64_t)n * C + c) * per;
        for (int64_t r = threadIdx.x; r < per; r += blockDim.x) {
            const int i = (int)(r / w), j = (int)(r - (r / w) * w);
            const float d = s * ld(dp, r);
            acc[KK] += d;
            for (int u = 0; u < K; ++u) {
                const int ii = i + u - R;
                if (ii < 0 || ii >= h) continue;
                for (int v = 0; v < K; ++v) {
                    const int jj = j + v - R;
                    if (jj < 0 || jj >= w) continue;
                    acc[u * K + v] += d * ld(ap, (int64_t)ii * w + jj);
                }
            }
        }
    }
    // fixed-order tree reduction over the workgroup, one value at a time
    for (int e = 0; e < L1; ++e) {
        red[threadIdx.x] = acc[e];
        __syncthreads();
        for (int d = kThreads / 2; d > 0; d >>= 1) {
            if ((int)threadIdx.x < d) red[threadIdx.x] += red[threadIdx.x + d];
            __syncthreads();
        }
        if (threadIdx.x == 0) part[((int64_t)g * C + c) * L1 + e] = red[0];
        __syncthreads();
    }
}

// Sum the G partials in group order: out[c * K*K + e] (e < K*K) and, if
// outb, outb[c] = the sum of s dz.
__global__ void k_corr_reduce(const float *part, int C, int G, int KK, float *out, float *outb)
{
    const int L1 = KK + 1;
    for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < C * L1; t += gridDim.x * blockDim.x) {
        const int c = t / L1, e = t - c * L1;
        float sum = 0.0f;
        for (int g = 0; g < G; ++g) sum += part[((int64_t)g * C + c) * L1 + e];
        if (e < KK) {
            if (out) out[(int64_t)c * KK + e] = sum;
        } else if (outb) {
            outb[c] = sum;
        }
    }
}

// ---------------------------------------------------------------- host side

struct Layout {
    // element offsets (activation type) of every intermediate, per level l = 1..L
    int64_t Y[WTCONV_MAX_LEVELS + 1], Zc[WTCONV_MAX_LEVELS + 1], Zs[WTCONV_MAX_LEVELS + 1];
    int64_t A[WTCONV_MAX_LEVELS + 1], Nx[WTCONV_MAX_LEVELS + 1];
    int64_t Bc, Bs;
    // backward
    int64_t D[WTCONV_MAX_LEVELS + 1], Dz[WTCONV_MAX_LEVELS + 1], dY[WTCONV_MAX_LEVELS + 1];
    int64_t S[WTCONV_MAX_LEVELS + 1], Sa[WTCONV_MAX_LEVELS + 1], Db, Ds;
    int64_t elems;      // activation-type elements
    int64_t ones_off;   // byte offset of 4C floats of 1.0 (unit scales of the convolution steps)
    int64_t zw_off;     // byte offset of 4C k^2 zero weights (the correlation steps' unused scale term)
    int64_t sdb_off;    // byte offset of 2 x 4C scratch floats (their unused bias and scale outputs)
    int64_t fws_off;    // byte offset of the correlation steps' own workspace, fws_bytes long
    int64_t fws_bytes;
    int64_t part_off;   // byte offset of the float partials
    int64_t groups;
    size_t bytes;
};

int64_t plane_elems(const wtconv_desc_t *d, int l) { return (d->h >> l) * (d->w >> l); }

void make_layout(const wtconv_desc_t *d, Layout *L)
{
    const int64_t NC = d->n * d->c, E = NC * d->h * d->w;
    int64_t off = 0;
    auto take = [&](int64_t n) {
        const int64_t o = off;
        off += (n + 63) / 64 * 64;
        return o;
    };
    for (int l = 1; l <= d->levels; ++l) {
        const int64_t q = NC * plane_elems(d, l);
        L->Y[l] = take(4 * q);
        L->Zc[l] = take(4 * q);
        L->Zs[l] = take(4 * q);
        L->A[l] = take(q);
        L->Nx[l] = take(NC * plane_elems(d, l - 1));  // synthesis output, level l-1 resolution
        L->D[l] = take(4 * q);
        L->Dz[l] = take(4 * q);
        L->dY[l] = take(4 * q);
        L->S[l] = take(NC * plane_elems(d, l - 1));
        L->Sa[l] = take(q);
    }
    L->Bc = take(E);
    L->Bs = take(E);
    L->Db = take(E);
    L->Ds = take(E);
    L->elems = off;
    const int eb = d->dtype == WTCONV_F32 ? 4 : 2;
    L->groups = d->n < 16 ? d->n : 16;
    L->ones_off = (off * eb + 255) / 256 * 256;
    L->zw_off = L->ones_off + (4 * d->c * 4 + 255) / 256 * 256;
    L->sdb_off = L->zw_off + (4 * d->c * d->k * d->k * 4 + 255) / 256 * 256;
    L->fws_off = L->sdb_off + (2 * 4 * d->c * 4 + 255) / 256 * 256;
    // the correlation steps run the library's weight-gradient path at L = 0
    // (k x k for the weights, 1 x 1 for the scales) on every level's shape
    int64_t fws = 0;
    for (int l = 0; l <= d->levels; ++l) {
        for (int kk : {d->k, 1}) {
            const wtconv_desc_t cd{d->n, l == 0 ? d->c : 4 * d->c, d->h >> l, d->w >> l, kk, 0, d->dtype};
            size_t b = 0;
            if (wtconv_workspace_size(&cd, WTCONV_OP_BWD_WEIGHT, &b) == WTCONV_OK && (int64_t)b > fws) fws = (int64_t)b;
        }
    }
    L->fws_bytes = fws;
    L->part_off = L->fws_off + (fws + 255) / 256 * 256;
    const int64_t kk1 = (int64_t)d->k * d->k + 1;
    L->bytes = (size_t)(L->part_off + L->groups * 4 * d->c * kk1 * 4);
}

bool desc_ok(const wtconv_desc_t *d)
{
    if (!d || d->n < 1 || d->c < 1 || d->h < 1 || d->w < 1) return false;
    if (d->levels < 0 || d->levels > WTCONV_MAX_LEVELS) return false;
    if (d->h % ((int64_t)1 << d->levels) || d->w % ((int64_t)1 << d->levels)) return false;
    if (d->k != 1 && d->k != 3 && d->k != 5 && d->k != 7) return false;
    if (d->n * d->c * d->h * d->w >= ((int64_t)1 << 31)) return false;  // 32-bit element indexes
    return d->dtype == WTCONV_F32 || d->dtype == WTCONV_F16;
}

__global__ void k_fill(float *p, int n, float v)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = v;
}

// One convolution step: the library's own depthwise convolution (the layer at
// L = 0 with unit scales: wtconv_forward / wtconv_backward_data), so that the
// baseline's convolutions are as fast as the fused path's; the plain kernel
// above if that call declines the shape.
template <typename T>
void dwconv(int k, const T *in, T *out, const float *wt, const float *bias, const float *ones, int C, int64_t P,
            int h, int w, int rotate, hipStream_t s)
{
    const wtconv_desc_t cd{P / C, C, h, w, k, 0, sizeof(T) == 4 ? WTCONV_F32 : WTCONV_F16};
    const wtconv_status_t st = rotate ? wtconv_backward_data(&cd, in, wt, ones, nullptr, nullptr, out, nullptr, 0, s)
                                      : wtconv_forward(&cd, in, wt, bias, ones, nullptr, nullptr, out, nullptr, 0, s);
    if (st == WTCONV_OK) return;
    const unsigned g = grid_for(P * h * w);
    switch (k) {
    case 1: hipLaunchKernelGGL((k_dwconv<T, 1>), dim3(g), dim3(kThreads), 0, s, in, out, wt, bias, C, P, h, w, rotate); break;
    case 3: hipLaunchKernelGGL((k_dwconv<T, 3>), dim3(g), dim3(kThreads), 0, s, in, out, wt, bias, C, P, h, w, rotate); break;
    case 5: hipLaunchKernelGGL((k_dwconv<T, 5>), dim3(g), dim3(kThreads), 0, s, in, out, wt, bias, C, P, h, w, rotate); break;
    default: hipLaunchKernelGGL((k_dwconv<T, 7>), dim3(g), dim3(kThreads), 0, s, in, out, wt, bias, C, P, h, w, rotate); break;
    }
}

template <typename T>
void corr(int k, const T *dz, const float *scale, const T *a, float *part, int C, int N, int G, int h, int w,
                float *out, float *outb, hipStream_t s);

// One correlation step through the library's weight-gradient path at L = 0
// with unit scales and zero weights: dw = G (the k x k correlation of dz with
// a), db = sum dz.  dz must already carry its scale.  Falls back to the plain
// kernel above if that call declines the shape.
template <typename T>
void corr_lib(int k, const T *dz, const T *a, const Layout &L, T *ws, float *part, int C, int N, int G, int h, int w,
              float *out, float *outb, hipStream_t s)
{
    char *base = (char *)ws;
    float *ones = (float *)(base + L.ones_off), *zw = (float *)(base + L.zw_off), *sdb = (float *)(base + L.sdb_off);
    const wtconv_desc_t cd{N, C, h, w, k, 0, sizeof(T) == 4 ? WTCONV_F32 : WTCONV_F16};
    const wtconv_status_t st =
        wtconv_backward_weight(&cd, a, dz, zw, nullptr, ones, nullptr, nullptr, out, outb ? outb : sdb, sdb + C,
                               nullptr, nullptr, base + L.fws_off, (size_t)L.fws_bytes, s);
    if (st != WTCONV_OK) corr<T>(k, dz, nullptr, a, part, C, N, G, h, w, out, outb, s);
}

template <typename T>
void corr(int k, const T *dz, const float *scale, const T *a, float *part, int C, int N, int G, int h, int w,
                float *out, float *outb, hipStream_t s)
{
    const dim3 grid((unsigned)(C * G));
    switch (k) {
    case 1: hipLaunchKernelGGL((k_corr<T, 1>), grid, dim3(kThreads), 0, s, dz, scale, a, part, C, N, G, h, w); break;
    case 3: hipLaunchKernelGGL((k_corr<T, 3>), grid, dim3(kThreads), 0, s, dz, scale, a, part, C, N, G, h, w); break;
    case 5: hipLaunchKernelGGL((k_corr<T, 5>), grid, dim3(kThreads), 0, s, dz, scale, a, part, C, N, G, h, w); break;
    default: hipLaunchKernelGGL((k_corr<T, 7>), grid, dim3(kThreads), 0, s, dz, scale, a, part, C, N, G, h, w); break;
    }
    hipLaunchKernelGGL(k_corr_reduce, dim3((unsigned)((C * (k * k + 1) + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       s, part, C, G, k * k, out, outb);
}

template <typename T>
wtconv_status_t forward_t(const wtconv_desc_t *d, const T *x, const float *w0, const float *b0, const float *s0,
                          const float *wl, const float *sl, T *y, T *ws, hipStream_t s)
{
    Layout L;
    make_layout(d, &L);
    const int C = (int)d->c, k = d->k, Lv = d->levels;
    const int64_t NC = d->n * d->c, kk = (int64_t)k * k;
    float *ones = (float *)((char *)ws + L.ones_off);
    hipLaunchKernelGGL(k_fill, dim3(1), dim3(kThreads), 0, s, ones, 4 * C, 1.0f);
    for (int l = 1; l <= Lv; ++l) {
        const int h = (int)(d->h >> (l - 1)), w = (int)(d->w >> (l - 1));
        const int64_t q = NC * plane_elems(d, l);
        const T *src = l == 1 ? x : ws + L.Y[l - 1];
        const int64_t istride = l == 1 ? (int64_t)h * w : 4 * (int64_t)h * w;
        hipLaunchKernelGGL(k_analysis<T>, dim3(grid_for(q)), dim3(kThreads), 0, s, src, istride, ws + L.Y[l],
                           4 * plane_elems(d, l), NC, h, w);
        dwconv<T>(k, ws + L.Y[l], ws + L.Zc[l], wl + (int64_t)(l - 1) * 4 * C * kk, nullptr, ones, 4 * C, 4 * NC,
                  h / 2, w / 2, 0, s);
        hipLaunchKernelGGL(k_scale_add<T>, dim3(grid_for(4 * q)), dim3(kThreads), 0, s, ws + L.Zc[l],
                           sl + (int64_t)(l - 1) * 4 * C, (const T *)nullptr, ws + L.Zs[l], 4 * C, 4 * NC,
                           plane_elems(d, l));
    }
    for (int l = Lv; l >= 1; --l) {
        const int h = (int)(d->h >> l), w = (int)(d->w >> l);
        const int64_t per = plane_elems(d, l);
        if (l == Lv) {
            // A_L = band 0 of Zs_L (nothing below to add): the synthesis reads it in place
            hipLaunchKernelGGL(k_synthesis<T>, dim3(grid_for(NC * per)), dim3(kThreads), 0, s, ws + L.Zs[l], 4 * per,
                               ws + L.Zs[l], 4 * per, ws + L.Nx[l], NC, h, w);
        } else {
            hipLaunchKernelGGL(k_add_strided<T>, dim3(grid_for(NC * per)), dim3(kThreads), 0, s, ws + L.Zs[l],
                               4 * per, ws + L.Nx[l + 1], per, ws + L.A[l], NC, per);
            hipLaunchKernelGGL(k_synthesis<T>, dim3(grid_for(NC * per)), dim3(kThreads), 0, s, ws + L.A[l], per,
                               ws + L.Zs[l], 4 * per, ws + L.Nx[l], NC, h, w);
        }
    }
    const int64_t E = NC * d->h * d->w, hw = d->h * d->w;
    dwconv<T>(k, x, ws + L.Bc, w0, b0, ones, C, NC, (int)d->h, (int)d->w, 0, s);
    hipLaunchKernelGGL(k_scale_add<T>, dim3(grid_for(E)), dim3(kThreads), 0, s, ws + L.Bc, s0,
                       Lv ? (const T *)(ws + L.Nx[1]) : (const T *)nullptr, y, C, NC, hw);
    return hipGetLastError() == hipSuccess ? WTCONV_OK : WTCONV_ERR_HIP;
}

// Reverse mode of the wavelet branch down to the dy-side bands D_l, the
// gradients of the scaled band outputs Zs_l.  (Launch errors are collected by
// the hipGetLastError at the end of each entry point.)
template <typename T>
void wavelet_adjoint_bands(const wtconv_desc_t *d, const Layout &L, const T *dy, T *ws, hipStream_t s)
{
    const int64_t NC = d->n * d->c;
    for (int l = 1; l <= d->levels; ++l) {
        const int h = (int)(d->h >> (l - 1)), w = (int)(d->w >> (l - 1));
        const T *src = l == 1 ? dy : ws + L.D[l - 1];
        const int64_t istride = l == 1 ? (int64_t)h * w : 4 * (int64_t)h * w;
        hipLaunchKernelGGL(k_analysis<T>, dim3(grid_for(NC * plane_elems(d, l))), dim3(kThreads), 0, s, src, istride,
                           ws + L.D[l], 4 * plane_elems(d, l), NC, h, w);
    }
}

template <typename T>
wtconv_status_t backward_data_t(const wtconv_desc_t *d, const T *dy, const float *w0, const float *s0,
                                const float *wl, const float *sl, T *dx, T *ws, hipStream_t s)
{
    Layout L;
    make_layout(d, &L);
    const int C = (int)d->c, k = d->k, Lv = d->levels;
    const int64_t NC = d->n * d->c, kk = (int64_t)k * k;
    float *ones = (float *)((char *)ws + L.ones_off);
    hipLaunchKernelGGL(k_fill, dim3(1), dim3(kThreads), 0, s, ones, 4 * C, 1.0f);
    wavelet_adjoint_bands<T>(d, L, dy, ws, s);
    for (int l = 1; l <= Lv; ++l) {
        const int64_t per = plane_elems(d, l);
        hipLaunchKernelGGL(k_scale_add<T>, dim3(grid_for(4 * NC * per)), dim3(kThreads), 0, s, ws + L.D[l],
                           sl + (int64_t)(l - 1) * 4 * C, (const T *)nullptr, ws + L.Dz[l], 4 * C, 4 * NC, per);
        dwconv<T>(k, ws + L.Dz[l], ws + L.dY[l], wl + (int64_t)(l - 1) * 4 * C * kk, nullptr, ones, 4 * C, 4 * NC,
                  (int)(d->h >> l), (int)(d->w >> l), 1, s);
    }
    // from the deepest level up: the low-pass band of dY_l also receives the
    // synthesis of level l+1's gradient; S_l = synthesis(dY_l) is the gradient
    // of LL_{l-1}
    for (int l = Lv; l >= 1; --l) {
        const int h = (int)(d->h >> l), w = (int)(d->w >> l);
        const int64_t per = plane_elems(d, l);
        if (l == Lv) {
            hipLaunchKernelGGL(k_synthesis<T>, dim3(grid_for(NC * per)), dim3(kThreads), 0, s, ws + L.dY[l], 4 * per,
                               ws + L.dY[l], 4 * per, ws + L.S[l], NC, h, w);
        } else {
            hipLaunchKernelGGL(k_add_strided<T>, dim3(grid_for(NC * per)), dim3(kThreads), 0, s, ws + L.dY[l],
                               4 * per, ws + L.S[l + 1], per, ws + L.Sa[l], NC, per);
            hipLaunchKernelGGL(k_synthesis<T>, dim3(grid_for(NC * per)), dim3(kThreads), 0, s, ws + L.Sa[l], per,
                               ws + L.dY[l], 4 * per, ws + L.S[l], NC, h, w);
        }
    }
    const int64_t E = NC * d->h * d->w, hw = d->h * d->w;
    hipLaunchKernelGGL(k_scale_add<T>, dim3(grid_for(E)), dim3(kThreads), 0, s, dy, s0, (const T *)nullptr,
                       ws + L.Ds, C, NC, hw);
    dwconv<T>(k, ws + L.Ds, Lv ? ws + L.Db : dx, w0, nullptr, ones, C, NC, (int)d->h, (int)d->w, 1, s);
    if (Lv)
        hipLaunchKernelGGL(k_scale_add<T>, dim3(grid_for(E)), dim3(kThreads), 0, s, ws + L.Db, (const float *)nullptr,
                           (const T *)(ws + L.S[1]), dx, C, NC, hw);
    return hipGetLastError() == hipSuccess ? WTCONV_OK : WTCONV_ERR_HIP;
}

template <typename T>
wtconv_status_t backward_weight_t(const wtconv_desc_t *d, const T *x, const T *dy, const float *s0,
                                  const float *sl, float *dw0, float *db0, float *ds0, float *dwl, float *dsl, T *ws,
                                  hipStream_t s)
{
    Layout L;
    make_layout(d, &L);
    const int C = (int)d->c, k = d->k, Lv = d->levels, N = (int)d->n, G = (int)L.groups;
    const int64_t kk = (int64_t)k * k;
    float *part = (float *)((char *)ws + L.part_off);
    const int64_t NC = d->n * d->c;
    hipLaunchKernelGGL(k_fill, dim3(1), dim3(kThreads), 0, s, (float *)((char *)ws + L.ones_off), 4 * C, 1.0f);
    hipLaunchKernelGGL(k_fill, dim3(4), dim3(kThreads), 0, s, (float *)((char *)ws + L.zw_off), (int)(4 * C * kk),
                       0.0f);
    wavelet_adjoint_bands<T>(d, L, dy, ws, s);
    for (int l = 1; l <= Lv; ++l) {
        const int h = (int)(d->h >> l), w = (int)(d->w >> l);
        const int64_t per = plane_elems(d, l);
        // dW_l = corr(s_l D_l, Y_l) (the scale backward, then the convolution's
        // weight gradient); ds_l = <D_l, Zc_l>
        hipLaunchKernelGGL(k_scale_add<T>, dim3(grid_for(4 * NC * per)), dim3(kThreads), 0, s, ws + L.D[l],
                           sl + (int64_t)(l - 1) * 4 * C, (const T *)nullptr, ws + L.Dz[l], 4 * C, 4 * NC, per);
        corr_lib<T>(k, ws + L.Dz[l], ws + L.Y[l], L, ws, part, 4 * C, N, G, h, w,
                    dwl + (int64_t)(l - 1) * 4 * C * kk, nullptr, s);
        corr_lib<T>(1, ws + L.D[l], ws + L.Zc[l], L, ws, part, 4 * C, N, G, h, w, dsl + (int64_t)(l - 1) * 4 * C,
                    nullptr, s);
    }
    // base: dW0 = corr(s0 dy, x), db0 = sum s0 dy, ds0 = <dy, Bc> (Bc = W0 (*) x + b0)
    const int64_t E = NC * d->h * d->w;
    hipLaunchKernelGGL(k_scale_add<T>, dim3(grid_for(E)), dim3(kThreads), 0, s, dy, s0, (const T *)nullptr, ws + L.Ds,
                       C, NC, d->h * d->w);
    corr_lib<T>(k, ws + L.Ds, x, L, ws, part, C, N, G, (int)d->h, (int)d->w, dw0, db0, s);
    corr_lib<T>(1, dy, ws + L.Bc, L, ws, part, C, N, G, (int)d->h, (int)d->w, ds0, nullptr, s);
    return hipGetLastError() == hipSuccess ? WTCONV_OK : WTCONV_ERR_HIP;
}

}  // namespace

extern "C" {

wtconv_status_t wtconv_unfused_workspace_size(const wtconv_desc_t *desc, size_t *bytes)
{
    if (!bytes) return WTCONV_ERR_NULL;
    if (!desc_ok(desc)) return WTCONV_ERR_SHAPE;
    Layout L;
    make_layout(desc, &L);
    *bytes = L.bytes;
    return WTCONV_OK;
}

wtconv_status_t wtconv_unfused_forward(const wtconv_desc_t *desc, const void *x, const float *w_base,
                                       const float *bias, const float *s_base, const float *w_lvl,
                                       const float *s_lvl, void *y, void *workspace, size_t workspace_bytes,
                                       wtconv_stream_t stream)
{
    if (!desc_ok(desc)) return WTCONV_ERR_SHAPE;
    if (!x || !y || !w_base || !s_base || !workspace || (desc->levels && (!w_lvl || !s_lvl))) return WTCONV_ERR_NULL;
    Layout L;
    make_layout(desc, &L);
    if (workspace_bytes < L.bytes) return WTCONV_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (desc->dtype == WTCONV_F32)
        return forward_t<float>(desc, (const float *)x, w_base, bias, s_base, w_lvl, s_lvl, (float *)y,
                                (float *)workspace, s);
    return forward_t<_Float16>(desc, (const _Float16 *)x, w_base, bias, s_base, w_lvl, s_lvl, (_Float16 *)y,
                               (_Float16 *)workspace, s);
}

wtconv_status_t wtconv_unfused_backward_data(const wtconv_desc_t *desc, const void *dy, const float *w_base,
                                             const float *s_base, const float *w_lvl, const float *s_lvl, void *dx,
                                             void *workspace, size_t workspace_bytes, wtconv_stream_t stream)
{
    if (!desc_ok(desc)) return WTCONV_ERR_SHAPE;
    if (!dy || !dx || !w_base || !s_base || !workspace || (desc->levels && (!w_lvl || !s_lvl))) return WTCONV_ERR_NULL;
    Layout L;
    make_layout(desc, &L);
    if (workspace_bytes < L.bytes) return WTCONV_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (desc->dtype == WTCONV_F32)
        return backward_data_t<float>(desc, (const float *)dy, w_base, s_base, w_lvl, s_lvl, (float *)dx,
                                      (float *)workspace, s);
    return backward_data_t<_Float16>(desc, (const _Float16 *)dy, w_base, s_base, w_lvl, s_lvl, (_Float16 *)dx,
                                     (_Float16 *)workspace, s);
}

wtconv_status_t wtconv_unfused_backward_weight(const wtconv_desc_t *desc, const void *x, const void *dy,
                                               const float *w_base, const float *bias, const float *s_base,
                                               const float *w_lvl, const float *s_lvl, float *dw_base,
                                               float *dbias, float *ds_base, float *dw_lvl, float *ds_lvl,
                                               void *workspace, size_t workspace_bytes, wtconv_stream_t stream)
{
    (void)w_base;
    (void)bias;
    (void)w_lvl;
    if (!desc_ok(desc)) return WTCONV_ERR_SHAPE;
    if (!x || !dy || !s_base || !dw_base || !dbias || !ds_base || !workspace) return WTCONV_ERR_NULL;
    if (desc->levels && (!s_lvl || !dw_lvl || !ds_lvl)) return WTCONV_ERR_NULL;
    Layout L;
    make_layout(desc, &L);
    if (workspace_bytes < L.bytes) return WTCONV_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    if (desc->dtype == WTCONV_F32)
        return backward_weight_t<float>(desc, (const float *)x, (const float *)dy, s_base, s_lvl, dw_base, dbias,
                                        ds_base, dw_lvl, ds_lvl, (float *)workspace, s);
    return backward_weight_t<_Float16>(desc, (const _Float16 *)x, (const _Float16 *)dy, s_base, s_lvl, dw_base,
                                       dbias, ds_base, dw_lvl, ds_lvl, (_Float16 *)workspace, s);
}

}  // extern "C"
