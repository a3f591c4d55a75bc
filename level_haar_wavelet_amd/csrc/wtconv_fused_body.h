// wtconv_fused_body.h -- the fused WTConv forward (and data backward) pass of
// one workgroup, written as a sequence of phases separated by workgroup
// barriers.  The kernel in wtconv_fused.hip runs the phases with
// __syncthreads() between them; a CPU emulation (tests) runs every thread of a
// phase in turn, with bounds checks on every LDS and global access.
//
// Source: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation" (arXiv 2608.10805), technical summary, Methodology:
//   reformulation 1 -- the Haar analysis (signed additions and power-of-two
//     scalings) is recomputed on chip instead of writing the subband tensor;
//   reformulation 2 -- the synthesis cascade is replaced by a closed-form sum in
//     which an output pixel takes each level's coefficient at its coordinates
//     shifted right by the level, with a sign given by the parity of the
//     coordinate bits;
//   reformulation 3 -- the per-channel scales are folded into the weights (and
//     the base scale into the bias).
//
// Arithmetic used here (all fp32):
//   U_0 = x, U_m = plain 2x2 sum of U_{m-1}     (so the orthonormal low-pass
//                                                band is 2^-m U_m)
//   B_m^b = plain signed 2x2 sums of U_{m-1}    (orthonormal band A = 2^-m B)
//   W''_m^b = 4^-m s_m^b W_m^b                  (folded weight; the two 2^-m
//                                                factors of analysis and
//                                                synthesis are exact)
//   Z_m^b = W''_m^b (*) B_m^b
//   y[h,w] = s0 W0 (*) x + s0 b0 + sum_m sum_b sign_b(p_m, q_m) Z_m^b[h>>m, w>>m]
//   with p_m = bit (m-1) of h, q_m = bit (m-1) of w, sign = +1, (-1)^p, (-1)^q,
//   (-1)^(p+q) for b = 0..3.
// Level 1 is evaluated per 2x2 output block as a butterfly (the same signs for
// its four pixels); levels >= 2 are constant over the block and summed first.
#ifndef WTCONV_FUSED_BODY_H
#define WTCONV_FUSED_BODY_H

#include "wtconv_plan.h"

#ifdef WTC_EMULATE
#include <cassert>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#define WTC_HD
#define WTC_INLINE inline
static inline float wtc_fma(float a, float b, float c) { return fmaf(a, b, c); }
static inline float wtc_uniform(float v) { return v; }
// product of two non-negative ints below 2^23 (LDS and in-plane indexes)
static inline int wtc_mul24(int a, int b)
{
    assert(a >= 0 && b >= 0 && a < (1 << 23) && b < (1 << 23));
    return a * b;
}
template <typename P>
static inline P &wtc_chk(P *base, int64_t i, int64_t n, int line)
{
    if (i < 0 || i >= n) {
        fprintf(stderr, "wtconv emulation: index %lld outside [0, %lld) at line %d\n", (long long)i, (long long)n,
                line);
        abort();
    }
    return base[i];
}
#define WTC_LDS(ctx, i) wtc_chk((ctx).lds, (int64_t)(i), (ctx).lds_n, __LINE__)
#define WTC_IN(ctx, i) wtc_chk((ctx).in, (int64_t)(i), (ctx).plane_n, __LINE__)
#define WTC_OUT(ctx, i) wtc_chk((ctx).out, (int64_t)(i), (ctx).plane_n, __LINE__)
#define WTC_PAR(ptr, i, n) wtc_chk((ptr), (int64_t)(i), (int64_t)(n), __LINE__)
#else
#include <hip/hip_runtime.h>
#define WTC_HD __device__
#define WTC_INLINE __forceinline__
static __device__ __forceinline__ float wtc_fma(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
// Product of two non-negative ints below 2^23 (LDS and in-plane indexes):
// the full-rate 24-bit multiply instead of the quarter-rate 32-bit one.
static __device__ __forceinline__ int wtc_mul24(int a, int b) { return __mul24(a, b); }
// A value that is the same in every lane, moved to a scalar register.
static __device__ __forceinline__ float wtc_uniform(float v)
{
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
#define WTC_LDS(ctx, i) ((ctx).lds[(i)])
#define WTC_IN(ctx, i) ((ctx).in[(i)])
#define WTC_OUT(ctx, i) ((ctx).out[(i)])
#define WTC_PAR(ptr, i, n) ((ptr)[(i)])
#endif

template <typename T>
WTC_HD WTC_INLINE float wtc_to_float(T v)
{
    return (float)v;
}
template <typename T>
WTC_HD WTC_INLINE T wtc_from_float(float v)
{
    return (T)v;  // fp16: round to nearest even
}

template <typename T>
struct WtcFusedArgs {
    const T *in;       // x (forward) or dy (data backward), NCHW
    T *out;            // y or dx
    const float *w_base, *bias, *s_base, *w_lvl, *s_lvl;
    WtcFusedPlan p;
};

// Per-thread view of one workgroup's work.
template <typename T>
struct WtcCtx {
    float *lds;
    const T *in;  // this plane
    T *out;       // this plane
    int tid, nth;
    int c;               // channel
    int ty0, tx0;        // tile origin (full resolution)
    float bias;          // folded bias of the channel (0 for the data backward)
#ifdef WTC_EMULATE
    int64_t lds_n, plane_n;
#endif
};

// Geometry of level m for the current tile.
struct WtcLvl {
    int H, W;          // map size
    int t0y, t0x;      // tile origin at level m
    int t1y, t1x;      // tile end at level m
    int oy, ox;        // origin of the low-pass map region in LDS
    int ey, ex;        // end of the low-pass map region
};

WTC_HD WTC_INLINE WtcLvl wtc_level(const WtcFusedPlan &p, int m, int ty0, int tx0)
{
    WtcLvl g;
    const int r = p.k / 2;
    g.H = p.h >> m;
    g.W = p.w >> m;
    g.t0y = ty0 >> m;
    g.t0x = tx0 >> m;
    g.t1y = (ty0 + p.tile_h) >> m;
    g.t1x = (tx0 + p.tile_w) >> m;
    const int hal = wtc_halo(r, p.levels, m);
    g.oy = wtc_max(g.t0y - hal, -r);
    g.ox = wtc_max(g.t0x - hal, -r);
    g.ey = wtc_min(g.t1y + hal, g.H + r);
    g.ex = wtc_min(g.t1x + hal, g.W + r);
    return g;
}

// Workgroup -> (plane, tile).  Workgroups are dealt to the 8 XCDs round-robin;
// when a plane has several tiles the index is permuted so that the tiles of a
// plane run on one XCD and share its L2 (their halos overlap).
WTC_HD WTC_INLINE void wtc_wg_to_tile(const WtcFusedPlan &p, int bid, int nblocks, int *plane, int *tile)
{
    const int ntiles = p.tiles_y * p.tiles_x;
    int id = bid;
    if (ntiles > 1 && nblocks % 8 == 0) id = (bid % 8) * (nblocks / 8) + bid / 8;
    *plane = id / ntiles;
    *tile = id % ntiles;
}

template <typename T>
WTC_HD WTC_INLINE void wtc_fused_setup(const WtcFusedArgs<T> &a, WtcCtx<T> &ctx, int bid, int nblocks)
{
    const WtcFusedPlan &p = a.p;
    int plane, tile;
    wtc_wg_to_tile(p, bid, nblocks, &plane, &tile);
    ctx.c = plane % p.c;
    ctx.ty0 = (tile / p.tiles_x) * p.tile_h;
    ctx.tx0 = (tile % p.tiles_x) * p.tile_w;
    const int64_t hw = (int64_t)p.h * p.w;
    ctx.in = a.in + (int64_t)plane * hw;
    ctx.out = a.out + (int64_t)plane * hw;
    float b = 0.0f;
    if (!p.rotate && a.bias) b = a.s_base[ctx.c] * a.bias[ctx.c];
    ctx.bias = b;
}

// Phase 0: folded weights of the channel into LDS.
//   base:    s0 * W0          level m band b: 4^-m * s_m^b * W_m^b
// For the data backward every kernel is turned by 180 degrees.
template <typename T, int K>
WTC_HD WTC_INLINE void wtc_phase_fold(const WtcFusedArgs<T> &a, WtcCtx<T> &ctx)
{
    const WtcFusedPlan &p = a.p;
    constexpr int kk = K * K;
    const int total = (1 + 4 * p.levels) * kk;
    const int C = p.c, c = ctx.c;
    for (int i = ctx.tid; i < total; i += ctx.nth) {
        const int blk = i / kk, e = i % kk;
        const int se = p.rotate ? (kk - 1 - e) : e;
        float v;
        if (blk == 0) {
            v = WTC_PAR(a.s_base, c, C) * WTC_PAR(a.w_base, c * kk + se, (int64_t)C * kk);
        } else {
            const int m = (blk - 1) / 4 + 1, b = (blk - 1) % 4;
            const int ch = (m - 1) * 4 * C + 4 * c + b;
            const float s = WTC_PAR(a.s_lvl, ch, (int64_t)p.levels * 4 * C);
            v = s * WTC_PAR(a.w_lvl, (int64_t)ch * kk + se, (int64_t)p.levels * 4 * C * kk);
            v = ldexpf(v, -2 * m);
        }
        WTC_LDS(ctx, p.wf_off + i) = v;
    }
}

// Phase 1: the level-1 low-pass map U_1 over the tile plus its halo, read
// straight from the input (zero outside the level-1 map).
template <typename T, int K>
WTC_HD WTC_INLINE void wtc_phase_coarse(const WtcFusedArgs<T> &a, WtcCtx<T> &ctx)
{
    const WtcFusedPlan &p = a.p;
    const WtcLvl g = wtc_level(p, 1, ctx.ty0, ctx.tx0);
    const int rows = g.ey - g.oy, cols = g.ex - g.ox;
    const int W = p.w;
    const WtcMap mp = p.ll[1];
    for (int idx = ctx.tid; idx < rows * cols; idx += ctx.nth) {
        const int ri = idx / cols, ci = idx - ri * cols;
        const int i = g.oy + ri, j = g.ox + ci;
        float v = 0.0f;
        if (i >= 0 && i < g.H && j >= 0 && j < g.W) {
            const int64_t o = (int64_t)(2 * i) * W + 2 * j;
            const float x00 = wtc_to_float(WTC_IN(ctx, o)), x01 = wtc_to_float(WTC_IN(ctx, o + 1));
            const float x10 = wtc_to_float(WTC_IN(ctx, o + W)), x11 = wtc_to_float(WTC_IN(ctx, o + W + 1));
            v = (x00 + x01) + (x10 + x11);
        }
        WTC_LDS(ctx, mp.off + ri * mp.pitch + ci) = v;
    }
}

// Phase 2 (m = 2..L): U_m over its region and the detail bands B_m^1..3 over the
// tile plus r, from U_{m-1} in LDS (zero outside the level-m map).
template <typename T, int K>
WTC_HD WTC_INLINE void wtc_phase_deep_level(const WtcFusedArgs<T> &a, WtcCtx<T> &ctx, int m)
{
    constexpr int R = K / 2;
    const WtcFusedPlan &p = a.p;
    const WtcLvl g = wtc_level(p, m, ctx.ty0, ctx.tx0);
    const WtcLvl gp = wtc_level(p, m - 1, ctx.ty0, ctx.tx0);
    const WtcMap src = p.ll[m - 1], dl = p.ll[m], db = p.band[m];
    const int rows = g.ey - g.oy, cols = g.ex - g.ox;
    for (int idx = ctx.tid; idx < rows * cols; idx += ctx.nth) {
        const int ri = idx / cols, ci = idx - ri * cols;
        const int i = g.oy + ri, j = g.ox + ci;
        float v = 0.0f;
        if (i >= 0 && i < g.H && j >= 0 && j < g.W) {
            const int s = src.off + (2 * i - gp.oy) * src.pitch + (2 * j - gp.ox);
            v = (WTC_LDS(ctx, s) + WTC_LDS(ctx, s + 1)) + (WTC_LDS(ctx, s + src.pitch) + WTC_LDS(ctx, s + src.pitch + 1));
        }
        WTC_LDS(ctx, dl.off + ri * dl.pitch + ci) = v;
    }
    const int brows = (g.t1y - g.t0y) + 2 * R, bcols = (g.t1x - g.t0x) + 2 * R;
    const int bstride = db.rows * db.pitch;
    for (int idx = ctx.tid; idx < brows * bcols; idx += ctx.nth) {
        const int ri = idx / bcols, ci = idx - ri * bcols;
        const int i = g.t0y - R + ri, j = g.t0x - R + ci;
        float b1 = 0.0f, b2 = 0.0f, b3 = 0.0f;
        if (i >= 0 && i < g.H && j >= 0 && j < g.W) {
            const int s = src.off + (2 * i - gp.oy) * src.pitch + (2 * j - gp.ox);
            const float x00 = WTC_LDS(ctx, s), x01 = WTC_LDS(ctx, s + 1);
            const float x10 = WTC_LDS(ctx, s + src.pitch), x11 = WTC_LDS(ctx, s + src.pitch + 1);
            const float sa = x00 + x01, sc = x10 + x11, da = x00 - x01, dc = x10 - x11;
            b1 = sa - sc;
            b2 = da + dc;
            b3 = da - dc;
        }
        const int o = db.off + ri * db.pitch + ci;
        WTC_LDS(ctx, o) = b1;
        WTC_LDS(ctx, o + bstride) = b2;
        WTC_LDS(ctx, o + 2 * bstride) = b3;
    }
}

// A PR x PC block of k x k cross-correlation outputs from an LDS map.
// src: LDS index of the input at (first output row - R, first output column - R).
// wk:  LDS index of the k x k weights.
template <typename T, int K, int PR, int PC>
WTC_HD WTC_INLINE void wtc_conv_block_lds(WtcCtx<T> &ctx, int src, int pitch, int wk, float (&acc)[PR][PC])
{
    float wr[K * K];
#pragma unroll
    for (int e = 0; e < K * K; ++e) wr[e] = WTC_LDS(ctx, wk + e);
#pragma unroll
    for (int t = 0; t < PR + K - 1; ++t) {
        float row[PC + K - 1];
#pragma unroll
        for (int e = 0; e < PC + K - 1; ++e) row[e] = WTC_LDS(ctx, src + t * pitch + e);
#pragma unroll
        for (int dr = 0; dr < PR; ++dr) {
            const int u = t - dr;
            if (u < 0 || u >= K) continue;
#pragma unroll
            for (int v = 0; v < K; ++v)
#pragma unroll
                for (int dc = 0; dc < PC; ++dc) acc[dr][dc] = wtc_fma(wr[u * K + v], row[dc + v], acc[dr][dc]);
        }
    }
}

// Phase 3: convolutions of the deep levels m = 2..L, all four bands, over the
// tile, into the Z maps.  Work is split into WTC_PR x WTC_PC pieces; the last
// piece of a row or column may hang over the map and its extra outputs are
// dropped.
template <typename T, int K>
WTC_HD WTC_INLINE void wtc_phase_deep_conv(const WtcFusedArgs<T> &a, WtcCtx<T> &ctx)
{
    constexpr int R = K / 2, kk = K * K;
    const WtcFusedPlan &p = a.p;
    int total = 0;
    for (int m = 2; m <= p.levels; ++m) {
        const int THm = p.tile_h >> m, TWm = p.tile_w >> m;
        total += 4 * ((THm + WTC_PR - 1) / WTC_PR) * ((TWm + WTC_PC - 1) / WTC_PC);
    }
    for (int pi = ctx.tid; pi < total; pi += ctx.nth) {
        int m = 2, rem = pi, npr = 0, npc = 0;
        for (; m <= p.levels; ++m) {
            npr = ((p.tile_h >> m) + WTC_PR - 1) / WTC_PR;
            npc = ((p.tile_w >> m) + WTC_PC - 1) / WTC_PC;
            if (rem < 4 * npr * npc) break;
            rem -= 4 * npr * npc;
        }
        const int b = rem / (npr * npc);
        rem -= b * npr * npc;
        const int pr = rem / npc, pc = rem - pr * npc;
        const WtcLvl g = wtc_level(p, m, ctx.ty0, ctx.tx0);
        const int i0 = g.t0y + WTC_PR * pr, j0 = g.t0x + WTC_PC * pc;
        int src, pitch;
        if (b == 0) {
            const WtcMap mp = p.ll[m];
            pitch = mp.pitch;
            src = mp.off + (i0 - R - g.oy) * pitch + (j0 - R - g.ox);
        } else {
            const WtcMap mp = p.band[m];
            pitch = mp.pitch;
            src = mp.off + (b - 1) * mp.rows * pitch + (i0 - R - (g.t0y - R)) * pitch + (j0 - R - (g.t0x - R));
        }
        float acc[WTC_PR][WTC_PC];
#pragma unroll
        for (int dr = 0; dr < WTC_PR; ++dr)
#pragma unroll
            for (int dc = 0; dc < WTC_PC; ++dc) acc[dr][dc] = 0.0f;
        wtc_conv_block_lds<T, K, WTC_PR, WTC_PC>(ctx, src, pitch, p.wf_off + (1 + 4 * (m - 1) + b) * kk, acc);
        const WtcMap zm = p.z[m];
        const int zb = zm.off + b * zm.rows * zm.pitch;
#pragma unroll
        for (int dr = 0; dr < WTC_PR; ++dr)
#pragma unroll
            for (int dc = 0; dc < WTC_PC; ++dc) {
                const int i = i0 + dr, j = j0 + dc;
                if (i < g.t1y && j < g.t1x) WTC_LDS(ctx, zb + (i - g.t0y) * zm.pitch + (j - g.t0x)) = acc[dr][dc];
            }
    }
}

// Phase 4a: stage the input rows [s0 - 2R, s0 + TS + 2R) x columns
// [tx0 - 2R, tx0 + TW + 2R) of the tile's strip (zero outside the image).
template <typename T, int K>
WTC_HD WTC_INLINE void wtc_phase_stage(const WtcFusedArgs<T> &a, WtcCtx<T> &ctx, int s0)
{
    constexpr int R = K / 2;
    const WtcFusedPlan &p = a.p;
    const int rows = p.strip_h + 4 * R, cols = p.tile_w + 4 * R;
    const WtcMap xs = p.xs;
    for (int idx = ctx.tid; idx < rows * cols; idx += ctx.nth) {
        const int ri = idx / cols, ci = idx - ri * cols;
        const int hh = s0 - 2 * R + ri, ww = ctx.tx0 - 2 * R + ci;
        float v = 0.0f;
        if (hh >= 0 && hh < p.h && ww >= 0 && ww < p.w) v = wtc_to_float(WTC_IN(ctx, (int64_t)hh * p.w + ww));
        WTC_LDS(ctx, xs.off + ri * xs.pitch + ci) = v;
    }
}

// Phase 4b: level-1 detail bands B_1^1..3 of the strip plus R level-1 pixels
// around it, from the staged strip (zero outside the level-1 map).
template <typename T, int K>
WTC_HD WTC_INLINE void wtc_phase_strip_bands(const WtcFusedArgs<T> &a, WtcCtx<T> &ctx, int s0)
{
    constexpr int R = K / 2;
    const WtcFusedPlan &p = a.p;
    const int H1 = p.h >> 1, W1 = p.w >> 1;
    const int rows = p.strip_h / 2 + 2 * R, cols = p.tile_w / 2 + 2 * R;
    const int i00 = s0 / 2 - R, j00 = ctx.tx0 / 2 - R;
    const WtcMap xs = p.xs, bs = p.b1s;
    const int bstride = bs.rows * bs.pitch;
    for (int idx = ctx.tid; idx < rows * cols; idx += ctx.nth) {
        const int ri = idx / cols, ci = idx - ri * cols;
        const int i = i00 + ri, j = j00 + ci;
        float b1 = 0.0f, b2 = 0.0f, b3 = 0.0f;
        if (i >= 0 && i < H1 && j >= 0 && j < W1) {
            // full-resolution row 2i is staged row 2i - (s0 - 2R) = 2 ri
            const int s = xs.off + (2 * ri) * xs.pitch + 2 * ci;
            const float x00 = WTC_LDS(ctx, s), x01 = WTC_LDS(ctx, s + 1);
            const float x10 = WTC_LDS(ctx, s + xs.pitch), x11 = WTC_LDS(ctx, s + xs.pitch + 1);
            const float sa = x00 + x01, sc = x10 + x11, da = x00 - x01, dc = x10 - x11;
            b1 = sa - sc;
            b2 = da + dc;
            b3 = da - dc;
        }
        const int o = bs.off + ri * bs.pitch + ci;
        WTC_LDS(ctx, o) = b1;
        WTC_LDS(ctx, o + bstride) = b2;
        WTC_LDS(ctx, o + 2 * bstride) = b3;
    }
}

// Phase 4c: level-1 convolutions of the strip, four bands, into Z1S.  Band 0
// reads the coarse map U_1, bands 1..3 the strip bands.
template <typename T, int K>
WTC_HD WTC_INLINE void wtc_phase_strip_conv1(const WtcFusedArgs<T> &a, WtcCtx<T> &ctx, int s0)
{
    constexpr int R = K / 2, kk = K * K;
    const WtcFusedPlan &p = a.p;
    const WtcLvl g = wtc_level(p, 1, ctx.ty0, ctx.tx0);
    const int TS1 = p.strip_h / 2, TW1 = p.tile_w / 2;
    const int npr = (TS1 + WTC_PR - 1) / WTC_PR, npc = (TW1 + WTC_PC - 1) / WTC_PC;
    const int total = 4 * npr * npc;
    const int si0 = s0 / 2;
    for (int pi = ctx.tid; pi < total; pi += ctx.nth) {
        const int b = pi / (npr * npc);
        const int rem = pi - b * npr * npc;
        const int pr = rem / npc, pc = rem - pr * npc;
        const int i0 = si0 + WTC_PR * pr, j0 = g.t0x + WTC_PC * pc;
        int src, pitch;
        if (b == 0) {
            const WtcMap mp = p.ll[1];
            pitch = mp.pitch;
            src = mp.off + (i0 - R - g.oy) * pitch + (j0 - R - g.ox);
        } else {
            const WtcMap mp = p.b1s;
            pitch = mp.pitch;
            src = mp.off + (b - 1) * mp.rows * pitch + (i0 - R - (si0 - R)) * pitch + (j0 - R - (g.t0x - R));
        }
        float acc[WTC_PR][WTC_PC];
#pragma unroll
        for (int dr = 0; dr < WTC_PR; ++dr)
#pragma unroll
            for (int dc = 0; dc < WTC_PC; ++dc) acc[dr][dc] = 0.0f;
        wtc_conv_block_lds<T, K, WTC_PR, WTC_PC>(ctx, src, pitch, p.wf_off + (1 + b) * kk, acc);
        const WtcMap zm = p.z1s;
        const int zb = zm.off + b * zm.rows * zm.pitch;
#pragma unroll
        for (int dr = 0; dr < WTC_PR; ++dr)
#pragma unroll
            for (int dc = 0; dc < WTC_PC; ++dc) {
                const int i = i0 + dr, j = j0 + dc;
                if (i < si0 + TS1 && j < g.t1x) WTC_LDS(ctx, zb + (i - si0) * zm.pitch + (j - g.t0x)) = acc[dr][dc];
            }
    }
}

// Sum of the deep levels m = 2..L for the 2x2 output block whose level-1
// coordinates are (i1, j1): the closed form with the coordinate bits of each
// level picking the signs.
template <typename T>
WTC_HD WTC_INLINE float wtc_deep_sum(const WtcFusedPlan &p, WtcCtx<T> &ctx, int i1, int j1)
{
    float d = 0.0f;
    for (int m = 2; m <= p.levels; ++m) {
        const WtcMap zm = p.z[m];
        const int zi = (i1 >> (m - 1)) - (ctx.ty0 >> m), zj = (j1 >> (m - 1)) - (ctx.tx0 >> m);
        const float sp = ((i1 >> (m - 2)) & 1) ? -1.0f : 1.0f;
        const float sq = ((j1 >> (m - 2)) & 1) ? -1.0f : 1.0f;
        const int o = zm.off + zi * zm.pitch + zj, st = zm.rows * zm.pitch;
        const float z0 = WTC_LDS(ctx, o), z1 = WTC_LDS(ctx, o + st), z2 = WTC_LDS(ctx, o + 2 * st),
                    z3 = WTC_LDS(ctx, o + 3 * st);
        d += z0;
        d = wtc_fma(sp, z1, d);
        d = wtc_fma(sq, z2, d);
        d = wtc_fma(sp * sq, z3, d);
    }
    return d;
}

template <typename T, int BW>
WTC_HD WTC_INLINE void wtc_store_row(WtcCtx<T> &ctx, int64_t o, const float (&v)[BW])
{
#ifdef WTC_EMULATE
    for (int e = 0; e < BW; ++e) WTC_OUT(ctx, o + e) = wtc_from_float<T>(v[e]);
#else
    T t[BW];
#pragma unroll
    for (int e = 0; e < BW; ++e) t[e] = wtc_from_float<T>(v[e]);
    // BW * sizeof(T) bytes at an address that is a multiple of that size
    // (the row length is a multiple of BW and buffers are 16-byte aligned);
    // non-temporal (streaming) stores: the output is not read again here, and
    // they measured 2-3 % faster than cached stores on the whole-plane kernel
    if constexpr (BW * sizeof(T) == 32) {
        typedef float v4 __attribute__((ext_vector_type(4)));
        v4 a, b;
        __builtin_memcpy(&a, &t[0], 16);
        __builtin_memcpy(&b, &t[BW / 2], 16);
        __builtin_nontemporal_store(a, (v4 *)(ctx.out + o));
        __builtin_nontemporal_store(b, (v4 *)(ctx.out + o + BW / 2));
    } else if constexpr (BW * sizeof(T) == 16) {
        typedef float v4 __attribute__((ext_vector_type(4)));
        v4 a;
        __builtin_memcpy(&a, &t[0], 16);
        __builtin_nontemporal_store(a, (v4 *)(ctx.out + o));
    } else if constexpr (BW * sizeof(T) == 8) {
        typedef float v2 __attribute__((ext_vector_type(2)));
        v2 a;
        __builtin_memcpy(&a, &t[0], 8);
        __builtin_nontemporal_store(a, (v2 *)(ctx.out + o));
    } else if constexpr (BW * sizeof(T) == 4) {
        float a;
        __builtin_memcpy(&a, &t[0], 4);
        *(float *)(ctx.out + o) = a;
    } else {
#pragma unroll
        for (int e = 0; e < BW; ++e) ctx.out[o + e] = t[e];
    }
#endif
}

// Phase 4d: the output of the strip in 2 x BW blocks: the base convolution from
// the staged strip plus bias, the level-1 butterfly of Z1S with the deep sum
// added to its low-pass input, one rounding, one store.
template <typename T, int K, int BW>
WTC_HD WTC_INLINE void wtc_phase_strip_out(const WtcFusedArgs<T> &a, WtcCtx<T> &ctx, int s0)
{
    constexpr int R = K / 2;
    const WtcFusedPlan &p = a.p;
    const int nbx = p.tile_w / BW, nby = p.strip_h / 2;
    const WtcMap xs = p.xs, zm = p.z1s;
    const int zst = zm.rows * zm.pitch;
    float w0[K * K];
#pragma unroll
    for (int e = 0; e < K * K; ++e) w0[e] = wtc_uniform(WTC_LDS(ctx, p.wf_off + e));
    const float bias = ctx.bias;
    for (int idx = ctx.tid; idx < nbx * nby; idx += ctx.nth) {
        const int by = idx / nbx, bx = idx - by * nbx;
        const int h0 = s0 + 2 * by, w0c = ctx.tx0 + BW * bx;
        float acc[2][BW];
#pragma unroll
        for (int dr = 0; dr < 2; ++dr)
#pragma unroll
            for (int dc = 0; dc < BW; ++dc) acc[dr][dc] = bias;
        // base conv: staged row of h0 - R is 2 by + R, column of w0c - R is BW bx + R
        const int src = xs.off + (2 * by + R) * xs.pitch + BW * bx + R;
#pragma unroll
        for (int t = 0; t < 2 + K - 1; ++t) {
            float row[BW + K - 1];
#pragma unroll
            for (int e = 0; e < BW + K - 1; ++e) row[e] = WTC_LDS(ctx, src + t * xs.pitch + e);
#pragma unroll
            for (int dr = 0; dr < 2; ++dr) {
                const int u = t - dr;
                if (u < 0 || u >= K) continue;
#pragma unroll
                for (int v = 0; v < K; ++v)
#pragma unroll
                    for (int dc = 0; dc < BW; ++dc) acc[dr][dc] = wtc_fma(w0[u * K + v], row[dc + v], acc[dr][dc]);
            }
        }
        // synthesis, one 2x2 block (one level-1 pixel) at a time
        const int i1 = h0 >> 1;
#pragma unroll
        for (int q = 0; q < BW / 2; ++q) {
            const int j1 = (w0c >> 1) + q;
            const int o = zm.off + (i1 - (s0 >> 1)) * zm.pitch + (j1 - (ctx.tx0 >> 1));
            float a0 = WTC_LDS(ctx, o);
            const float a1 = WTC_LDS(ctx, o + zst), a2 = WTC_LDS(ctx, o + 2 * zst), a3 = WTC_LDS(ctx, o + 3 * zst);
            a0 += wtc_deep_sum<T>(p, ctx, i1, j1);
            const float s01 = a0 + a1, d01 = a0 - a1, s23 = a2 + a3, d23 = a2 - a3;
            acc[0][2 * q] += s01 + s23;
            acc[0][2 * q + 1] += s01 - s23;
            acc[1][2 * q] += d01 + d23;
            acc[1][2 * q + 1] += d01 - d23;
        }
        const int64_t o0 = (int64_t)h0 * p.w + w0c;
        wtc_store_row<T, BW>(ctx, o0, acc[0]);
        wtc_store_row<T, BW>(ctx, o0 + p.w, acc[1]);
    }
}

#endif  // WTCONV_FUSED_BODY_H
