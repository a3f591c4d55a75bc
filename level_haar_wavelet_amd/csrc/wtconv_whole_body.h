// wtconv_whole_body.h -- fused WTConv forward / data backward for planes that
// fit in LDS whole ("whole-plane" kernel), written as phases separated by
// workgroup barriers so that a CPU emulation can run the same code.
//
// Source: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation" (arXiv 2608.10805), technical summary, Methodology,
// reformulations 1-3 (on-chip Haar analysis, closed-form bit-indexed
// synthesis, scales folded into the weights).  The arithmetic is the one
// described at the top of wtconv_fused_body.h:
//   U_m = plain 2x2 sums (low-pass), B_m^b = plain signed 2x2 sums (details),
//   W''_m^b = 4^-m s_m^b W_m^b, Z_m^b = W''_m^b (*) B_m^b (with B_m^0 = U_m),
//   y = s0 W0 (*) x + s0 b0 + sum_m sum_b sign_b(bits of h, w) Z_m^b[h>>m, w>>m].
//
// Organisation for gfx950:
//   * a workgroup owns one channel and P consecutive images of it (the
//     channel's folded weights are computed once); the input of the next image
//     is loaded into registers while the current one is computed, and the
//     workgroup barriers only wait for LDS traffic, so those loads stay in
//     flight across them;
//   * LDS is zeroed once: every map keeps a zero border of r pixels, which is
//     the convolutions' zero padding, and only interiors are rewritten;
//   * all maps have an odd row pitch, and consecutive lanes take consecutive
//     2-row blocks, so the 2-row window reads of a wave fall in distinct banks;
//   * one convolution phase holds the base-convolution blocks (whose results
//     stay in registers until the synthesis) and every per-level piece of
//     every level and band, dealt round-robin to the threads.
#ifndef WTCONV_WHOLE_BODY_H
#define WTCONV_WHOLE_BODY_H

#include "wtconv_fused_body.h"

#define WTC_WHOLE_NCH 4   // 16-byte (or smaller) input chunks per thread and image

struct WtcWholePlan {
    int32_t n, c, h, w, k, levels;
    int32_t rotate;
    int32_t nthreads;
    int32_t planes;      // images per workgroup (same channel)
    int32_t vec;         // activation elements per global chunk
    int32_t out_bw;      // output block width (2, 4 or 8)
    WtcMap x;            // input, rows h + 4r, image origin at (2r, 2r)
    WtcMap u[WTC_MAXL + 1];   // U_m plus three detail bands, m = 1..L, origin (r, r)
    WtcMap z[WTC_MAXL + 1];   // four conv outputs of level m, origin (0, 0)
    int32_t wf_off;
    int32_t items;       // convolution items per image: base blocks, then pieces
    int32_t tab_off;     // item descriptors, 4 ints each
    int32_t lds_floats;
};

WTC_PLAN_HD static inline int32_t wtc_odd_pitch(int32_t cols) { return cols | 1; }

// Fills the LDS layout; returns the number of floats.
static inline int32_t wtc_whole_layout(WtcWholePlan *p)
{
    const int32_t L = p->levels, r = p->k / 2, kk = p->k * p->k;
    int32_t off = 0;
    p->wf_off = off;
    off += wtc_roundup((1 + 4 * L) * kk, 4);
    p->x.off = off;
    p->x.rows = p->h + 4 * r;
    p->x.pitch = wtc_odd_pitch(wtc_roundup(p->w, 8) + 4 * r);
    off += p->x.rows * p->x.pitch;
    for (int32_t m = 0; m <= WTC_MAXL; ++m) {
        p->u[m].off = p->u[m].pitch = p->u[m].rows = 0;
        p->z[m] = p->u[m];
    }
    for (int32_t m = 1; m <= L; ++m) {
        const int32_t Hm = p->h >> m, Wm = p->w >> m;
        // map plus r-wide zero border; room for the ragged last piece
        p->u[m].off = off;
        p->u[m].rows = wtc_roundup(Hm, WTC_PR) + 2 * r;
        p->u[m].pitch = wtc_odd_pitch(wtc_roundup(Wm, WTC_PC) + 2 * r);
        off += 4 * p->u[m].rows * p->u[m].pitch;
    }
    for (int32_t m = 1; m <= L; ++m) {
        const int32_t Hm = p->h >> m, Wm = p->w >> m;
        p->z[m].off = off;
        p->z[m].rows = Hm;
        p->z[m].pitch = wtc_odd_pitch(Wm);
        off += 4 * p->z[m].rows * p->z[m].pitch;
    }
    int32_t items = (p->h / 2) * (p->w / p->out_bw);
    for (int32_t m = 1; m <= L; ++m)
        items += 4 * (((p->h >> m) + WTC_PR - 1) / WTC_PR) * (((p->w >> m) + WTC_PC - 1) / WTC_PC);
    p->items = items;
    off = wtc_roundup(off, 4);
    p->tab_off = off;
    off += 4 * items;
    p->lds_floats = wtc_roundup(off, 4);
    return p->lds_floats;
}

static inline int32_t wtc_whole_blocks(const WtcWholePlan *p) { return (p->h / 2) * (p->w / p->out_bw); }

// Plan of the whole-plane kernel, or -1 when the plane does not fit (LDS,
// per-thread chunk or block limits).  `planes` is the requested number of
// images per workgroup (clamped to n).
static inline int wtc_make_whole_plan(WtcWholePlan *p, int32_t n, int32_t c, int32_t h, int32_t w, int32_t k,
                                      int32_t levels, int32_t rotate, int32_t nthreads, int32_t planes,
                                      int32_t elem_bytes, int32_t budget_floats)
{
    p->n = n;
    p->c = c;
    p->h = h;
    p->w = w;
    p->k = k;
    p->levels = levels;
    p->rotate = rotate;
    p->nthreads = nthreads;
    p->planes = planes < 1 ? 1 : (planes > n ? n : planes);
    if (levels < 1 || levels > WTC_MAXL) return -1;
    if (h % (1 << levels) || w % (1 << levels)) return -1;
    int32_t vec = 16 / elem_bytes;
    while (vec > 1 && w % vec) vec /= 2;
    p->vec = vec;
    p->out_bw = (w % 8 == 0) ? 8 : (w % 4 == 0) ? 4 : 2;
    const int64_t chunks = (int64_t)h * (w / vec);
    if (chunks > (int64_t)WTC_WHOLE_NCH * nthreads) return -1;
    if (wtc_whole_blocks(p) > nthreads) return -1;  // one base block per thread
    wtc_whole_layout(p);
    return p->lds_floats <= budget_floats ? 0 : -1;
}

template <typename T>
struct WtcWholeArgs {
    const T *in;
    T *out;
    const float *w_base, *bias, *s_base, *w_lvl, *s_lvl;
    WtcWholePlan p;
};

// Per-thread state of the whole-plane kernel.
template <typename T>
struct WtcWholeCtx {
    float *lds;
    const T *in;  // image pointer of the current image
    T *out;
    int tid, nth;
    int c, n0, nimg;  // channel, first image, images of this workgroup
    float bias;
    // prefetched raw chunk values (as loaded: T)
    T pre[WTC_WHOLE_NCH][16 / sizeof(T)];
    // base-convolution result of this thread's block
    float y0[2][8];
#ifdef WTC_EMULATE
    int64_t lds_n, img_n;
#endif
};

#ifdef WTC_EMULATE
#define WTC_WIN(ctx, i) wtc_chk((ctx).in, (int64_t)(i), (ctx).img_n, __LINE__)
#define WTC_WOUT(ctx, i) wtc_chk((ctx).out, (int64_t)(i), (ctx).img_n, __LINE__)
#else
#define WTC_WIN(ctx, i) ((ctx).in[(i)])
#define WTC_WOUT(ctx, i) ((ctx).out[(i)])
#endif

template <typename T>
WTC_HD WTC_INLINE void wtc_whole_setup(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx, int bid)
{
    const WtcWholePlan &p = a.p;
    const int groups = (p.n + p.planes - 1) / p.planes;
    // consecutive workgroups take consecutive channels of the same image group
    ctx.c = bid % p.c;
    const int g = bid / p.c;
    ctx.n0 = g * p.planes;
    ctx.nimg = wtc_min(p.planes, p.n - ctx.n0);
    (void)groups;
    float b = 0.0f;
    if (!p.rotate && a.bias) b = a.s_base[ctx.c] * a.bias[ctx.c];
    ctx.bias = b;
}

template <typename T>
WTC_HD WTC_INLINE void wtc_whole_select(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx, int img)
{
    const int64_t hw = (int64_t)a.p.h * a.p.w;
    const int64_t plane = (int64_t)(ctx.n0 + img) * a.p.c + ctx.c;
    ctx.in = a.in + plane * hw;
    ctx.out = a.out + plane * hw;
}

// Phase: zero all of LDS (once per workgroup) and fold the channel's weights.
template <typename T, int K>
WTC_HD WTC_INLINE void wtc_whole_init(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    const WtcWholePlan &p = a.p;
    for (int i = ctx.tid; i < p.lds_floats; i += ctx.nth) WTC_LDS(ctx, i) = 0.0f;
}

template <typename T, int K>
WTC_HD WTC_INLINE void wtc_whole_fold(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    const WtcWholePlan &p = a.p;
    constexpr int kk = K * K;
    const int total = (1 + 4 * p.levels) * kk;
    const int C = p.c, c = ctx.c;
    for (int i = ctx.tid; i < total; i += ctx.nth) {
        const int blk = i / kk, e = i - blk * kk;
        const int se = p.rotate ? (kk - 1 - e) : e;
        float v;
        if (blk == 0) {
            v = WTC_PAR(a.s_base, c, C) * WTC_PAR(a.w_base, c * kk + se, (int64_t)C * kk);
        } else {
            const int m = (blk - 1) / 4 + 1, b = (blk - 1) % 4;
            const int ch = (m - 1) * 4 * C + 4 * c + b;
            const float s = WTC_PAR(a.s_lvl, ch, (int64_t)p.levels * 4 * C);
            v = ldexpf(s * WTC_PAR(a.w_lvl, (int64_t)ch * kk + se, (int64_t)p.levels * 4 * C * kk), -2 * m);
        }
        WTC_LDS(ctx, p.wf_off + i) = v;
    }
}

// Elements per global chunk: 16 bytes, or the output block width if smaller
// (the plan picks the same value from the image width).
template <typename T, int BW>
struct WtcVec {
    static constexpr int v = BW < (int)(16 / sizeof(T)) ? BW : (int)(16 / sizeof(T));
};

// Issue the loads of image `img` of the workgroup into registers.
template <typename T, int K, int BW>
WTC_HD WTC_INLINE void wtc_whole_load(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx, int img)
{
    const WtcWholePlan &p = a.p;
    const T *src = a.in + ((int64_t)(ctx.n0 + img) * p.c + ctx.c) * ((int64_t)p.h * p.w);
    constexpr int vec = WtcVec<T, BW>::v;
    const int cpr = p.w / vec, total = p.h * cpr;
#pragma unroll
    for (int q = 0; q < WTC_WHOLE_NCH; ++q) {
        // every lane loads (a valid chunk) so that no branch surrounds the loads;
        // lanes past the end repeat the last chunk and do not store it
        const int idx = wtc_min(ctx.tid + q * ctx.nth, total - 1);
        {
            const int64_t e = (int64_t)idx * vec;  // chunks tile the image row-major
#ifdef WTC_EMULATE
            const int64_t base = src - a.in, all = (int64_t)p.n * p.c * p.h * p.w;
            for (int t = 0; t < vec; ++t) ctx.pre[q][t] = wtc_chk(a.in, base + e + t, all, __LINE__);
#else
            if constexpr (vec * sizeof(T) == 16) {
                typedef float v4 __attribute__((ext_vector_type(4)));
                v4 d = __builtin_nontemporal_load((const v4 *)(src + e));
                __builtin_memcpy(&ctx.pre[q][0], &d, 16);
            } else if constexpr (vec * sizeof(T) == 8) {
                typedef float v2 __attribute__((ext_vector_type(2)));
                v2 d = __builtin_nontemporal_load((const v2 *)(src + e));
                __builtin_memcpy(&ctx.pre[q][0], &d, 8);
            } else if constexpr (vec * sizeof(T) == 4) {
                float d = __builtin_nontemporal_load((const float *)(src + e));
                __builtin_memcpy(&ctx.pre[q][0], &d, 4);
            } else {
#pragma unroll
                for (int t = 0; t < vec; ++t) ctx.pre[q][t] = src[e + t];
            }
#endif
        }
    }
}

// Write the prefetched chunks into the interior of the input map.
template <typename T, int K, int BW>
WTC_HD WTC_INLINE void wtc_whole_store_input(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    constexpr int R = K / 2;
    const WtcWholePlan &p = a.p;
    constexpr int vec = WtcVec<T, BW>::v;
    const int cpr = p.w / vec, total = p.h * cpr;
    const WtcMap xm = p.x;
#pragma unroll
    for (int q = 0; q < WTC_WHOLE_NCH; ++q) {
        const int idx = ctx.tid + q * ctx.nth;
        if (idx < total) {
            const int row = idx / cpr, col = (idx - row * cpr) * vec;
            const int o = xm.off + (row + 2 * R) * xm.pitch + col + 2 * R;
#pragma unroll
            for (int t = 0; t < vec; ++t) WTC_LDS(ctx, o + t) = wtc_to_float(ctx.pre[q][t]);
        }
    }
}

// Level-1 analysis: U_1 and B_1^1..3 from the input map (interior only).
template <typename T, int K>
WTC_HD WTC_INLINE void wtc_whole_analysis1(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    constexpr int R = K / 2;
    const WtcWholePlan &p = a.p;
    const int H1 = p.h >> 1, W1 = p.w >> 1;
    const WtcMap xm = p.x, um = p.u[1];
    const int st = um.rows * um.pitch;
    const int total = H1 * W1;
    int i = ctx.tid / W1, j = ctx.tid - (ctx.tid / W1) * W1;
    const int di = ctx.nth / W1, dj = ctx.nth - di * W1;
    for (int idx = ctx.tid; idx < total; idx += ctx.nth) {
        const int s = xm.off + (2 * i + 2 * R) * xm.pitch + 2 * j + 2 * R;
        const float x00 = WTC_LDS(ctx, s), x01 = WTC_LDS(ctx, s + 1);
        const float x10 = WTC_LDS(ctx, s + xm.pitch), x11 = WTC_LDS(ctx, s + xm.pitch + 1);
        const float sa = x00 + x01, sc = x10 + x11, da = x00 - x01, dc = x10 - x11;
        const int o = um.off + (i + R) * um.pitch + j + R;
        WTC_LDS(ctx, o) = sa + sc;
        WTC_LDS(ctx, o + st) = sa - sc;
        WTC_LDS(ctx, o + 2 * st) = da + dc;
        WTC_LDS(ctx, o + 3 * st) = da - dc;
        i += di;
        j += dj;
        if (j >= W1) {
            j -= W1;
            ++i;
        }
    }
}

// Level-m analysis (m >= 2) from U_{m-1}.
template <typename T, int K>
WTC_HD WTC_INLINE void wtc_whole_analysis(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx, int m)
{
    constexpr int R = K / 2;
    const WtcWholePlan &p = a.p;
    const int Hm = p.h >> m, Wm = p.w >> m;
    const WtcMap sm = p.u[m - 1], um = p.u[m];
    const int st = um.rows * um.pitch;
    const int total = Hm * Wm;
    int i = ctx.tid / Wm, j = ctx.tid - (ctx.tid / Wm) * Wm;
    const int di = ctx.nth / Wm, dj = ctx.nth - di * Wm;
    for (int idx = ctx.tid; idx < total; idx += ctx.nth) {
        const int s = sm.off + (2 * i + R) * sm.pitch + 2 * j + R;
        const float x00 = WTC_LDS(ctx, s), x01 = WTC_LDS(ctx, s + 1);
        const float x10 = WTC_LDS(ctx, s + sm.pitch), x11 = WTC_LDS(ctx, s + sm.pitch + 1);
        const float sa = x00 + x01, sc = x10 + x11, da = x00 - x01, dc = x10 - x11;
        const int o = um.off + (i + R) * um.pitch + j + R;
        WTC_LDS(ctx, o) = sa + sc;
        WTC_LDS(ctx, o + st) = sa - sc;
        WTC_LDS(ctx, o + 2 * st) = da + dc;
        WTC_LDS(ctx, o + 3 * st) = da - dc;
        i += di;
        j += dj;
        if (j >= Wm) {
            j -= Wm;
            ++i;
        }
    }
}

// Item descriptors, built once per workgroup (they depend only on the plan).
// Items [0, nblk) are base-convolution blocks of 2 x BW outputs, block rows
// fastest (consecutive lanes take consecutive row pairs: with the odd pitch
// their window reads fall in distinct banks):
//   d0 = LDS index of the input window (row 2by - R, column BW bx - R)
//   d1 = offset of the block's first output in the image
//   d2 = LDS index of the level-1 outputs of the block's first 2x2 quad
//   d3 = by | (bx << 16)
// The remaining items are WTC_PR x WTC_PC pieces of one band of one level,
// piece rows fastest:
//   d0 = LDS index of the input window of the band map
//   d1 = LDS index of the first output in the band's output map
//   d2 = LDS index of the folded weights | (input pitch << 16)
//   d3 = valid output rows | (valid columns << 8) | (output pitch << 16)
template <typename T, int K, int BW>
WTC_HD WTC_INLINE void wtc_whole_table(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    constexpr int R = K / 2, kk = K * K;
    const WtcWholePlan &p = a.p;
    const int nby = p.h / 2, nblk = nby * (p.w / BW);
    const WtcMap xm = p.x, z1 = p.z[1];
    for (int it = ctx.tid; it < p.items; it += ctx.nth) {
        int d0, d1, d2, d3;
        if (it < nblk) {
            const int by = it % nby, bx = it / nby;
            d0 = xm.off + (2 * by + R) * xm.pitch + BW * bx + R;
            d1 = 2 * by * p.w + BW * bx;
            d2 = z1.off + by * z1.pitch + (BW / 2) * bx;
            d3 = by | (bx << 16);
        } else {
            int rem = it - nblk, m = 1, npr = 0, npc = 0;
            for (; m <= p.levels; ++m) {
                npr = ((p.h >> m) + WTC_PR - 1) / WTC_PR;
                npc = ((p.w >> m) + WTC_PC - 1) / WTC_PC;
                if (rem < 4 * npr * npc) break;
                rem -= 4 * npr * npc;
            }
            const int b = rem / (npr * npc);
            rem -= b * npr * npc;
            const int pc = rem / npr, pr = rem - pc * npr;
            const WtcMap um = p.u[m], zm = p.z[m];
            const int Hm = p.h >> m, Wm = p.w >> m;
            d0 = um.off + b * um.rows * um.pitch + (WTC_PR * pr) * um.pitch + WTC_PC * pc;
            d1 = zm.off + b * zm.rows * zm.pitch + (WTC_PR * pr) * zm.pitch + WTC_PC * pc;
            d2 = (p.wf_off + (1 + 4 * (m - 1) + b) * kk) | (um.pitch << 16);
            d3 = wtc_min(WTC_PR, Hm - WTC_PR * pr) | (wtc_min(WTC_PC, Wm - WTC_PC * pc) << 8) | (zm.pitch << 16);
        }
        int *tab = (int *)&WTC_LDS(ctx, p.tab_off + 4 * it);
        tab[0] = d0;
        tab[1] = d1;
        tab[2] = d2;
        tab[3] = d3;
    }
}

template <typename T>
WTC_HD WTC_INLINE void wtc_whole_desc(WtcWholeCtx<T> &ctx, int off, int &d0, int &d1, int &d2, int &d3)
{
#ifdef WTC_EMULATE
    const int *t = (const int *)&WTC_LDS(ctx, off + 3) - 3;
#else
    const int *t = (const int *)&ctx.lds[off];
#endif
    d0 = t[0];
    d1 = t[1];
    d2 = t[2];
    d3 = t[3];
}

// The convolution phase: each thread takes items tid, tid + nth, ...; its base
// block (item tid, if any) stays in registers for the synthesis.
template <typename T, int K, int BW>
WTC_HD WTC_INLINE void wtc_whole_conv(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    constexpr int kk = K * K;
    const WtcWholePlan &p = a.p;
    const int nblk = (p.h / 2) * (p.w / BW);
    const WtcMap xm = p.x;
    for (int it = ctx.tid; it < p.items; it += ctx.nth) {
        int d0, d1, d2, d3;
        wtc_whole_desc<T>(ctx, p.tab_off + 4 * it, d0, d1, d2, d3);
        if (it < nblk) {
            float w0[kk];
#pragma unroll
            for (int e = 0; e < kk; ++e) w0[e] = wtc_uniform(WTC_LDS(ctx, p.wf_off + e));
            float acc[2][BW];
#pragma unroll
            for (int dr = 0; dr < 2; ++dr)
#pragma unroll
                for (int dc = 0; dc < BW; ++dc) acc[dr][dc] = ctx.bias;
#pragma unroll
            for (int t = 0; t < 2 + K - 1; ++t) {
                float row[BW + K - 1];
#pragma unroll
                for (int e = 0; e < BW + K - 1; ++e) row[e] = WTC_LDS(ctx, d0 + t * xm.pitch + e);
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
#pragma unroll
            for (int dr = 0; dr < 2; ++dr)
#pragma unroll
                for (int dc = 0; dc < BW; ++dc) ctx.y0[dr][dc] = acc[dr][dc];
        } else {
            const int wk = d2 & 0xffff, spitch = d2 >> 16;
            const int vr = d3 & 0xff, vc = (d3 >> 8) & 0xff, zpitch = d3 >> 16;
            float acc[WTC_PR][WTC_PC];
#pragma unroll
            for (int dr = 0; dr < WTC_PR; ++dr)
#pragma unroll
                for (int dc = 0; dc < WTC_PC; ++dc) acc[dr][dc] = 0.0f;
            // wtc_conv_block_lds takes a context only for its LDS pointer
            WtcCtx<T> lc;
            lc.lds = ctx.lds;
#ifdef WTC_EMULATE
            lc.lds_n = ctx.lds_n;
#endif
            wtc_conv_block_lds<T, K, WTC_PR, WTC_PC>(lc, d0, spitch, wk, acc);
#pragma unroll
            for (int dr = 0; dr < WTC_PR; ++dr)
#pragma unroll
                for (int dc = 0; dc < WTC_PC; ++dc)
                    if (dr < vr && dc < vc) WTC_LDS(ctx, d1 + dr * zpitch + dc) = acc[dr][dc];
        }
    }
}

// Synthesis and store of this thread's base block: level 1 through the 2x2
// butterfly, the deeper levels through the closed form with the coordinate
// bits picking the signs, added to the low-pass input of the butterfly.
template <typename T, int K, int BW>
WTC_HD WTC_INLINE void wtc_whole_out(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    const WtcWholePlan &p = a.p;
    const int nblk = (p.h / 2) * (p.w / BW);
    const int it = ctx.tid;
    if (it >= nblk) return;
    int d0, d1, d2, d3;
    wtc_whole_desc<T>(ctx, p.tab_off + 4 * it, d0, d1, d2, d3);
    const int i1 = d3 & 0xffff, bx = d3 >> 16;
    const WtcMap z1 = p.z[1];
    const int st1 = z1.rows * z1.pitch;
    float acc[2][BW];
#pragma unroll
    for (int dr = 0; dr < 2; ++dr)
#pragma unroll
        for (int dc = 0; dc < BW; ++dc) acc[dr][dc] = ctx.y0[dr][dc];
    float deep[BW / 2];
#pragma unroll
    for (int q = 0; q < BW / 2; ++q) deep[q] = 0.0f;
    for (int m = 2; m <= p.levels; ++m) {
        const WtcMap zm = p.z[m];
        const int sz = zm.rows * zm.pitch;
        const float sp = ((i1 >> (m - 2)) & 1) ? -1.0f : 1.0f;
        const int rowo = zm.off + (i1 >> (m - 1)) * zm.pitch;
#pragma unroll
        for (int q = 0; q < BW / 2; ++q) {
            const int j1 = (BW / 2) * bx + q;
            const float sq = ((j1 >> (m - 2)) & 1) ? -1.0f : 1.0f;
            const int oz = rowo + (j1 >> (m - 1));
            float d = deep[q] + WTC_LDS(ctx, oz);
            d = wtc_fma(sp, WTC_LDS(ctx, oz + sz), d);
            d = wtc_fma(sq, WTC_LDS(ctx, oz + 2 * sz), d);
            deep[q] = wtc_fma(sp * sq, WTC_LDS(ctx, oz + 3 * sz), d);
        }
    }
#pragma unroll
    for (int q = 0; q < BW / 2; ++q) {
        const int o = d2 + q;
        const float a0 = WTC_LDS(ctx, o) + deep[q];
        const float a1 = WTC_LDS(ctx, o + st1), a2 = WTC_LDS(ctx, o + 2 * st1), a3 = WTC_LDS(ctx, o + 3 * st1);
        const float s01 = a0 + a1, d01 = a0 - a1, s23 = a2 + a3, d23 = a2 - a3;
        acc[0][2 * q] += s01 + s23;
        acc[0][2 * q + 1] += s01 - s23;
        acc[1][2 * q] += d01 + d23;
        acc[1][2 * q + 1] += d01 - d23;
    }
#ifdef WTC_EMULATE
    for (int dr = 0; dr < 2; ++dr)
        for (int e = 0; e < BW; ++e) WTC_WOUT(ctx, d1 + dr * p.w + e) = wtc_from_float<T>(acc[dr][e]);
#else
    WtcCtx<T> oc;
    oc.out = ctx.out;
    wtc_store_row<T, BW>(oc, d1, acc[0]);
    wtc_store_row<T, BW>(oc, d1 + p.w, acc[1]);
#endif
}

#endif  // WTCONV_WHOLE_BODY_H
