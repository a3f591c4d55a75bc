// wtconv_wgrad_tile_body.h -- parameter gradients of the WTConv layer for
// planes too large to keep whole in LDS: one launch per level, on tiles.
//
// Step j (j = 0..L) takes the level-j low-pass maps of x and dy (U_0 = x,
// U_0(dy) = dy; later steps read the fp32 maps the previous step wrote) and
//   * correlates U_j(dy) with U_j(x): for j = 0 this is the base-convolution
//     gradient G_0 (and G_b = sum dy), for j >= 1 the low-pass band of level j;
//   * if j < L, forms the three detail bands of level j+1 of both maps and
//     correlates them, and writes U_{j+1}(x), U_{j+1}(dy) for step j+1.
// The per-map results go to the same per-workgroup partial rows as the
// whole-plane kernel's (wtconv_wgrad_body.h), so one finalize pass serves
// both.  Sources and arithmetic: see wtconv_wgrad_body.h.
//
// A workgroup owns one channel and a fixed share of the (image, tile) units
// of that channel; each thread owns fixed 4x4 pieces of the tile's dy-side
// maps and keeps their accumulators across all units, so the cross-thread
// reduction happens once per workgroup, in a fixed order.
#ifndef WTCONV_WGRAD_TILE_BODY_H
#define WTCONV_WGRAD_TILE_BODY_H

#include "wtconv_wgrad_body.h"

#define WTC_WT_QMAX 3

struct WtcWtilePlan {
    int32_t n, c, k, levels;
    int32_t step;            // j
    int32_t h, w;            // level-j map size
    int32_t th, tw;          // tile (even, divides h, w)
    int32_t tiles_y, tiles_x;
    int32_t units_per_wg;    // (image, tile) units of one workgroup
    int32_t groups;          // workgroups per channel
    int32_t nthreads;
    int32_t q;               // pieces per thread
    int32_t npieces;
    int32_t nmaps_here;      // 1 (last step) or 4
    int32_t first[5];
    int32_t plen;
    WtcMap x;                // U_j(x) over the tile plus 2r (origin (2r, 2r + xs))
    int32_t xs;              // left pad of the x map: correlation windows start on 16-byte boundaries
    WtcMap dy;               // U_j(dy) over the tile
    WtcMap bx;               // 3 detail bands of level j+1 of x, tile/2 plus r (origin (r, r))
    WtcMap bd;               // 3 detail bands of level j+1 of dy, tile/2
    int32_t tab_off, res_off, red_off;
    int32_t lds_floats;
};

static inline int32_t wtc_wtile_layout(WtcWtilePlan *p)
{
    const int32_t r = p->k / 2, kk = p->k * p->k, P = WTC_WG_P;
    const int32_t TH = p->th, TW = p->tw, last = p->step == p->levels;
    int32_t off = 0;
    // Rows are 16-byte aligned and the shared piece routine reads a window
    // row as roundup(P + k - 1, 4) floats from a 16-byte boundary: the x map
    // is shifted right by xs so that a window (starting r columns left of its
    // piece) starts on one, and every pitch leaves room for the last read.
    p->xs = (4 - r % 4) % 4;
    p->x.off = off;
    p->x.rows = wtc_roundup(TH, P) + 4 * r;
    p->x.pitch = wtc_roundup(p->xs + wtc_roundup(TW, P) + 4 * r, 4);
    off += p->x.rows * p->x.pitch;
    p->dy.off = off;
    p->dy.rows = wtc_roundup(TH, P);
    p->dy.pitch = wtc_roundup(TW, P);
    off += p->dy.rows * p->dy.pitch;
    p->bx.off = p->bx.rows = p->bx.pitch = 0;
    p->bd = p->bx;
    if (!last) {
        p->bx.off = off;
        p->bx.rows = wtc_roundup(TH / 2, P) + 2 * r;
        p->bx.pitch = wtc_roundup(wtc_roundup(TW / 2, P) + 2 * r, 4);
        off += 3 * p->bx.rows * p->bx.pitch;
        p->bd.off = off;
        p->bd.rows = wtc_roundup(TH / 2, P);
        p->bd.pitch = wtc_roundup(TW / 2, P);
        off += 3 * p->bd.rows * p->bd.pitch;
    }
    p->nmaps_here = last ? 1 : 4;
    int32_t np = 0;
    for (int32_t g = 0; g < p->nmaps_here; ++g) {
        p->first[g] = np;
        const int32_t hh = g == 0 ? TH : TH / 2, ww = g == 0 ? TW : TW / 2;
        np += ((hh + P - 1) / P) * ((ww + P - 1) / P);
    }
    p->first[p->nmaps_here] = np;
    p->npieces = np;
    p->q = (np + p->nthreads - 1) / p->nthreads;
    p->plen = kk + 1 + 4 * p->levels * kk;
    off = wtc_roundup(off, 4);
    p->tab_off = off;
    off += 2 * np;
    p->red_off = 0;
    off = wtc_max(off, p->nthreads * (kk + 1));
    p->res_off = wtc_roundup(off, 4);
    off = p->res_off + p->nmaps_here * (kk + 1);
    p->lds_floats = wtc_roundup(off, 4);
    return p->lds_floats;
}

// Largest even tile side <= cap that divides `side` (0 if none).
static inline int32_t wtc_wtile_side(int32_t side, int32_t cap)
{
    for (int32_t d = wtc_min(side, cap); d >= 2; --d)
        if (d % 2 == 0 && side % d == 0) return d;
    return 0;
}

static inline int wtc_make_wtile_plan(WtcWtilePlan *p, int32_t n, int32_t c, int32_t k, int32_t levels, int32_t step,
                                      int32_t h, int32_t w, int32_t nthreads, int32_t groups, int32_t budget_floats)
{
    p->n = n;
    p->c = c;
    p->k = k;
    p->levels = levels;
    p->step = step;
    p->h = h;
    p->w = w;
    p->nthreads = nthreads;
    if (step < levels && (h % 2 || w % 2)) return -1;
    for (int32_t cap = 64; cap >= 8; cap /= 2) {
        int32_t th = step < levels ? wtc_wtile_side(h, cap) : wtc_min(h, cap);
        int32_t tw = step < levels ? wtc_wtile_side(w, cap) : wtc_min(w, cap);
        if (step == levels) {
            // the last step needs no even tiles: any divisor
            th = h;
            while (th > cap) {
                int32_t d = th - 1;
                while (d > 1 && h % d) --d;
                th = d;
            }
            tw = w;
            while (tw > cap) {
                int32_t d = tw - 1;
                while (d > 1 && w % d) --d;
                tw = d;
            }
        }
        if (!th || !tw) continue;
        p->th = th;
        p->tw = tw;
        p->tiles_y = h / th;
        p->tiles_x = w / tw;
        // every step uses the same number of workgroups per channel (the
        // partial rows are shared); a workgroup without units writes zeros
        const int32_t units = n * p->tiles_y * p->tiles_x;
        p->groups = groups;
        p->units_per_wg = (units + groups - 1) / groups;
        wtc_wtile_layout(p);
        if (p->q <= WTC_WT_QMAX && p->lds_floats <= budget_floats && p->x.pitch < 256 && p->dy.pitch < 256 &&
            p->lds_floats < 65536)
            return 0;
    }
    return -1;
}

// Workspace of the tiled path: [partial rows][U(x) even steps][U(x) odd steps]
// [U(dy) even][U(dy) odd], each region 256-byte aligned.  Step j (< L) writes
// the level-(j+1) maps into the regions of parity j % 2; step j+1 reads them.
struct WtcWtileCarve {
    size_t partial_bytes, map_bytes[2];
    size_t off_ux[2], off_ud[2];
    size_t total;
};

static inline size_t wtc_align256(size_t b) { return (b + 255) / 256 * 256; }

static inline void wtc_wtile_carve(WtcWtileCarve *cv, int64_t n, int64_t c, int64_t h, int64_t w, int levels,
                                   int groups, int plen)
{
    cv->partial_bytes = (size_t)groups * (size_t)c * (size_t)plen * sizeof(float);
    cv->map_bytes[0] = cv->map_bytes[1] = 0;
    for (int j = 1; j <= levels; ++j) {
        const size_t sz = (size_t)(n * c * (h >> j) * (w >> j)) * sizeof(float);
        if (sz > cv->map_bytes[(j - 1) % 2]) cv->map_bytes[(j - 1) % 2] = sz;
    }
    size_t off = wtc_align256(cv->partial_bytes);
    cv->off_ux[0] = off;
    off += wtc_align256(cv->map_bytes[0]);
    cv->off_ux[1] = off;
    off += wtc_align256(cv->map_bytes[1]);
    cv->off_ud[0] = off;
    off += wtc_align256(cv->map_bytes[0]);
    cv->off_ud[1] = off;
    off += wtc_align256(cv->map_bytes[1]);
    cv->total = off;
}

template <typename TI>
struct WtcWtileArgs {
    const TI *x;      // U_j(x), [N][C][h][w]
    const TI *dy;     // U_j(dy)
    float *ux;        // U_{j+1}(x) out, [N][C][h/2][w/2] (unused on the last step)
    float *ud;        // U_{j+1}(dy) out
    float *partial;   // [groups][C][plen]
    WtcWtilePlan p;
};

struct WtcWtileCtx {
    float *lds;
    int tid, nth;
    int c, group;
#ifdef WTC_EMULATE
    int64_t lds_n;
#endif
};

WTC_HD WTC_INLINE void wtc_wtile_unit(const WtcWtilePlan &p, int c, int u, int64_t *plane, int *ty0, int *tx0)
{
    const int tiles = p.tiles_y * p.tiles_x;
    const int img = u / tiles, t = u - img * tiles;
    *plane = (int64_t)img * p.c + c;
    *ty0 = (t / p.tiles_x) * p.th;
    *tx0 = (t % p.tiles_x) * p.tw;
}

template <typename TI>
WTC_HD WTC_INLINE void wtc_wtile_zero(const WtcWtileArgs<TI> &a, WtcWtileCtx &ctx)
{
    for (int i = ctx.tid; i < a.p.lds_floats; i += ctx.nth) WTC_LDS(ctx, i) = 0.0f;
}

// Descriptors as in the whole-plane kernel: map 0 is the tile of U_j,
// maps 1..3 the detail bands of level j+1.
template <typename TI, int K>
WTC_HD WTC_INLINE void wtc_wtile_table(const WtcWtileArgs<TI> &a, WtcWtileCtx &ctx)
{
    constexpr int P = WTC_WG_P, R = K / 2;
    const WtcWtilePlan &p = a.p;
    for (int it = ctx.tid; it < p.npieces; it += ctx.nth) {
        int g = 0;
        while (g + 1 < p.nmaps_here && it >= p.first[g + 1]) ++g;
        const int ww = g == 0 ? p.tw : p.tw / 2, npc = (ww + P - 1) / P;
        const int rem = it - p.first[g];
        const int pr = rem / npc, pc = rem - pr * npc;
        int d0, d1, xp, dp;
        if (g == 0) {
            // x origin (2R, 2R + xs): element (i0 - R, j0 - R) sits at (i0 + R, j0 + R + xs)
            d0 = p.x.off + (P * pr + R) * p.x.pitch + P * pc + R + p.xs;
            d1 = p.dy.off + (P * pr) * p.dy.pitch + P * pc;
            xp = p.x.pitch;
            dp = p.dy.pitch;
        } else {
            d0 = p.bx.off + (g - 1) * p.bx.rows * p.bx.pitch + (P * pr) * p.bx.pitch + P * pc;
            d1 = p.bd.off + (g - 1) * p.bd.rows * p.bd.pitch + (P * pr) * p.bd.pitch + P * pc;
            xp = p.bx.pitch;
            dp = p.bd.pitch;
        }
        int *tab = (int *)&WTC_LDS(ctx, p.tab_off + 2 * it + 1) - 1;
        tab[0] = (int)((unsigned)d0 | ((unsigned)d1 << 16));
        tab[1] = xp | (dp << 8) | (g << 16);
    }
}

// Stage one unit: U_j(x) over the tile plus 2R (zero outside the map) and
// U_j(dy) over the tile.
template <typename TI, int K>
WTC_HD WTC_INLINE void wtc_wtile_stage(const WtcWtileArgs<TI> &a, WtcWtileCtx &ctx, int u)
{
    constexpr int R = K / 2;
    const WtcWtilePlan &p = a.p;
    int64_t plane;
    int ty0, tx0;
    wtc_wtile_unit(p, ctx.c, u, &plane, &ty0, &tx0);
    const int64_t base = plane * ((int64_t)p.h * p.w);
    const int64_t all = (int64_t)p.n * p.c * p.h * p.w;
    (void)all;
    const int rows = p.th + 4 * R, cols = p.tw + 4 * R;
    for (int idx = ctx.tid; idx < rows * cols; idx += ctx.nth) {
        const int ri = idx / cols, ci = idx - ri * cols;
        const int hh = ty0 - 2 * R + ri, ww = tx0 - 2 * R + ci;
        float v = 0.0f;
        if (hh >= 0 && hh < p.h && ww >= 0 && ww < p.w) v = wtc_to_float(WTC_PAR(a.x, base + (int64_t)hh * p.w + ww, all));
        WTC_LDS(ctx, p.x.off + ri * p.x.pitch + ci + p.xs) = v;
    }
    for (int idx = ctx.tid; idx < p.th * p.tw; idx += ctx.nth) {
        const int ri = idx / p.tw, ci = idx - ri * p.tw;
        const float v = wtc_to_float(WTC_PAR(a.dy, base + (int64_t)(ty0 + ri) * p.w + tx0 + ci, all));
        WTC_LDS(ctx, p.dy.off + ri * p.dy.pitch + ci) = v;
    }
}

// Level j+1 of both maps over the unit: detail bands into LDS (x side over the
// half tile plus R, zero outside the level-(j+1) map), low-pass maps over the
// half tile to global memory.
template <typename TI, int K>
WTC_HD WTC_INLINE void wtc_wtile_analysis(const WtcWtileArgs<TI> &a, WtcWtileCtx &ctx, int u)
{
    constexpr int R = K / 2;
    const WtcWtilePlan &p = a.p;
    int64_t plane;
    int ty0, tx0;
    wtc_wtile_unit(p, ctx.c, u, &plane, &ty0, &tx0);
    const int h1 = p.h / 2, w1 = p.w / 2, i00 = ty0 / 2 - R, j00 = tx0 / 2 - R;
    const int rows = p.th / 2 + 2 * R, cols = p.tw / 2 + 2 * R;
    const int stx = p.bx.rows * p.bx.pitch, std_ = p.bd.rows * p.bd.pitch;
    const int64_t obase = plane * ((int64_t)h1 * w1);
    const int64_t oall = (int64_t)p.n * p.c * h1 * w1;
    (void)oall;
    for (int idx = ctx.tid; idx < rows * cols; idx += ctx.nth) {
        const int ri = idx / cols, ci = idx - ri * cols;
        const int i = i00 + ri, j = j00 + ci;
        float b1 = 0.0f, b2 = 0.0f, b3 = 0.0f, ll = 0.0f;
        if (i >= 0 && i < h1 && j >= 0 && j < w1) {
            // full-resolution row 2i is staged row 2i - (ty0 - 2R) = 2 ri
            const int s = p.x.off + (2 * ri) * p.x.pitch + 2 * ci + p.xs;
            const float x00 = WTC_LDS(ctx, s), x01 = WTC_LDS(ctx, s + 1);
            const float x10 = WTC_LDS(ctx, s + p.x.pitch), x11 = WTC_LDS(ctx, s + p.x.pitch + 1);
            const float sa = x00 + x01, sc = x10 + x11, da = x00 - x01, dc = x10 - x11;
            ll = sa + sc;
            b1 = sa - sc;
            b2 = da + dc;
            b3 = da - dc;
        }
        const int o = p.bx.off + ri * p.bx.pitch + ci;
        WTC_LDS(ctx, o) = b1;
        WTC_LDS(ctx, o + stx) = b2;
        WTC_LDS(ctx, o + 2 * stx) = b3;
        const bool inner = ri >= R && ri < rows - R && ci >= R && ci < cols - R;
        if (inner) WTC_PAR(a.ux, obase + (int64_t)i * w1 + j, oall) = ll;
    }
    for (int idx = ctx.tid; idx < (p.th / 2) * (p.tw / 2); idx += ctx.nth) {
        const int ri = idx / (p.tw / 2), ci = idx - ri * (p.tw / 2);
        const int s = p.dy.off + (2 * ri) * p.dy.pitch + 2 * ci;
        const float x00 = WTC_LDS(ctx, s), x01 = WTC_LDS(ctx, s + 1);
        const float x10 = WTC_LDS(ctx, s + p.dy.pitch), x11 = WTC_LDS(ctx, s + p.dy.pitch + 1);
        const float sa = x00 + x01, sc = x10 + x11, da = x00 - x01, dc = x10 - x11;
        const int o = p.bd.off + ri * p.bd.pitch + ci;
        WTC_LDS(ctx, o) = sa - sc;
        WTC_LDS(ctx, o + std_) = da + dc;
        WTC_LDS(ctx, o + 2 * std_) = da - dc;
        WTC_PAR(a.ud, obase + (int64_t)(ty0 / 2 + ri) * w1 + tx0 / 2 + ci, oall) = sa + sc;
    }
}

template <typename TI, int K>
WTC_HD WTC_INLINE void wtc_wtile_correlate(const WtcWtileArgs<TI> &a, WtcWtileCtx &ctx,
                                          float (&acc)[WTC_WT_QMAX][K * K + 1])
{
    const WtcWtilePlan &p = a.p;
    WtcWgradCtx<float, 1> lc;
    lc.lds = ctx.lds;
#ifdef WTC_EMULATE
    lc.lds_n = ctx.lds_n;
#endif
#pragma unroll
    for (int s = 0; s < WTC_WT_QMAX; ++s) {
        const int it = p.q * ctx.tid + s;
        if (s < p.q && it < p.npieces) {
            const int *tab = (const int *)&WTC_LDS(ctx, p.tab_off + 2 * it + 1) - 1;
            const unsigned t0 = (unsigned)tab[0], t1 = (unsigned)tab[1];
            wtc_wgrad_piece<float, K, 1>(lc, (int)(t0 & 0xffffu), (int)(t0 >> 16), (int)(t1 & 0xffu),
                                         (int)((t1 >> 8) & 0xffu), true, acc[s]);
        }
    }
}

template <typename TI, int K>
WTC_HD WTC_INLINE void wtc_wtile_park(const WtcWtileArgs<TI> &a, WtcWtileCtx &ctx, const float (&acc)[K * K + 1])
{
    constexpr int n1 = K * K + 1;
#pragma unroll
    for (int e = 0; e < n1; ++e) WTC_LDS(ctx, a.p.red_off + ctx.tid * n1 + e) = acc[e];
}

template <typename TI, int K>
WTC_HD WTC_INLINE void wtc_wtile_gather(const WtcWtileArgs<TI> &a, WtcWtileCtx &ctx, int s)
{
    constexpr int n1 = K * K + 1;
    const WtcWtilePlan &p = a.p;
    for (int idx = ctx.tid; idx < p.nmaps_here * n1; idx += ctx.nth) {
        const int g = idx / n1, e = idx - g * n1;
        const int lo = wtc_max(0, (p.first[g] - s + p.q - 1) / p.q);
        const int hi = wtc_min(p.nthreads, (p.first[g + 1] - s + p.q - 1) / p.q);
        float sum = WTC_LDS(ctx, p.res_off + idx);
        for (int t = lo; t < hi; ++t) sum += WTC_LDS(ctx, p.red_off + t * n1 + e);
        WTC_LDS(ctx, p.res_off + idx) = sum;
    }
}

// This step's maps into the partial row: map 0 is G_0 (+ G_b) on step 0 and
// the low-pass band of level j otherwise; maps 1..3 the detail bands of level
// j+1.
template <typename TI, int K>
WTC_HD WTC_INLINE void wtc_wtile_write(const WtcWtileArgs<TI> &a, WtcWtileCtx &ctx)
{
    constexpr int kk = K * K, n1 = kk + 1;
    const WtcWtilePlan &p = a.p;
    const int64_t row = ((int64_t)ctx.group * p.c + ctx.c) * p.plen;
    const int64_t all = (int64_t)p.groups * p.c * p.plen;
    (void)all;
    for (int idx = ctx.tid; idx < p.nmaps_here * n1; idx += ctx.nth) {
        const int g = idx / n1, e = idx - g * n1;
        int dst;
        if (g == 0) {
            if (p.step == 0) dst = e;  // G_0 then G_b
            else if (e < kk) dst = kk + 1 + (4 * (p.step - 1)) * kk + e;
            else continue;
        } else {
            if (e == kk) continue;
            dst = kk + 1 + (4 * p.step + g) * kk + e;
        }
        WTC_PAR(a.partial, row + dst, all) = WTC_LDS(ctx, p.res_off + idx);
    }
}

#endif  // WTCONV_WGRAD_TILE_BODY_H
