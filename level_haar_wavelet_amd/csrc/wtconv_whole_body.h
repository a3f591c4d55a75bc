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
//   * each thread stages a group of gr rows x vec columns of the input (one
//     load of at most 16 bytes per row; 4 columns where the width allows) and
//     computes Haar level 1, and level 2 when the group has 4 rows and 4
//     columns, from those registers; with L >= 3 the four lanes of a quad hold
//     a 2 x 2 block of groups and build level 3 by DPP exchange; deeper levels
//     are computed from LDS;
//   * every convolution -- the base one at full resolution and the four bands
//     of every level -- is cut into the same 4x4-output pieces, dealt
//     round-robin to the threads from a descriptor table built once per
//     workgroup, so the work is balanced and a wave runs one code path;
//   * maps are stored with their zero border at (r, r) and 16-byte rows, so a
//     piece's input window starts on a 16-byte boundary and is read with
//     128-bit LDS reads (consecutive lanes take consecutive column pieces);
//   * the base convolution's output goes to LDS like the level outputs, and a
//     last pass combines them per 2 x BW output block and stores y.
#ifndef WTCONV_WHOLE_BODY_H
#define WTCONV_WHOLE_BODY_H

#include "wtconv_fused_body.h"


struct WtcWholePlan {
    int32_t n, c, h, w, k, levels;
    int32_t rotate;
    int32_t nthreads;
    int32_t planes;      // images per workgroup (same channel)
    int32_t vec;         // activation elements per global chunk
    int32_t out_bw;      // output block width (2, 4 or 8)
    int32_t gr;          // input rows per staging group (2 or 4)
    int32_t groups;      // staging groups per image (one per thread at most)
    int32_t stage_l3;    // the staging also computes Haar level 3 (2 x 2 groups per lane quad)
    int32_t ws;          // floats per folded kernel (k*k rounded up to 4)
    WtcMap x;            // input with an r border, origin (r, r)
    WtcMap u[WTC_MAXL + 1];   // U_m plus three detail bands, m = 1..L, origin (r, r)
    WtcMap z[WTC_MAXL + 1];   // z[0]: base output; z[m]: four conv outputs of level m; origin (0, 0)
    int32_t wf_off;
    int32_t items;       // convolution pieces per image
    int32_t tail;        // the last `tail` pieces run as one-row pieces (see wtc_whole_layout)
    int32_t halves;      // every piece runs as two 2-row halves, one per thread (see wtc_whole_layout)
    int32_t tab_off;     // piece descriptors, 4 ints each
    int32_t lds_floats;
    // Tiling, for planes too large for one workgroup: h x w above is then one
    // tile of an ih x iw image and a unit of work is one (image, tile); lh
    // input rows and columns around the tile are loaded too (zero outside the
    // image), the maps are stored from origins that keep the convolution
    // windows on 16-byte boundaries, L is 1, and the low-pass contribution of
    // the deeper levels, computed beforehand at level-1 resolution, is added
    // before level 1's synthesis.  Untiled: ih = h, iw = w, one tile, lh = 0.
    int32_t tiled, ih, iw, tiles_x, tiles_y, units;
    int32_t lh;          // loaded halo (input pixels, a multiple of 4 and of vec)
    int32_t xr, xc;      // stored row / column of tile element (0, 0) in the input map
    int32_t u1r, u1c;    // the same for the level-1 maps (deeper maps: (r, r))
    // the base path is known to be zero (the deeper levels of a larger layer,
    // whose base scale is 0): no base convolution pieces, no base output read
    int32_t nobase;
    // Small planes: `stack` images of sh rows stacked down one plane of h
    // rows, separated by sgap zero rows (r rows at every level's resolution,
    // so no convolution window reaches from one image into the next); a unit
    // is then a stack of images.  1: one image per plane.  Stacked plans run
    // a kernel instance of their own (ST), so the others carry no checks.
    int32_t stack, sh, sgap;
    // The deeper levels' term in LDS (the fused large-plane kernel): an fp32
    // map of (ih/2) x (iw/2) at deep_off with row pitch deep_pitch, written by
    // the output pass of the deeper-levels plan and read by the tiled plan's
    // output pass in place of the global `low`.
    int32_t deep_off, deep_pitch;
};

#define WTC_WP 4  // piece side (outputs)

// Rows of 16 bytes, at least `cols` floats.
WTC_PLAN_HD static inline int32_t wtc_pitch16(int32_t cols) { return wtc_roundup(cols, 4); }

// Fills the LDS layout; returns the number of floats.
static inline int32_t wtc_whole_layout(WtcWholePlan *p)
{
    const int32_t L = p->levels, r = p->k / 2, kk = p->k * p->k, P = WTC_WP;
    int32_t off = 0;
    p->ws = wtc_roundup(kk, 4);
    p->wf_off = off;
    off += (1 + 4 * L) * p->ws;
    for (int32_t m = 0; m <= WTC_MAXL; ++m) {
        p->u[m].off = p->u[m].pitch = p->u[m].rows = 0;
        p->z[m] = p->u[m];
    }
    // input map: the base convolution's pieces read windows of P + 2r rows
    // (and roundup(P + 2r, 4) columns, as read) starting r before multiples of
    // P; the map holds the loaded region (the tile plus lh) and every window
    const int32_t NR = wtc_roundup(P + 2 * r, 4);
    p->x.off = off;
    p->x.rows = wtc_max(p->lh + p->h + p->xr, wtc_roundup(p->h, P) - P - r + p->xr + P + 2 * r);
    p->x.pitch = wtc_pitch16(wtc_max(p->lh + p->w + p->xc, wtc_roundup(p->w, P) - P - r + p->xc + NR));
    if (p->nobase) {
        // without the base path nothing reads the input map: one row with a
        // zero pitch takes the staging's stores (every row lands on it)
        off += p->x.pitch;
        p->x.rows = 1;
        p->x.pitch = 0;
    } else {
        off += p->x.rows * p->x.pitch;
    }
    for (int32_t m = 1; m <= L; ++m) {
        const int32_t Hm = p->h >> m, Wm = p->w >> m;
        const int32_t orow = m == 1 ? p->u1r : r, ocol = m == 1 ? p->u1c : r, lm = m == 1 ? p->lh / 2 : 0;
        p->u[m].off = off;
        p->u[m].rows = wtc_max(lm + Hm + orow, wtc_roundup(Hm, P) - P - r + orow + P + 2 * r);
        p->u[m].pitch = wtc_pitch16(wtc_max(lm + Wm + ocol, wtc_roundup(Wm, P) - P - r + ocol + NR));
        off += 4 * p->u[m].rows * p->u[m].pitch;
    }
    for (int32_t m = 0; m <= L; ++m) {
        const int32_t Hm = p->h >> m, Wm = p->w >> m;
        p->z[m].off = off;
        p->z[m].rows = wtc_roundup(Hm, P);
        p->z[m].pitch = wtc_pitch16(wtc_roundup(Wm, P));
        if (m == 0 && p->nobase) {
            // no base output: the output pass reads one zero row for every row
            off += p->z[0].pitch;
            p->z[0].rows = 1;
            p->z[0].pitch = 0;
            continue;
        }
        off += (m == 0 ? 1 : 4) * p->z[m].rows * p->z[m].pitch;
    }
    int32_t items = p->nobase ? 0 : ((p->h + P - 1) / P) * ((p->w + P - 1) / P);
    for (int32_t m = 1; m <= L; ++m) items += 4 * (((p->h >> m) + P - 1) / P) * (((p->w >> m) + P - 1) / P);
    p->items = items;
    // Pieces past the last full round of the workgroup's threads, when their
    // P one-row pieces fit one round, run as those (a quarter of a piece per
    // thread): otherwise a few threads would take a whole extra piece while
    // the rest of the workgroup waits at the barrier (the stacked 28 x 28
    // L = 2 plan, 272 pieces on 256 threads: forward 40.1 -> 36.4 us).  Tiled
    // plans have none (their kernel instances carry no tail loop).
    const int32_t rem = items % p->nthreads;
    p->tail = !p->tiled && items > p->nthreads && P * rem <= p->nthreads ? rem : 0;
    // Tiles without the base path have level 1's pieces only, half as many as
    // threads: as 2-row halves every wave (and so every SIMD) takes a share
    // instead of half the waves taking all of it.
    p->halves = p->tiled && p->nobase && 2 * items == p->nthreads;
    p->tab_off = off;
    off += 4 * items;
    p->lds_floats = wtc_roundup(off, 4);
    return p->lds_floats;
}

static inline int32_t wtc_whole_blocks(const WtcWholePlan *p) { return (p->h / 2) * (p->w / p->out_bw); }

// The staging phase computes Haar level 2 too (4-row groups of at least 4
// columns); the analysis phase then starts at level 3.
WTC_HD WTC_INLINE bool wtc_whole_stage_l2(const WtcWholePlan &p) { return p.gr == 4 && p.vec >= 4 && p.levels >= 2; }
WTC_HD WTC_INLINE int wtc_whole_first_deep(const WtcWholePlan &p)
{
    return p.stage_l3 ? 4 : (wtc_whole_stage_l2(p) ? 3 : 2);
}

// Plan of the whole-plane kernel on h x w planes (or tiles), or -1 when it
// does not fit (LDS, per-thread chunk or block limits).  `planes` is the
// requested number of units (images, or (image, tile) pairs) per workgroup.
static inline int wtc_whole_plan_common(WtcWholePlan *p, int32_t n, int32_t c, int32_t h, int32_t w, int32_t k,
                                        int32_t levels, int32_t rotate, int32_t nthreads, int32_t planes,
                                        int32_t elem_bytes, int32_t budget_floats, int32_t ih, int32_t iw,
                                        int32_t nobase, int32_t stack = 1)
{
    const int32_t r = k / 2;
    p->nobase = nobase && levels >= 1;
    p->stack = stack < 2 ? 1 : stack;
    p->sh = h;
    p->sgap = 0;
    if (p->stack > 1) {
        if (ih != h || iw != w || levels < 1 || levels > WTC_MAXL) return -1;
        if (h % wtc_max(4, 1 << levels)) return -1;  // whole staging groups and level cells per image
        p->sgap = wtc_roundup(r << levels, wtc_max(4, 1 << levels));
        h = p->stack * h + (p->stack - 1) * p->sgap;
        ih = h;
    }
    p->n = n;
    p->c = c;
    p->h = h;
    p->w = w;
    p->k = k;
    p->levels = levels;
    p->rotate = rotate;
    p->nthreads = nthreads;
    p->deep_off = p->deep_pitch = 0;
    p->tiled = ih != h || iw != w;
    p->ih = ih;
    p->iw = iw;
    if (h < 1 || w < 1 || ih % h || iw % w) return -1;
    p->tiles_y = ih / h;
    p->tiles_x = iw / w;
    p->units = n * p->tiles_y * p->tiles_x;
    if (p->stack > 1) p->units = (n + p->stack - 1) / p->stack;
    p->planes = planes < 1 ? 1 : (planes > p->units ? p->units : planes);
    // L = 0 (a plain depthwise convolution) needs even sides: the staging and
    // output passes work on 2-row groups and blocks
    if (levels < 0 || levels > WTC_MAXL) return -1;
    if (p->tiled && levels > 1) return -1;
    if (h % (2 << levels) && levels == 0) return -1;
    if (h % (1 << levels) || w % (1 << levels) || w % 2) return -1;
    // Output blocks of 2 x BW with BW = 4 (16-byte fp32 stores, 8-byte fp16
    // ones) where the row allows, doubled when blocks would be more than two
    // per thread; the kernel stages rows in segments of vec = min(BW, 16-byte
    // width) elements, a compile-time function of its BW.  Wider default
    // blocks are slower: 8-element fp16 segments put the staging's LDS writes
    // 32 bytes apart across lanes and double their bank conflicts.
    const int32_t wide = 16 / elem_bytes;
    int32_t bw = 4;
    while (bw > 2 && w % bw) bw /= 2;
    if (bw < 8 && (h / 2) * (w / bw) > 2 * nthreads && w % (2 * bw) == 0) bw *= 2;
    if (w % bw) return -1;
    p->out_bw = bw;
    const int32_t vec = bw < wide ? bw : wide;
    p->vec = vec;
    // staging groups of 4 rows where the height allows (their threads also
    // compute Haar level 2 when L >= 2 and vec >= 4), else 2
    p->gr = (h % 4 == 0 && vec >= 2) ? 4 : 2;
    // tiled and stacked instances assume 4-row groups
    if (p->stack > 1 && p->gr != 4) return -1;
    if (p->tiled) {
        // the tile plus 2r input pixels (level 1's convolution needs r level-1
        // pixels around the tile), rounded to whole staging segments and groups
        p->lh = wtc_roundup(wtc_max(2 * r, 1), wtc_max(4, vec));
        p->xr = p->lh;
        p->xc = p->lh + r;
        p->u1r = p->lh / 2;
        p->u1c = p->lh / 2 + ((r - p->lh / 2) % 4 + 4) % 4;
        if (p->gr != 4 || h % 4 || w % vec) return -1;
    } else {
        p->lh = 0;
        p->xr = p->xc = p->u1r = p->u1c = r;
    }
    // with L >= 3 and 4 x 4 groups (so 2^3 divides both sides and the group
    // grid has even sides), the four lanes of a quad take a 2 x 2 block of
    // groups and compute Haar level 3 from their level-2 sums by lane exchange
    p->stage_l3 = !p->tiled && levels >= 3 && p->gr == 4 && vec == 4;
    p->groups = ((h + 2 * p->lh) / p->gr) * ((w + 2 * p->lh) / vec);
    if (p->groups > nthreads) return -1;
    if (wtc_whole_blocks(p) > 2 * nthreads) return -1;
    wtc_whole_layout(p);
    return p->lds_floats <= budget_floats ? 0 : -1;
}

// nobase: the base path is zero (L >= 1 only; the base weights, bias and
// scale are then not read).
// stack: images stacked per plane (small planes; L >= 1).
static inline int wtc_make_whole_plan(WtcWholePlan *p, int32_t n, int32_t c, int32_t h, int32_t w, int32_t k,
                                      int32_t levels, int32_t rotate, int32_t nthreads, int32_t planes,
                                      int32_t elem_bytes, int32_t budget_floats, int32_t nobase = 0,
                                      int32_t stack = 1)
{
    return wtc_whole_plan_common(p, n, c, h, w, k, levels, rotate, nthreads, planes, elem_bytes, budget_floats, h,
                                 w, nobase, stack);
}

// Tiled plan: th x tw tiles of ih x iw images, L = 1 (plus the added low-pass
// term of the deeper levels) or L = 0 (a plain depthwise convolution).
static inline int wtc_make_whole_tile_plan(WtcWholePlan *p, int32_t n, int32_t c, int32_t ih, int32_t iw,
                                           int32_t th, int32_t tw, int32_t k, int32_t levels, int32_t rotate,
                                           int32_t nthreads, int32_t planes, int32_t elem_bytes,
                                           int32_t budget_floats, int32_t nobase = 0)
{
    if (th == ih && tw == iw) return -1;
    return wtc_whole_plan_common(p, n, c, th, tw, k, levels, rotate, nthreads, planes, elem_bytes, budget_floats,
                                 ih, iw, nobase);
}

template <typename T>
struct WtcWholeArgs {
    const T *in;
    T *out;
    const float *w_base, *bias, *s_base, *w_lvl, *s_lvl;
    WtcWholePlan p;
    // tiled plans: the deeper levels' low-pass contribution at level-1
    // resolution, (N, C, ih/2, iw/2) orthonormal, fp32 whatever T is (the
    // outputs are rounded once, at the store), or null
    const float *low = nullptr;
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
    // staging group of this thread (gvalid: it has one) and its prefetched
    // input rows (as loaded: T)
    int grow, gcol;
    bool gvalid;
    int oblk;  // this thread's first output block: row << 16 | column (set once)
    int ty0, tx0;  // current unit's tile origin in the image
    int64_t plane;  // current unit's plane index (n * C + c)
    int vmask;     // rows of the prefetched group that lie in the image (bit q)
    float u2;      // the group's level-2 low-pass sum (for level 3 across the lane quad)
    int cur;       // unit of the output pass (stacked plans)
    T pre[4][16 / sizeof(T)];
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
    // consecutive workgroups take consecutive channels of the same group of
    // units (images, or (image, tile) pairs with the tiles of an image
    // consecutive)
    ctx.c = bid % p.c;
    const int g = bid / p.c;
    ctx.n0 = g * p.planes;
    ctx.nimg = wtc_min(p.planes, p.units - ctx.n0);
    float b = 0.0f;
    if (!p.rotate && !p.nobase && a.bias) b = a.s_base[ctx.c] * a.bias[ctx.c];
    ctx.bias = b;
    const int gpr = (p.w + 2 * p.lh) / p.vec;
    const int grp = wtc_min(ctx.tid, p.groups - 1);  // threads past the last group repeat it, unstored
    ctx.gvalid = ctx.tid < p.groups;
    if (p.stage_l3) {
        // lane quad q takes groups (2 qr + dr, 2 qc + dc), dr, dc from lane bits
        // 1 and 0 (the group count is a multiple of 4, so quads are whole)
        const int q = grp >> 2, qr = q / (gpr / 2), qc = q - qr * (gpr / 2);
        ctx.grow = 2 * qr + ((grp >> 1) & 1);
        ctx.gcol = 2 * qc + (grp & 1);
    } else {
        ctx.grow = grp / gpr;
        ctx.gcol = grp - ctx.grow * gpr;
    }
    const int nbx = p.w / p.out_bw, by = ctx.tid / nbx;
    ctx.oblk = (by << 16) | (ctx.tid - by * nbx);
}

// Image plane and tile origin of unit `u` of the workgroup.
template <typename T>
WTC_HD WTC_INLINE void wtc_whole_unit(const WtcWholeArgs<T> &a, const WtcWholeCtx<T> &ctx, int u, int64_t &plane,
                                      int &ty0, int &tx0)
{
    const WtcWholePlan &p = a.p;
    const int tiles = p.tiles_x * p.tiles_y, unit = ctx.n0 + u;
    const int img = unit / tiles, t = unit - img * tiles;
    const int ty = t / p.tiles_x;
    plane = (int64_t)img * p.c + ctx.c;
    ty0 = ty * p.h;
    tx0 = (t - ty * p.tiles_x) * p.w;
}

template <typename T, bool ST = false>
WTC_HD WTC_INLINE void wtc_whole_select(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx, int img)
{
    const int64_t hw = (int64_t)a.p.ih * a.p.iw;
    wtc_whole_unit(a, ctx, img, ctx.plane, ctx.ty0, ctx.tx0);
    if constexpr (ST) {
        // stacked plans address every output row on its own, from the tensor base
        ctx.cur = img;
        ctx.in = a.in;
        ctx.out = a.out;
    } else {
        ctx.in = a.in + ctx.plane * hw;
        ctx.out = a.out + ctx.plane * hw;
    }
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
            v = p.nobase ? 0.0f : WTC_PAR(a.s_base, c, C) * WTC_PAR(a.w_base, c * kk + se, (int64_t)C * kk);
        } else {
            const int m = (blk - 1) / 4 + 1, b = (blk - 1) % 4;
            const int ch = (m - 1) * 4 * C + 4 * c + b;
            const float s = WTC_PAR(a.s_lvl, ch, (int64_t)p.levels * 4 * C);
            v = ldexpf(s * WTC_PAR(a.w_lvl, (int64_t)ch * kk + se, (int64_t)p.levels * 4 * C * kk), -2 * m);
        }
        WTC_LDS(ctx, p.wf_off + blk * p.ws + e) = v;
    }
}

#ifndef WTC_EMULATE
// Input loads: non-temporal where every element is read once (whole planes);
// plain in tiled plans, whose halos are read again by the neighbouring tiles
// (the same workgroup's next units), so the lines are worth keeping in L2.
template <typename V, bool NT>
static __device__ __forceinline__ V wtc_stream_load(const V *p)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}
#endif

// Elements per global chunk: 16 bytes, or the output block width if smaller
// (the plan picks the same value from the image width).
template <typename T, int BW>
struct WtcVec {
    static constexpr int v = BW < (int)(16 / sizeof(T)) ? BW : (int)(16 / sizeof(T));
};

// Issue the loads of image `img` of the workgroup into registers: this
// thread's staging group, gr rows of vec elements (every lane loads a valid
// group, so that no branch surrounds the loads).
// TL: tiled plan (halo loads, bounds, shifted map origins, the added
// low-pass term); untiled plans compile without any of it.
template <typename T, int K, int BW, bool TL, bool ST = false, bool G4 = TL || ST>
WTC_HD WTC_INLINE void wtc_whole_load(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx, int img)
{
    const WtcWholePlan &p = a.p;
    constexpr int vec = WtcVec<T, BW>::v;
#ifndef WTC_EMULATE
    // Everything still in flight here was issued a phase or more ago (the
    // previous prefetch, consumed by the staging just before, and older
    // output stores): waiting for it now costs nothing and tells the
    // compiler's wait insertion that the prefetch registers are free, so the
    // loads below issue back to back (vmcnt 0, expcnt and lgkmcnt unchanged).
    __builtin_amdgcn_s_waitcnt(0x0F70);
#endif
    int64_t plane;
    int ty0 = 0, tx0 = 0;
    int grow0 = p.gr * ctx.grow;  // the group's first row in its image
    bool sval = true;             // stacked plans: the group lies in an image
    if constexpr (TL) {
        wtc_whole_unit(a, ctx, img, plane, ty0, tx0);
    } else if constexpr (ST) {
        // image `sub` of the stack, or the zero rows between images (or an
        // image past the batch): those load image 0's first rows and are
        // zeroed when staged
        const int per = p.sh + p.sgap, sub = grow0 / per;
        const int im = (ctx.n0 + img) * p.stack + sub;
        grow0 -= sub * per;
        sval = grow0 < p.sh && im < p.n;
        plane = (int64_t)(sval ? im : 0) * p.c + ctx.c;
        if (!sval) grow0 = 0;
    } else {
        plane = (int64_t)(ctx.n0 + img) * p.c + ctx.c;
    }
    const T *src = a.in + plane * ((int64_t)(ST ? p.sh : p.ih) * p.iw);
    if constexpr (TL) {
        // Tiled plans load through a buffer resource over the image plane:
        // the hardware returns zeros for every offset past the plane, which
        // is what the rows above and below the image get (a negative offset
        // reads as a large unsigned one); segments left or right of the image
        // are sent past the plane.  No clamp, no mask, no select.
        const int row0 = ty0 - p.lh + grow0, col = tx0 - p.lh + vec * ctx.gcol;
        const bool colok = col >= 0 && col < p.iw;
        // a column past any plane (sides <= 4096: offsets stay below 2^31);
        // one select, so that the loads below need no branch
        const int colx = colok ? col : (1 << 27);
        const int plane_bytes = p.ih * p.iw * (int)sizeof(T);
#ifndef WTC_EMULATE
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, plane_bytes, 0x00020000);
#endif
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = row0 + q;
            const int off = (row * p.iw + colx) * (int)sizeof(T);
#ifdef WTC_EMULATE
            // the hardware's rule: a load whose bytes lie past the range
            // (the offset read as unsigned) returns zeros; it must agree with
            // the segment lying in the image
            const bool ok = (uint64_t)(uint32_t)off + vec * sizeof(T) <= (uint64_t)plane_bytes;
            if (ok != (colok && row >= 0 && row < p.ih)) {
                fprintf(stderr, "wtconv emulation: buffer range check disagrees at row %d col %d\n", row, col);
                abort();
            }
            const int64_t base = src - a.in, all = (int64_t)p.n * p.c * p.ih * p.iw;
            for (int t = 0; t < vec; ++t)
                ctx.pre[q][t] = ok ? wtc_chk(a.in, base + (int64_t)row * p.iw + col + t, all, __LINE__) : (T)0.0f;
#else
            if constexpr (vec * sizeof(T) == 16) {
                const auto d = __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)off, 0, 0);
                __builtin_memcpy(&ctx.pre[q][0], &d, 16);
            } else if constexpr (vec * sizeof(T) == 8) {
                const auto d = __builtin_amdgcn_raw_buffer_load_b64(rs, (unsigned)off, 0, 0);
                __builtin_memcpy(&ctx.pre[q][0], &d, 8);
            } else if constexpr (vec * sizeof(T) == 4) {
                const auto d = __builtin_amdgcn_raw_buffer_load_b32(rs, (unsigned)off, 0, 0);
                __builtin_memcpy(&ctx.pre[q][0], &d, 4);
            } else {
                const auto d = __builtin_amdgcn_raw_buffer_load_b16(rs, (unsigned)off, 0, 0);
                __builtin_memcpy(&ctx.pre[q][0], &d, 2);
            }
#endif
        }
        ctx.vmask = 0xF;
        return;
    }
    // image row / column of the group's first element
    const int lh = TL ? p.lh : 0;
    const int row0 = ty0 - lh + grow0, col = tx0 - lh + vec * ctx.gcol;
    const bool colok = !TL || (col >= 0 && col < p.iw);
    const int ccol = TL ? wtc_min(wtc_max(col, 0), p.iw - vec) : col;
    int vm = 0;
    // untiled: one base offset plus q rows (the address stays in one register
    // pair, so no prefetch load waits on the one before it)
    const int64_t e0 = (int64_t)row0 * p.iw + col;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (G4 || q < p.gr) {
            const int row = row0 + q;
            vm |= (TL ? (colok && row >= 0 && row < p.ih) : (!ST || sval)) ? (1 << q) : 0;
            const int64_t e = TL ? (int64_t)wtc_min(wtc_max(row, 0), p.ih - 1) * p.iw + ccol
                                 : e0 + (int64_t)q * p.iw;
#ifdef WTC_EMULATE
            const int64_t base = src - a.in, all = (int64_t)p.n * p.c * (ST ? p.sh : p.ih) * p.iw;
            for (int t = 0; t < vec; ++t) ctx.pre[q][t] = wtc_chk(a.in, base + e + t, all, __LINE__);
#else
            if constexpr (vec * sizeof(T) == 16) {
                typedef float v4 __attribute__((ext_vector_type(4)));
                v4 d = wtc_stream_load<v4, !TL>((const v4 *)(src + e));
                __builtin_memcpy(&ctx.pre[q][0], &d, 16);
            } else if constexpr (vec * sizeof(T) == 8) {
                typedef float v2 __attribute__((ext_vector_type(2)));
                v2 d = wtc_stream_load<v2, !TL>((const v2 *)(src + e));
                __builtin_memcpy(&ctx.pre[q][0], &d, 8);
            } else if constexpr (vec * sizeof(T) == 4) {
                float d = wtc_stream_load<float, !TL>((const float *)(src + e));
                __builtin_memcpy(&ctx.pre[q][0], &d, 4);
            } else {
#pragma unroll
                for (int t = 0; t < vec; ++t) ctx.pre[q][t] = src[e + t];
            }
#endif
        }
    }
    ctx.vmask = vm;
}

// N floats to LDS at an index that is a multiple of A (16-, 8- or 4-byte stores).
template <int N, int A, typename Ctx>
WTC_HD WTC_INLINE void wtc_lds_put(Ctx &ctx, int idx, const float (&src)[N])
{
#ifdef WTC_EMULATE
    if (idx % A) {
        fprintf(stderr, "wtconv emulation: LDS index %d not a multiple of %d\n", idx, A);
        abort();
    }
    for (int e = 0; e < N; ++e) WTC_LDS(ctx, idx + e) = src[e];
#else
    if constexpr (A >= 4 && N % 4 == 0) {
        typedef float v4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int q = 0; q < N / 4; ++q) {
            v4 v;
            v.x = src[4 * q];
            v.y = src[4 * q + 1];
            v.z = src[4 * q + 2];
            v.w = src[4 * q + 3];
            *(v4 *)&ctx.lds[idx + 4 * q] = v;
        }
    } else if constexpr (A >= 2 && N % 2 == 0) {
        typedef float v2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int q = 0; q < N / 2; ++q) {
            v2 v;
            v.x = src[2 * q];
            v.y = src[2 * q + 1];
            *(v2 *)&ctx.lds[idx + 2 * q] = v;
        }
    } else {
#pragma unroll
        for (int e = 0; e < N; ++e) ctx.lds[idx + e] = src[e];
    }
#endif
}

// largest of 4, 2, 1 dividing both a and b (a, b powers of two or 0 for "any")
WTC_HD constexpr int wtc_align_of(int a, int b)
{
    const int la = a == 0 ? 4 : (a % 4 == 0 ? 4 : (a % 2 == 0 ? 2 : 1));
    const int lb = b == 0 ? 4 : (b % 4 == 0 ? 4 : (b % 2 == 0 ? 2 : 1));
    return la < lb ? la : lb;
}

// Haar level 3 of a 2 x 2 block of staging groups from the level-2 sums
// v[0..3] of its four lanes (top-left, top-right, bottom-left, bottom-right):
// lane dr dc of the quad writes band 2 dr + dc of the block's level-3 cell.
template <typename T>
WTC_HD WTC_INLINE void wtc_whole_stage_l3(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx, const float (&v)[4])
{
    const WtcWholePlan &p = a.p;
    const int R = p.k / 2;
    const WtcMap u3 = p.u[3];
    const float sa = v[0] + v[1], sc = v[2] + v[3], da = v[0] - v[1], dc = v[2] - v[3];
    const int band = 2 * (ctx.grow & 1) + (ctx.gcol & 1);
    const float val = band == 0 ? sa + sc : (band == 1 ? sa - sc : (band == 2 ? da + dc : da - dc));
    const int o = u3.off + band * u3.rows * u3.pitch + wtc_mul24((ctx.grow >> 1) + R, u3.pitch) + (ctx.gcol >> 1) + R;
    WTC_LDS(ctx, o) = val;
}

// Write the prefetched group into the input map and compute Haar level 1
// (and level 2 when the group has 4 rows) of it straight from registers:
//   U_1 and B_1^1..3 at the group's (gr/2) x (vec/2) level-1 positions,
//   U_2 and B_2^1..3 at its 1 x (vec/4) level-2 positions.
// G4: the plan's staging groups are known to have 4 rows (tiled and stacked
// plans always; whole-plane plans where the launch checked it), so no row of a
// group needs a test.
template <typename T, int K, int BW, bool TL, bool ST = false, bool G4 = TL || ST, int LV = 0>
WTC_HD WTC_INLINE void wtc_whole_stage_vals(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx,
                                            const float (&x)[4][WtcVec<T, BW>::v]);

template <typename T, int K, int BW, bool TL, bool ST = false, bool G4 = TL || ST>
WTC_HD WTC_INLINE void wtc_whole_stage(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    constexpr int vec = WtcVec<T, BW>::v;
    const WtcWholePlan &p = a.p;
    if (!ctx.gvalid) return;
    float x[4][vec];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < vec; ++t)
            x[q][t] = ((G4 || q < p.gr) && (!ST || ((ctx.vmask >> q) & 1))) ? wtc_to_float(ctx.pre[q][t]) : 0.0f;
    wtc_whole_stage_vals<T, K, BW, TL, ST, G4>(a, ctx, x);
}

// The staging of a group from its values (gr rows of vec fp32 values): the
// input map, Haar level 1 and (4-row groups) level 2, and with L >= 3 the
// lane-quad exchange for level 3.
template <typename T, int K, int BW, bool TL, bool ST, bool G4, int LV>
WTC_HD WTC_INLINE void wtc_whole_stage_vals(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx,
                                            const float (&x)[4][WtcVec<T, BW>::v])
{
    constexpr int R = K / 2;
    constexpr int vec = WtcVec<T, BW>::v, h1 = vec / 2, h2 = vec / 4 > 0 ? vec / 4 : 1;
    const WtcWholePlan &p = a.p;
    if (!ctx.gvalid) return;
    const WtcMap xm = p.x, u1 = p.u[1];
    const int st1 = u1.rows * u1.pitch;
    // r0, c0: the group's position in the loaded region (the tile plus lh);
    // map origins are the plan's in tiled plans, (r, r) otherwise
    const int lh = TL ? p.lh : 0, xr = TL ? p.xr : R, xc = TL ? p.xc : R;
    const int u1r = TL ? p.u1r : R, u1c = TL ? p.u1c : R;
    const int r0 = p.gr * ctx.grow, c0 = vec * ctx.gcol;
    const int xo = xm.off + wtc_mul24(r0 - lh + xr, xm.pitch) + c0 - lh + xc;
    // the x map's origin column is r (mod 4) and c0 a multiple of vec: 8-byte
    // stores for even r (two per 4-element row: half the bank conflicts of
    // 4-byte stores from lanes 16 bytes apart)
    // without the base path nothing reads the input map (a scalar branch:
    // its one zero-pitch row would take every thread's stores)
    if (!p.nobase) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (G4 || q < p.gr) wtc_lds_put<vec, wtc_align_of(vec, R)>(ctx, xo + wtc_mul24(q, xm.pitch), x[q]);
    }
    const int lv = LV ? LV : p.levels;  // LV: the plan's levels, known at compile time (0: not)
    if (lv < 1) return;
    // level 1: 2x2 blocks (rows 2a, 2a+1; columns 2b, 2b+1) of the group
    float ll[2][h1];
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
        if (G4 || 2 * aa < p.gr) {
            const int i = (r0 - lh) / 2 + aa;
            float bnd[4][h1];
#pragma unroll
            for (int bb = 0; bb < h1; ++bb) {
                const float x00 = x[2 * aa][2 * bb], x01 = x[2 * aa][2 * bb + 1];
                const float x10 = x[2 * aa + 1][2 * bb], x11 = x[2 * aa + 1][2 * bb + 1];
                const float sa = x00 + x01, sc = x10 + x11, da = x00 - x01, dc = x10 - x11;
                ll[aa][bb] = sa + sc;
                bnd[0][bb] = sa + sc;
                bnd[1][bb] = sa - sc;
                bnd[2][bb] = da + dc;
                bnd[3][bb] = da - dc;
            }
            // origin column u1c = r (mod 4), (c0 - lh) / 2 a multiple of h1
            const int o = u1.off + wtc_mul24(i + u1r, u1.pitch) + (c0 - lh) / 2 + u1c;
#pragma unroll
            for (int b = 0; b < 4; ++b) wtc_lds_put<h1, wtc_align_of(h1, R)>(ctx, o + b * st1, bnd[b]);
        }
    }
    // tiled plans carry levels 0 and 1 only (their deeper levels come from
    // another pass or plan)
    if (!TL && vec >= 4 && (LV ? G4 && LV >= 2 : wtc_whole_stage_l2(p))) {
        const WtcMap u2 = p.u[2];
        const int st2 = u2.rows * u2.pitch;
#pragma unroll
        for (int bb = 0; bb < h2; ++bb) {
            const float x00 = ll[0][2 * bb], x01 = ll[0][2 * bb + 1];
            const float x10 = ll[1][2 * bb], x11 = ll[1][2 * bb + 1];
            const float sa = x00 + x01, sc = x10 + x11, da = x00 - x01, dc = x10 - x11;
            const int o = u2.off + wtc_mul24(ctx.grow + R, u2.pitch) + c0 / 4 + bb + R;
            WTC_LDS(ctx, o) = sa + sc;
            WTC_LDS(ctx, o + st2) = sa - sc;
            WTC_LDS(ctx, o + 2 * st2) = da + dc;
            WTC_LDS(ctx, o + 3 * st2) = da - dc;
            ctx.u2 = sa + sc;
        }
    }
#ifndef WTC_EMULATE
    if (!TL && (LV ? G4 && vec == 4 && LV >= 3 : p.stage_l3)) {
        // the quad's four level-2 sums (lanes: top-left, top-right,
        // bottom-left, bottom-right), broadcast within the quad by DPP
        float v[4];
        v[0] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ctx.u2), 0x00, 0xf, 0xf, false));
        v[1] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ctx.u2), 0x55, 0xf, 0xf, false));
        v[2] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ctx.u2), 0xaa, 0xf, 0xf, false));
        v[3] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(ctx.u2), 0xff, 0xf, 0xf, false));
        wtc_whole_stage_l3(a, ctx, v);
    }
#endif
}

// Level-m analysis from U_{m-1} in LDS, for the levels the staging phase did
// not compute.
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
        const int s = sm.off + wtc_mul24(2 * i + R, sm.pitch) + 2 * j + R;
        const float x00 = WTC_LDS(ctx, s), x01 = WTC_LDS(ctx, s + 1);
        const float x10 = WTC_LDS(ctx, s + sm.pitch), x11 = WTC_LDS(ctx, s + sm.pitch + 1);
        const float sa = x00 + x01, sc = x10 + x11, da = x00 - x01, dc = x10 - x11;
        const int o = um.off + wtc_mul24(i + R, um.pitch) + j + R;
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

// Piece descriptors, built once per workgroup (they depend only on the plan).
// Piece order: the base map (full resolution), then band 0..3 of level 1, 2,
// ...; inside a map, column pieces fastest.  Four ints:
//   d0 = LDS index of the input window (stored row P pr, column P pc, i.e.
//        map element (P pr - r, P pc - r)), a multiple of 4
//   d1 = LDS index of the first output in the output map
//   d2 = input pitch | output pitch << 16
//   d3 = LDS index of the folded weights | (1 << 16 for the base map)
template <typename T, int K, int BW>
WTC_HD WTC_INLINE void wtc_whole_table(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    constexpr int P = WTC_WP;
    const WtcWholePlan &p = a.p;
    // without the base path the pieces start at level 1's
    const int skip = p.nobase ? ((p.h + P - 1) / P) * ((p.w + P - 1) / P) : 0;
    for (int it = ctx.tid; it < p.items; it += ctx.nth) {
        int rem = it + skip, g = 0, npc = 0, npr = 0, m = 0, b = 0;
        for (;;) {
            m = g == 0 ? 0 : (g - 1) / 4 + 1;
            b = g == 0 ? 0 : (g - 1) % 4;
            npr = ((p.h >> m) + P - 1) / P;
            npc = ((p.w >> m) + P - 1) / P;
            if (rem < npr * npc) break;
            rem -= npr * npc;
            ++g;
        }
        const int pr = rem / npc, pc = rem - pr * npc;
        const WtcMap im = m == 0 ? p.x : p.u[m], om = p.z[m];
        // window of output (P pr, P pc): map element (P pr - r, P pc - r),
        // stored at that plus the map's origin
        const int orow = m == 0 ? p.xr : (m == 1 ? p.u1r : K / 2), ocol = m == 0 ? p.xc : (m == 1 ? p.u1c : K / 2);
        const int d0 = im.off + b * im.rows * im.pitch + (P * pr - K / 2 + orow) * im.pitch + P * pc - K / 2 + ocol;
        const int d1 = om.off + b * om.rows * om.pitch + (P * pr) * om.pitch + P * pc;
        const int d2 = im.pitch | (om.pitch << 16);
        const int d3 = (p.wf_off + g * p.ws) | ((g == 0) << 16);
        int *tab = (int *)&WTC_LDS(ctx, p.tab_off + 4 * it + 3) - 3;
        tab[0] = d0;
        tab[1] = d1;
        tab[2] = d2;
        tab[3] = d3;
    }
}

// N consecutive LDS floats starting at a multiple of 4 (16-byte reads).
#ifdef WTC_EMULATE
// the vector LDS accesses need their natural alignment (16 or 8 bytes)
static inline void wtc_check_align(int idx, int n, int line)
{
    const int a = n % 4 == 0 ? 4 : (n == 2 ? 2 : 1);
    if (idx % a) {
        fprintf(stderr, "wtconv emulation: LDS index %d of a %d-float access not aligned (line %d)\n", idx, n, line);
        abort();
    }
}
#endif

template <typename T, int N, typename Ctx>
WTC_HD WTC_INLINE void wtc_lds_row(Ctx &ctx, int idx, float (&dst)[N])
{
#ifdef WTC_EMULATE
    wtc_check_align(idx, N, __LINE__);
    for (int e = 0; e < N; ++e) dst[e] = WTC_LDS(ctx, idx + e);
#else
    typedef float v4 __attribute__((ext_vector_type(4)));
    static_assert(N % 4 == 0, "16-byte LDS rows");
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
        const v4 v = *(const v4 *)&ctx.lds[idx + 4 * q];
        dst[4 * q] = v.x;
        dst[4 * q + 1] = v.y;
        dst[4 * q + 2] = v.z;
        dst[4 * q + 3] = v.w;
    }
#endif
}

// N consecutive LDS floats starting at an index aligned to min(N, 4).
template <typename T, int N, typename Ctx>
WTC_HD WTC_INLINE void wtc_lds_vec(Ctx &ctx, int idx, float (&dst)[N])
{
#ifdef WTC_EMULATE
    wtc_check_align(idx, N, __LINE__);
    for (int e = 0; e < N; ++e) dst[e] = WTC_LDS(ctx, idx + e);
#else
    if constexpr (N % 4 == 0) {
        wtc_lds_row<T, N>(ctx, idx, dst);
    } else if constexpr (N == 2) {
        typedef float v2 __attribute__((ext_vector_type(2)));
        const v2 v = *(const v2 *)&ctx.lds[idx];
        dst[0] = v.x;
        dst[1] = v.y;
    } else {
#pragma unroll
        for (int e = 0; e < N; ++e) dst[e] = ctx.lds[idx + e];
    }
#endif
}

template <typename T, int N, typename Ctx>
WTC_HD WTC_INLINE void wtc_lds_store4(Ctx &ctx, int idx, const float (&src)[N])
{
#ifdef WTC_EMULATE
    wtc_check_align(idx, N, __LINE__);
    for (int e = 0; e < N; ++e) WTC_LDS(ctx, idx + e) = src[e];
#else
    typedef float v4 __attribute__((ext_vector_type(4)));
    static_assert(N % 4 == 0, "16-byte LDS rows");
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
        v4 v;
        v.x = src[4 * q];
        v.y = src[4 * q + 1];
        v.z = src[4 * q + 2];
        v.w = src[4 * q + 3];
        *(v4 *)&ctx.lds[idx + 4 * q] = v;
    }
#endif
}

// One output row of P columns of piece `it` (row r0 of the piece).
template <typename T, int K>
WTC_HD WTC_INLINE void wtc_whole_row_piece(const WtcWholePlan &p, WtcWholeCtx<T> &ctx, int it, int r0)
{
    constexpr int P = WTC_WP, KK = K * K, WS = (KK + 3) / 4 * 4;
    constexpr int NW = P + K - 1, NR = (NW + 3) / 4 * 4;  // window width, as read
    int dsc[4];
    {
        float tmp[4];
        wtc_lds_row<T, 4>(ctx, p.tab_off + 4 * it, tmp);
        for (int e = 0; e < 4; ++e) {
#ifdef WTC_EMULATE
            __builtin_memcpy(&dsc[e], &tmp[e], 4);
#else
            dsc[e] = __float_as_int(tmp[e]);
#endif
        }
    }
    const int ip = dsc[2] & 0xffff, op = dsc[2] >> 16;
    const int src = dsc[0] + r0 * ip, dst = dsc[1] + r0 * op;
    const int wk = dsc[3] & 0xffff;
    const float init = (dsc[3] >> 16) ? ctx.bias : 0.0f;
    float wv[WS];
    wtc_lds_row<T, WS>(ctx, wk, wv);
    float acc[P];
#pragma unroll
    for (int dc = 0; dc < P; ++dc) acc[dc] = init;
#pragma unroll
    for (int u = 0; u < K; ++u) {
        float row[NR];
        wtc_lds_row<T, NR>(ctx, src + u * ip, row);
#pragma unroll
        for (int v = 0; v < K; ++v)
#pragma unroll
            for (int dc = 0; dc < P; ++dc) acc[dc] = wtc_fma(wv[u * K + v], row[dc + v], acc[dc]);
    }
    wtc_lds_store4<T, P>(ctx, dst, acc);
}

// R output rows of P columns of piece `it`, from its row r0 (plans with
// halves: two threads to a piece).
template <typename T, int K, int R>
WTC_HD WTC_INLINE void wtc_whole_piece_rows(const WtcWholePlan &p, WtcWholeCtx<T> &ctx, int it, int r0)
{
    constexpr int P = WTC_WP, KK = K * K, WS = (KK + 3) / 4 * 4;
    constexpr int NW = P + K - 1, NR = (NW + 3) / 4 * 4;  // window width, as read
    int dsc[4];
    {
        float tmp[4];
        wtc_lds_row<T, 4>(ctx, p.tab_off + 4 * it, tmp);
        for (int e = 0; e < 4; ++e) {
#ifdef WTC_EMULATE
            __builtin_memcpy(&dsc[e], &tmp[e], 4);
#else
            dsc[e] = __float_as_int(tmp[e]);
#endif
        }
    }
    const int ip = dsc[2] & 0xffff, op = dsc[2] >> 16;
    const int src = dsc[0] + r0 * ip, dst = dsc[1] + r0 * op;
    const int wk = dsc[3] & 0xffff;
    const float init = (dsc[3] >> 16) ? ctx.bias : 0.0f;
    float wv[WS];
    wtc_lds_row<T, WS>(ctx, wk, wv);
    float acc[R][P];
#pragma unroll
    for (int dr = 0; dr < R; ++dr)
#pragma unroll
        for (int dc = 0; dc < P; ++dc) acc[dr][dc] = init;
    float row[NR];
    wtc_lds_row<T, NR>(ctx, src, row);
#pragma unroll
    for (int t = 0; t < R + K - 1; ++t) {
        float nxt[NR];
        if (t + 1 < R + K - 1) wtc_lds_row<T, NR>(ctx, src + (t + 1) * ip, nxt);
#pragma unroll
        for (int dr = 0; dr < R; ++dr) {
            const int u = t - dr;
            if (u < 0 || u >= K) continue;
#pragma unroll
            for (int v = 0; v < K; ++v)
#pragma unroll
                for (int dc = 0; dc < P; ++dc) acc[dr][dc] = wtc_fma(wv[u * K + v], row[dc + v], acc[dr][dc]);
        }
        if (t + 1 < R + K - 1) {
#pragma unroll
            for (int e = 0; e < NR; ++e) row[e] = nxt[e];
        }
    }
#pragma unroll
    for (int dr = 0; dr < R; ++dr) wtc_lds_store4<T, P>(ctx, dst + dr * op, acc[dr]);
}

// The convolution phase: every thread computes pieces tid, tid + nth, ...,
// then one-row pieces of the plan's tail (four lanes to a piece).  TAIL =
// false: an instance whose plans have no tail (tiles, the large-plane
// kernel), compiled without that loop.  HALF: an instance whose plans run
// every piece as two 2-row halves (plans with halves).
template <typename T, int K, int BW, bool TAIL = true, bool HALF = false>
WTC_HD WTC_INLINE void wtc_whole_conv(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    constexpr int P = WTC_WP, KK = K * K, WS = (KK + 3) / 4 * 4;
    constexpr int NW = P + K - 1, NR = (NW + 3) / 4 * 4;  // window width, as read
    const WtcWholePlan &p = a.p;
    if constexpr (HALF) {
        for (int it = ctx.tid; it < 2 * p.items; it += ctx.nth)
            wtc_whole_piece_rows<T, K, 2>(p, ctx, it >> 1, 2 * (it & 1));
        return;
    }
    const int full = p.items - p.tail;
    for (int it = ctx.tid; it < full; it += ctx.nth) {
        int dsc[4];
        {
            float tmp[4];
            wtc_lds_row<T, 4>(ctx, p.tab_off + 4 * it, tmp);
            for (int e = 0; e < 4; ++e) {
#ifdef WTC_EMULATE
                __builtin_memcpy(&dsc[e], &tmp[e], 4);
#else
                dsc[e] = __float_as_int(tmp[e]);
#endif
            }
        }
        const int src = dsc[0], dst = dsc[1];
        const int ip = dsc[2] & 0xffff, op = dsc[2] >> 16;
        const int wk = dsc[3] & 0xffff;
        const float init = (dsc[3] >> 16) ? ctx.bias : 0.0f;
        float wv[WS];
        wtc_lds_row<T, WS>(ctx, wk, wv);
        float acc[P][P];
#pragma unroll
        for (int dr = 0; dr < P; ++dr)
#pragma unroll
            for (int dc = 0; dc < P; ++dc) acc[dr][dc] = init;
        float row[NR];
        wtc_lds_row<T, NR>(ctx, src, row);
#pragma unroll
        for (int t = 0; t < P + K - 1; ++t) {
            float nxt[NR];
            if (t + 1 < P + K - 1) wtc_lds_row<T, NR>(ctx, src + (t + 1) * ip, nxt);
#pragma unroll
            for (int dr = 0; dr < P; ++dr) {
                const int u = t - dr;
                if (u < 0 || u >= K) continue;
#pragma unroll
                for (int v = 0; v < K; ++v)
#pragma unroll
                    for (int dc = 0; dc < P; ++dc) acc[dr][dc] = wtc_fma(wv[u * K + v], row[dc + v], acc[dr][dc]);
            }
            if (t + 1 < P + K - 1) {
#pragma unroll
                for (int e = 0; e < NR; ++e) row[e] = nxt[e];
            }
        }
#pragma unroll
        for (int dr = 0; dr < P; ++dr) wtc_lds_store4<T, P>(ctx, dst + dr * op, acc[dr]);
    }
    if constexpr (TAIL) {
        for (int it = ctx.tid; it < P * p.tail; it += ctx.nth)
            wtc_whole_row_piece<T, K>(p, ctx, full + it / P, it % P);
    }
}

// Synthesis and store, one 2 x BW output block per item (column blocks
// fastest): base output plus bias (already in the base map), level 1 through
// the 2x2 butterfly, the deeper levels through the closed form with the
// coordinate bits picking the signs, added to the low-pass input of the
// butterfly; one rounding, one store.
// DEEP = 1: a tiled plan adds the deeper levels' term from the LDS map at
// p.deep_off instead of the global `low`; DEEP = 2: an untiled plan writes its
// result to that LDS map (the deeper levels of a larger plane) instead of
// storing it.
template <typename T, int K, int BW, bool TL, bool ST = false, int DEEP = 0, int LV = 0>
WTC_HD WTC_INLINE void wtc_whole_out(const WtcWholeArgs<T> &a, WtcWholeCtx<T> &ctx)
{
    constexpr int Q = BW / 2;
    const WtcWholePlan &p = a.p;
    const int nbx = p.w / BW, nblk = (p.h / 2) * nbx;
    const WtcMap z0 = p.z[0], z1 = p.z[1];
    const int st1 = z1.rows * z1.pitch;
    for (int it = ctx.tid; it < nblk; it += ctx.nth) {
        // the first block's coordinates were computed once per workgroup
        const int by = it == ctx.tid ? ctx.oblk >> 16 : it / nbx;
        const int bx = it == ctx.tid ? ctx.oblk & 0xffff : it - by * nbx;
        const int i1 = by;
        // the base output (without the base path the map is never written
        // and reads as the zeros LDS was cleared to, so no branch here)
        float acc[2][BW];
        if (DEEP == 2) {
            // the deeper levels of a larger plane have no base path
#pragma unroll
            for (int e = 0; e < BW; ++e) acc[0][e] = acc[1][e] = 0.0f;
        } else {
            const int oz0 = z0.off + wtc_mul24(2 * by, z0.pitch) + BW * bx;
            wtc_lds_vec<T, BW>(ctx, oz0, acc[0]);
            wtc_lds_vec<T, BW>(ctx, oz0 + z0.pitch, acc[1]);
        }
        float band[4][Q];
        const int lv = LV ? LV : p.levels;  // LV: the plan's levels, known at compile time (0: not)
        if (lv >= 1) {
            const int o1 = z1.off + wtc_mul24(i1, z1.pitch) + Q * bx;
#pragma unroll
            for (int b = 0; b < 4; ++b) wtc_lds_vec<T, Q>(ctx, o1 + b * st1, band[b]);
        } else {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int q = 0; q < Q; ++q) band[b][q] = 0.0f;
        }
        // deep levels, closed form: level m adds, to the low-pass value of
        // level-1 cell (i1, j1), the four band outputs of level-m cell
        // (i1 >> (m-1), j1 >> (m-1)) with signs from bit m-2 of i1 (sp) and of
        // j1 (sq).  The block's Q level-1 cells (Q <= 4, starting at a
        // multiple of Q) span Q/2 cells of level 2 and one cell of every
        // deeper level, and each is read once.
        static_assert(Q <= 4, "one cell of level 3 and deeper per block");
        if (!TL && lv >= 2) {
            constexpr int C2 = Q >= 2 ? Q / 2 : 1;
            const WtcMap z2 = p.z[2];
            const int sz = z2.rows * z2.pitch;
            const float sp = (i1 & 1) ? -1.0f : 1.0f;
            const int oz = z2.off + wtc_mul24(i1 >> 1, z2.pitch) + (Q * bx) / 2;
            float zc[4][C2];
#pragma unroll
            for (int b = 0; b < 4; ++b) wtc_lds_vec<T, C2>(ctx, oz + b * sz, zc[b]);
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int c = Q >= 2 ? q / 2 : 0;
                const float sq = Q >= 2 ? ((q & 1) ? -1.0f : 1.0f) : ((bx & 1) ? -1.0f : 1.0f);
                const float t0 = wtc_fma(sp, zc[1][c], zc[0][c]), t1 = wtc_fma(sp, zc[3][c], zc[2][c]);
                band[0][q] += wtc_fma(sq, t1, t0);
            }
        }
        for (int m = 3; !TL && m <= lv; ++m) {
            const WtcMap zm = p.z[m];
            const int sz = zm.rows * zm.pitch;
            const float sp = ((i1 >> (m - 2)) & 1) ? -1.0f : 1.0f;
            const int oz = zm.off + wtc_mul24(i1 >> (m - 1), zm.pitch) + ((Q * bx) >> (m - 1));
            const float t0 = wtc_fma(sp, WTC_LDS(ctx, oz + sz), WTC_LDS(ctx, oz));
            const float t1 = wtc_fma(sp, WTC_LDS(ctx, oz + 3 * sz), WTC_LDS(ctx, oz + 2 * sz));
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const float sq = (((Q * bx + q) >> (m - 2)) & 1) ? -1.0f : 1.0f;
                band[0][q] += wtc_fma(sq, t1, t0);
            }
        }
        if constexpr (DEEP == 1) {
            // the deeper levels' term (orthonormal, at level-1 resolution of
            // the image), half of it in these unnormalised sums
            float v[Q];
            wtc_lds_vec<T, Q>(ctx, p.deep_off + wtc_mul24(ctx.ty0 / 2 + i1, p.deep_pitch) + ctx.tx0 / 2 + Q * bx, v);
#pragma unroll
            for (int q = 0; q < Q; ++q) band[0][q] = wtc_fma(0.5f, v[q], band[0][q]);
        }
        if (TL && DEEP == 0 && a.low) {
            // the deeper levels' low-pass term (orthonormal) enters level 1's
            // synthesis as half its value in these unnormalised sums
            const int64_t lo = ctx.plane * ((int64_t)(p.ih / 2) * (p.iw / 2)) +
                               (int64_t)(ctx.ty0 / 2 + i1) * (p.iw / 2) + ctx.tx0 / 2 + Q * bx;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
#ifdef WTC_EMULATE
                const float v = wtc_chk(a.low, lo + q, (int64_t)p.n * p.c * (p.ih / 2) * (p.iw / 2), __LINE__);
#else
                const float v = a.low[lo + q];
#endif
                band[0][q] = wtc_fma(0.5f, v, band[0][q]);
            }
        }
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const float a0 = band[0][q], a1 = band[1][q], a2 = band[2][q], a3 = band[3][q];
            const float s01 = a0 + a1, d01 = a0 - a1, s23 = a2 + a3, d23 = a2 - a3;
            acc[0][2 * q] += s01 + s23;
            acc[0][2 * q + 1] += s01 - s23;
            acc[1][2 * q] += d01 + d23;
            acc[1][2 * q + 1] += d01 - d23;
        }
        if constexpr (DEEP == 2) {
            const int od = p.deep_off + wtc_mul24(2 * by, p.deep_pitch) + BW * bx;
            wtc_lds_put<BW, wtc_align_of(BW, 0)>(ctx, od, acc[0]);
            wtc_lds_put<BW, wtc_align_of(BW, 0)>(ctx, od + p.deep_pitch, acc[1]);
            continue;
        }
        int64_t o0 = TL ? (int64_t)(ctx.ty0 + 2 * by) * p.iw + ctx.tx0 + BW * bx
                        : (int64_t)wtc_mul24(2 * by, p.w) + BW * bx;
        if constexpr (ST) {
            // the block's image in the stack and its row there; blocks in the
            // zero rows between images (or past the batch) store nothing
            const int per = p.sh + p.sgap, sub = (2 * by) / per, rr = 2 * by - sub * per;
            const int im = (ctx.n0 + ctx.cur) * p.stack + sub;
            if (rr >= p.sh || im >= p.n) continue;
            o0 = (((int64_t)im * p.c + ctx.c) * p.sh + rr) * p.iw + BW * bx;
        }
#ifdef WTC_EMULATE
        for (int dr = 0; dr < 2; ++dr)
            for (int e = 0; e < BW; ++e) WTC_WOUT(ctx, o0 + dr * p.iw + e) = wtc_from_float<T>(acc[dr][e]);
#else
        WtcCtx<T> oc;
        oc.out = ctx.out;
        wtc_store_row<T, BW>(oc, o0, acc[0]);
        wtc_store_row<T, BW>(oc, o0 + p.iw, acc[1]);
#endif
    }
}

#endif  // WTCONV_WHOLE_BODY_H
