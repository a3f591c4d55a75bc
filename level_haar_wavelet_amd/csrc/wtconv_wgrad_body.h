// wtconv_wgrad_body.h -- fused parameter gradients of the WTConv layer for
// planes that fit in LDS whole, written as phases separated by workgroup
// barriers (the kernel in wtconv_wgrad.hip and a CPU emulation run the same
// code).
//
// Source: "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
// Reformulation" (arXiv 2608.10805), technical summary: Key Contributions
// (all parameter gradients of the layer) and Methodology, reformulations 1 and
// 3 (Haar analysis recomputed on chip; scales folded into the weights, so the
// chain rule brings the scale back into the weight and scale gradients).
//
// With U_m / B_m^b the plain (unnormalised) Haar sums of the forward pass, the
// orthonormal subbands are A = 2^-m B(x) and the gradient at a level's band
// outputs is dZ = 2^-m B(dy) (the synthesis is the transposed analysis), so
//   G_m^b[u][v] = sum_{n,i,j} dZ[i][j] A[i+u-r][j+v-r]
//               = 4^-m sum B(dy)[i][j] B(x)[i+u-r][j+v-r],
//   G_0[u][v]   = sum dy[h][w] x[h+u-r][w+v-r],   G_b = sum dy,
// and then (in the second kernel)
//   dW_m^b = s_m^b G_m^b,  ds_m^b = <W_m^b, G_m^b>,
//   dW_0 = s_0 G_0,  db_0 = s_0 G_b,  ds_0 = <W_0, G_0> + b_0 G_b.
//
// One workgroup owns one channel and P images.  The correlation work is cut
// into 4x4 pieces of the dy-side maps ("A" maps: dy itself, then the four
// bands of every level); thread t owns pieces t, t + nth, t + 2 nth, ... for
// the whole life of the workgroup and keeps one k x k (+1) accumulator set per
// piece, so the cross-thread reduction happens once per workgroup, in a fixed
// order.  Consecutive lanes take horizontally adjacent pieces and every map
// row starts on a 16-byte boundary, so the 16-byte LDS reads of a wave cover
// consecutive banks.
#ifndef WTCONV_WGRAD_BODY_H
#define WTCONV_WGRAD_BODY_H

#include "wtconv_whole_body.h"

#define WTC_WG_QMAX 3  // pieces per thread
#define WTC_WG_P 4     // piece side
#define WTC_WG_CH 16   // threads summed by one job of the reduction's first stage
#define WTC_WG_MAXT 512  // threads per workgroup, at most
#define WTC_WG_NMAPS (1 + 4 * WTC_MAXL)
#define WTC_WG_CHMAX (WTC_WG_MAXT / WTC_WG_CH + WTC_WG_NMAPS)  // first-stage jobs of a set, at most

struct WtcWgradPlan {
    int32_t n, c, h, w, k, levels;
    int32_t nthreads;
    int32_t planes;     // images per workgroup
    int32_t groups;     // workgroups per channel
    int32_t q;          // pieces per thread
    int32_t npieces;
    int32_t tail;       // the last `tail` pieces run as one-row pieces (see wtc_wgrad_layout)
    int32_t nmaps;      // 1 + 4L
    int32_t plen;       // floats of one partial result: k*k + 1 + 4L k*k
    int32_t vec;        // activation elements per staged row segment (at most 16 bytes)
    int32_t gr;         // rows per staging group (4, 2 or 1)
    int32_t sgroups;    // staging groups of a plane, (h / gr) (w / vec) <= nthreads
    int32_t first_deep; // first level computed from LDS (the staging computes the ones before)
    WtcMap x;           // x with an r-wide zero border (origin (r, r))
    WtcMap dy;          // dy (origin (0, 0)), zero beyond the image
    WtcMap u[WTC_MAXL + 1];  // B_m(x): 4 bands with an r border
    WtcMap d[WTC_MAXL + 1];  // B_m(dy): 4 bands, origin (0, 0)
    int32_t first[1 + 4 * WTC_MAXL + 1];  // first piece of every map, then the total
    int32_t tab_off;    // piece descriptors, 2 ints each
    int32_t res_off;    // per-map results, nmaps x (k*k + 1)
    int32_t red_off;    // parked accumulators, nthreads x n1p (aliases the maps)
    int32_t csum_off;   // first-stage sums of the reduction (aliases the maps)
    int32_t ctab_off;   // reduction tables in LDS: per set, chunk[] then mapc[]
    int32_t lds_floats;
    // Reduction tables (host-built): per set s, the threads of first-stage job
    // c (t0 | t1 << 16) and, per map, its first job and job count (c0 | n << 16).
    int32_t nchunks[WTC_WG_QMAX];
    int32_t chunk[WTC_WG_QMAX][WTC_WG_CHMAX];
    int32_t mapc[WTC_WG_QMAX][WTC_WG_NMAPS];
    // Tiling, for planes too large for one workgroup: h x w above is one tile
    // of an ih x iw image and a unit of work is one (image, tile); the x side
    // is loaded with lh pixels around the tile (zero outside the image) and
    // stored from origins that keep the correlation windows on 16-byte
    // boundaries; the dy side is the tile only; L is 1 (the deeper levels are
    // a separate call on the level-1 low-pass maps).  Untiled: ih = h, iw = w,
    // one tile, lh = 0, origins (r, r).
    int32_t tiled, ih, iw, tiles_x, tiles_y, units;
    int32_t lh, xr, xc, u1r, u1c;
    // the base gradients are not wanted (the deeper levels of a larger
    // layer): the base map has no pieces and its partial-row entries are 0
    int32_t nobase;
};

// stride of one thread's parked accumulators: k*k + 1 rounded up to odd
WTC_PLAN_HD static inline int32_t wtc_wgrad_n1p(int32_t k) { return (k * k + 1) | 1; }

static inline int32_t wtc_wgrad_layout(WtcWgradPlan *p)
{
    const int32_t L = p->levels, r = p->k / 2, kk = p->k * p->k, P = WTC_WG_P;
    // Every row starts on a 16-byte boundary.  A piece's x-side window row is
    // read as roundup(P + k - 1, 4) floats from column 4 pc, which stays inside
    // the row: the pitch is roundup(roundup(W, 4) + 2r, 4).
    int32_t off = 0;
    const int32_t NR = wtc_roundup(P + 2 * r, 4);  // window row, as read
    p->x.off = off;
    p->x.rows = wtc_max(p->lh + p->h + p->xr, wtc_roundup(p->h, P) - P - r + p->xr + P + 2 * r);
    p->x.pitch = wtc_roundup(wtc_max(p->lh + p->w + p->xc, wtc_roundup(p->w, P) - P - r + p->xc + NR), 4);
    p->dy.rows = wtc_roundup(p->h, P);
    p->dy.pitch = wtc_roundup(p->w, P);
    if (p->nobase) {
        // without the base correlation nothing reads the full-resolution maps:
        // one row each with a zero pitch takes the staging's stores
        off += p->x.pitch;
        p->dy.off = off;
        off += p->dy.pitch;
        p->x.rows = p->dy.rows = 1;
        p->x.pitch = p->dy.pitch = 0;
    } else {
        off += p->x.rows * p->x.pitch;
        p->dy.off = off;
        off += p->dy.rows * p->dy.pitch;
    }
    for (int32_t m = 0; m <= WTC_MAXL; ++m) {
        p->u[m].off = p->u[m].pitch = p->u[m].rows = 0;
        p->d[m] = p->u[m];
    }
    for (int32_t m = 1; m <= L; ++m) {
        const int32_t Hm = p->h >> m, Wm = p->w >> m;
        const int32_t orow = m == 1 ? p->u1r : r, ocol = m == 1 ? p->u1c : r, lm = m == 1 ? p->lh / 2 : 0;
        p->u[m].off = off;
        p->u[m].rows = wtc_max(lm + Hm + orow, wtc_roundup(Hm, P) - P - r + orow + P + 2 * r);
        p->u[m].pitch = wtc_roundup(wtc_max(lm + Wm + ocol, wtc_roundup(Wm, P) - P - r + ocol + NR), 4);
        off += 4 * p->u[m].rows * p->u[m].pitch;
        p->d[m].off = off;
        p->d[m].rows = wtc_roundup(Hm, P);
        p->d[m].pitch = wtc_roundup(Wm, P);
        off += 4 * p->d[m].rows * p->d[m].pitch;
    }
    // pieces: map 0 is the base (full resolution), map 1 + 4(m-1) + b is band b of level m
    p->nmaps = 1 + 4 * L;
    int32_t np = 0;
    for (int32_t g = 0; g < p->nmaps; ++g) {
        const int32_t m = g == 0 ? 0 : (g - 1) / 4 + 1;
        p->first[g] = np;
        if (g > 0 || !p->nobase) np += ((p->h >> m) + P - 1) / P * (((p->w >> m) + P - 1) / P);
    }
    p->first[p->nmaps] = np;
    p->npieces = np;
    p->q = (np + p->nthreads - 1) / p->nthreads;
    // One set of pieces whose last wave would hold a few: those run as P
    // one-row pieces each on the lanes after the full waves (at most two
    // waves of them, a quarter of a piece each), so that no wave runs a whole
    // piece for a few lanes (the 28 x 28 L = 2 plan: 129 pieces on 256
    // threads).  Untiled plans only; the reduction tables count threads.
    p->tail = 0;
    if (p->q == 1 && !p->tiled) {
        const int32_t full = np / 64 * 64, rest = np - full;
        if (full > 0 && rest > 0 && P * rest <= 128 && full + P * rest <= p->nthreads) p->tail = rest;
    }
    p->plen = kk + 1 + 4 * L * kk;
    off = wtc_roundup(off, 4);
    p->tab_off = off;
    off += 2 * np;
    // the reduction runs after the last image: its buffers reuse the maps and
    // the table; the per-map results come after both.  A set of pieces splits
    // into at most nthreads / CH + nmaps first-stage jobs per tap.
    p->red_off = 0;
    p->csum_off = p->nthreads * wtc_wgrad_n1p(p->k);
    const int32_t red_end = p->csum_off + (p->nthreads / WTC_WG_CH + p->nmaps) * (kk + 1);
    off = wtc_max(off, red_end);
    p->res_off = wtc_roundup(off, 4);
    off = p->res_off + p->nmaps * (kk + 1);
    p->ctab_off = off;
    off += WTC_WG_QMAX * (WTC_WG_CHMAX + WTC_WG_NMAPS);
    p->lds_floats = wtc_roundup(off, 4);
    // reduction tables: set s holds pieces s nth .. s nth + nth - 1 (thread
    // t: piece s nth + t), except that piece j >= F = npieces - tail of a
    // one-set plan runs on threads F + P (j - F) .. F + P (j - F) + P - 1
    const int32_t tf = np - p->tail;
    auto tpos = [&](int32_t j) { return j <= tf ? j : tf + P * (j - tf); };
    for (int32_t s = 0; s < WTC_WG_QMAX; ++s) {
        int32_t nc = 0;
        for (int32_t g = 0; g < WTC_WG_NMAPS; ++g) {
            int32_t lo = 0, hi = 0;
            if (g < p->nmaps) {
                lo = wtc_max(0, tpos(p->first[g]) - s * p->nthreads);
                hi = wtc_min(p->nthreads, tpos(p->first[g + 1]) - s * p->nthreads);
            }
            const int32_t cnt = hi > lo ? (hi - lo + WTC_WG_CH - 1) / WTC_WG_CH : 0;
            p->mapc[s][g] = nc | (cnt << 16);
            for (int32_t j = 0; j < cnt; ++j) {
                const int32_t t0 = lo + j * WTC_WG_CH, t1 = wtc_min(hi, t0 + WTC_WG_CH);
                p->chunk[s][nc + j] = t0 | (t1 << 16);
            }
            nc += cnt;
        }
        for (int32_t j = nc; j < WTC_WG_CHMAX; ++j) p->chunk[s][j] = 0;
        p->nchunks[s] = nc;
    }
    return p->lds_floats;
}

static inline int wtc_wgrad_plan_common(WtcWgradPlan *p, int32_t n, int32_t c, int32_t h, int32_t w, int32_t k,
                                        int32_t levels, int32_t nthreads, int32_t planes, int32_t elem_bytes,
                                        int32_t budget_floats, int32_t ih, int32_t iw, int32_t nobase)
{
    const int32_t r = k / 2;
    p->nobase = nobase && levels >= 1;
    p->n = n;
    p->c = c;
    p->h = h;
    p->w = w;
    p->k = k;
    p->levels = levels;
    p->nthreads = nthreads;
    p->tiled = ih != h || iw != w;
    p->ih = ih;
    p->iw = iw;
    if (h < 1 || w < 1 || ih % h || iw % w) return -1;
    p->tiles_y = ih / h;
    p->tiles_x = iw / w;
    p->units = n * p->tiles_y * p->tiles_x;
    p->planes = planes < 1 ? 1 : (planes > p->units ? p->units : planes);
    p->groups = (p->units + p->planes - 1) / p->planes;
    if (levels < 0 || levels > WTC_MAXL) return -1;
    if (p->tiled && levels > 1) return -1;
    if (h % (1 << levels) || w % (1 << levels)) return -1;
    if (nthreads % WTC_WG_CH || nthreads > WTC_WG_MAXT) return -1;
    // 4-element segments in both storage types (16 bytes of fp32, 8 of
    // fp16): with 8 fp16 per thread the staging's LDS writes from lanes 32
    // bytes apart conflict twice as often
    int32_t vec = 16 / elem_bytes < 4 ? 16 / elem_bytes : 4;
    while (vec > 1 && w % vec) vec /= 2;
    p->vec = vec;
    p->gr = h % 4 == 0 ? 4 : (h % 2 == 0 ? 2 : 1);
    if (levels >= 1 && (p->gr < 2 || vec < 2)) return -1;
    if (p->tiled) {
        // x loaded with 2r pixels around the tile (level 1's windows need r
        // level-1 pixels), rounded to whole staging groups and segments
        if (p->gr != 4 || vec != 4) return -1;
        p->lh = wtc_roundup(wtc_max(2 * r, 1), wtc_max(4, vec));
        p->xr = p->lh;
        p->xc = p->lh + r;
        p->u1r = p->lh / 2;
        p->u1c = p->lh / 2 + ((r - p->lh / 2) % 4 + 4) % 4;
    } else {
        p->lh = 0;
        p->xr = p->xc = p->u1r = p->u1c = r;
    }
    p->sgroups = ((h + 2 * p->lh) / p->gr) * ((w + 2 * p->lh) / vec);
    if (p->sgroups > nthreads) return -1;
    p->first_deep = (levels >= 2 && p->gr == 4 && vec >= 4) ? 3 : 2;
    wtc_wgrad_layout(p);
    if (p->q > WTC_WG_QMAX) return -1;
    // descriptor fields: pitches below 256 and LDS indexes below 65536; the
    // pitch of every map a piece reads counts, the level maps' too (without
    // the base path the full-resolution maps are one zero-pitch row and the
    // level-1 maps are the widest)
    int32_t maxp = wtc_max(p->x.pitch, p->dy.pitch);
    for (int32_t m = 1; m <= levels; ++m) maxp = wtc_max(maxp, wtc_max(p->u[m].pitch, p->d[m].pitch));
    if (maxp > 255 || p->lds_floats > 65535) return -1;
    return p->lds_floats <= budget_floats ? 0 : -1;
}

// nobase: the base gradients are not wanted (L >= 1 only).
static inline int wtc_make_wgrad_plan(WtcWgradPlan *p, int32_t n, int32_t c, int32_t h, int32_t w, int32_t k,
                                      int32_t levels, int32_t nthreads, int32_t planes, int32_t elem_bytes,
                                      int32_t budget_floats, int32_t nobase = 0)
{
    return wtc_wgrad_plan_common(p, n, c, h, w, k, levels, nthreads, planes, elem_bytes, budget_floats, h, w,
                                 nobase);
}

// Tiled plan: th x tw tiles of ih x iw images, L = 1 (base and level-1
// gradients) or L = 0.
static inline int wtc_make_wgrad_tile_plan(WtcWgradPlan *p, int32_t n, int32_t c, int32_t ih, int32_t iw,
                                           int32_t th, int32_t tw, int32_t k, int32_t levels, int32_t nthreads,
                                           int32_t planes, int32_t elem_bytes, int32_t budget_floats,
                                           int32_t nobase = 0)
{
    if (th == ih && tw == iw) return -1;
    return wtc_wgrad_plan_common(p, n, c, th, tw, k, levels, nthreads, planes, elem_bytes, budget_floats, ih, iw,
                                 nobase);
}

template <typename T>
struct WtcWgradArgs {
    const T *x;
    const T *dy;
    float *partial;  // [groups][C][plen]
    WtcWgradPlan p;
    // tiled plans: the level-1 low-pass maps of x and dy, (N, C, ih/2, iw/2)
    // orthonormal, fp32 whatever T is, written for every tile's interior (the
    // input of the deeper levels' gradients), or null
    float *llx = nullptr;
    float *lld = nullptr;
};

template <typename T, int VEC>
struct WtcWgradCtx {
    float *lds;
    int tid, nth;
    int c, n0, nimg, group;
    int grow, gcol;  // this thread's staging group
    bool gvalid;
    int vmask;       // rows of the prefetched group that lie in the image (bit q)
    int64_t llo;     // tiled: the prefetched unit's tile origin in the level-1 low-pass maps
    T prex[4][VEC];
    T prey[4][VEC];
#ifdef WTC_EMULATE
    int64_t lds_n;
#endif
};

template <typename T, int VEC>
WTC_HD WTC_INLINE void wtc_wgrad_setup(const WtcWgradArgs<T> &a, WtcWgradCtx<T, VEC> &ctx, int bid)
{
    const WtcWgradPlan &p = a.p;
    ctx.c = bid % p.c;
    ctx.group = bid / p.c;
    ctx.n0 = ctx.group * p.planes;
    ctx.nimg = wtc_min(p.planes, p.units - ctx.n0);
    const int g = wtc_min(ctx.tid, p.sgroups - 1), cpr = (p.w + 2 * p.lh) / VEC;
    ctx.grow = g / cpr;
    ctx.gcol = g - ctx.grow * cpr;
    ctx.gvalid = ctx.tid < p.sgroups;
}

template <typename T, int VEC>
WTC_HD WTC_INLINE void wtc_wgrad_zero(const WtcWgradArgs<T> &a, WtcWgradCtx<T, VEC> &ctx)
{
    const float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int i = 4 * ctx.tid; i < a.p.lds_floats; i += 4 * ctx.nth) wtc_lds_put<4, 4>(ctx, i, z);
}

// Loads of this thread's staging group (gr rows of VEC elements) of image
// `img`, x and dy, into registers; every lane loads a valid group.
// TL: tiled plan (units of (image, tile), halo loads with bounds, shifted
// origins); untiled plans compile without any of it.
template <typename T, int VEC, bool TL = false>
WTC_HD WTC_INLINE void wtc_wgrad_load(const WtcWgradArgs<T> &a, WtcWgradCtx<T, VEC> &ctx, int img)
{
    const WtcWgradPlan &p = a.p;
#ifndef WTC_EMULATE
    // everything in flight was issued a phase or more ago: one wait here keeps
    // the compiler from draining each load before the next (vmcnt 0 only)
    __builtin_amdgcn_s_waitcnt(0x0F70);
#endif
    int64_t plane, e0;
    int row0 = 0, col = 0;
    if constexpr (TL) {
        // Tiled plans load through buffer resources over the x and dy planes:
        // the hardware returns zeros for every offset past a plane, which is
        // what the rows above and below the image get (a negative offset reads
        // as a large unsigned one); segments left or right of the image, and
        // the dy side of groups in the halo (the correlation reads dy inside
        // the tile only), are sent past the plane and fetch nothing.
        const int tiles = p.tiles_x * p.tiles_y, unit = ctx.n0 + img;
        const int im = unit / tiles, t = unit - im * tiles, ty = t / p.tiles_x;
        const int tx = t - ty * p.tiles_x;
        const int64_t pl = ((int64_t)im * p.c + ctx.c) * ((int64_t)p.ih * p.iw);
        const int r0 = p.gr * ctx.grow - p.lh, c0 = VEC * ctx.gcol - p.lh;  // in the tile
        row0 = ty * p.h + r0;
        col = tx * p.w + c0;
        ctx.llo = ((int64_t)im * p.c + ctx.c) * ((int64_t)(p.ih / 2) * (p.iw / 2)) +
                  (int64_t)(ty * p.h / 2) * (p.iw / 2) + tx * p.w / 2;
        const bool colok = col >= 0 && col < p.iw;
        const bool dyin = r0 >= 0 && r0 < p.h && c0 >= 0 && c0 < p.w;
        // columns past any plane (sides <= 4096: offsets stay below 2^31);
        // two selects, so that the loads below need no branch
        const int colx = colok ? col : (1 << 27), cold = dyin ? col : (1 << 27);
        const int plane_bytes = p.ih * p.iw * (int)sizeof(T);
#ifndef WTC_EMULATE
        const __amdgpu_buffer_rsrc_t rx =
            __builtin_amdgcn_make_buffer_rsrc((void *)(a.x + pl), (short)0, plane_bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rd =
            __builtin_amdgcn_make_buffer_rsrc((void *)(a.dy + pl), (short)0, plane_bytes, 0x00020000);
#endif
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < p.gr) {
                const int row = row0 + q;
                const int ox = (row * p.iw + colx) * (int)sizeof(T), od = (row * p.iw + cold) * (int)sizeof(T);
#ifdef WTC_EMULATE
                // the hardware's rule: a load whose bytes lie past the range
                // (the offset read as unsigned) returns zeros; it must agree
                // with the segment lying in the image (and, for dy, in the tile)
                const uint64_t seg = VEC * sizeof(T);
                const bool ok = (uint64_t)(uint32_t)ox + seg <= (uint64_t)plane_bytes;
                const bool okd = (uint64_t)(uint32_t)od + seg <= (uint64_t)plane_bytes;
                if (ok != (colok && row >= 0 && row < p.ih) || okd != (ok && dyin)) {
                    fprintf(stderr, "wtconv emulation: buffer range check disagrees at row %d col %d\n", row, col);
                    abort();
                }
                const int64_t all = (int64_t)p.n * p.c * p.ih * p.iw, e = pl + (int64_t)row * p.iw + col;
                for (int t2 = 0; t2 < VEC; ++t2) {
                    ctx.prex[q][t2] = ok ? wtc_chk(a.x, e + t2, all, __LINE__) : (T)0.0f;
                    ctx.prey[q][t2] = okd ? wtc_chk(a.dy, e + t2, all, __LINE__) : (T)0.0f;
                }
#else
                static_assert(VEC * sizeof(T) == 16 || VEC * sizeof(T) == 8, "tiled plans stage 4-element segments");
                if constexpr (VEC * sizeof(T) == 16) {
                    const auto dx4 = __builtin_amdgcn_raw_buffer_load_b128(rx, (unsigned)ox, 0, 0);
                    const auto dd4 = __builtin_amdgcn_raw_buffer_load_b128(rd, (unsigned)od, 0, 0);
                    __builtin_memcpy(&ctx.prex[q][0], &dx4, 16);
                    __builtin_memcpy(&ctx.prey[q][0], &dd4, 16);
                } else {
                    const auto dx2 = __builtin_amdgcn_raw_buffer_load_b64(rx, (unsigned)ox, 0, 0);
                    const auto dd2 = __builtin_amdgcn_raw_buffer_load_b64(rd, (unsigned)od, 0, 0);
                    __builtin_memcpy(&ctx.prex[q][0], &dx2, 8);
                    __builtin_memcpy(&ctx.prey[q][0], &dd2, 8);
                }
#endif
            }
        }
        ctx.vmask = 0xF;
        return;
    }
    // untiled: whole planes, every group in the image
    plane = ((int64_t)(ctx.n0 + img) * p.c + ctx.c) * ((int64_t)p.h * p.w);
    e0 = plane + (int64_t)(p.gr * ctx.grow) * p.w + VEC * ctx.gcol;
    (void)row0;
    (void)col;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (q < p.gr) {
            const int64_t e = e0 + (int64_t)q * p.w;
#ifdef WTC_EMULATE
            const int64_t all = (int64_t)p.n * p.c * p.ih * p.iw;
            for (int t = 0; t < VEC; ++t) {
                ctx.prex[q][t] = wtc_chk(a.x, e + t, all, __LINE__);
                ctx.prey[q][t] = wtc_chk(a.dy, e + t, all, __LINE__);
            }
#else
            if constexpr (VEC * sizeof(T) == 16) {
                typedef float v4 __attribute__((ext_vector_type(4)));
                v4 d0 = __builtin_nontemporal_load((const v4 *)(a.x + e));
                v4 d1 = __builtin_nontemporal_load((const v4 *)(a.dy + e));
                __builtin_memcpy(&ctx.prex[q][0], &d0, 16);
                __builtin_memcpy(&ctx.prey[q][0], &d1, 16);
            } else if constexpr (VEC * sizeof(T) == 8) {
                typedef float v2 __attribute__((ext_vector_type(2)));
                v2 d0 = __builtin_nontemporal_load((const v2 *)(a.x + e));
                v2 d1 = __builtin_nontemporal_load((const v2 *)(a.dy + e));
                __builtin_memcpy(&ctx.prex[q][0], &d0, 8);
                __builtin_memcpy(&ctx.prey[q][0], &d1, 8);
            } else {
#pragma unroll
                for (int t = 0; t < VEC; ++t) {
                    ctx.prex[q][t] = a.x[e + t];
                    ctx.prey[q][t] = a.dy[e + t];
                }
            }
#endif
        }
    }
    ctx.vmask = 0xF;
}

// One 2x2 Haar step on four pairs of rows held in registers: out[b][j] for
// band b (LL, top-bottom, left-right, diagonal) at column j of the half rows.
template <int N>
WTC_HD WTC_INLINE void wtc_haar_rows(const float (&top)[2 * N], const float (&bot)[2 * N], float (&out)[4][N])
{
#pragma unroll
    for (int j = 0; j < N; ++j) {
        const float x00 = top[2 * j], x01 = top[2 * j + 1], x10 = bot[2 * j], x11 = bot[2 * j + 1];
        const float sa = x00 + x01, sc = x10 + x11, da = x00 - x01, dc = x10 - x11;
        out[0][j] = sa + sc;
        out[1][j] = sa - sc;
        out[2][j] = da + dc;
        out[3][j] = da - dc;
    }
}

// LDS row offsets of the staging: 24-bit multiplies in tiled plans (measured
// 5-7 % faster on the tiled weight backward), plain ones otherwise (the
// whole-plane kernel at 56 x 56 measured 1 % slower with them).
template <bool TL>
WTC_HD WTC_INLINE int wtc_wg_mul(int a, int b)
{
    if constexpr (TL)
        return wtc_mul24(a, b);
    else
        return a * b;
}

// Write the prefetched groups of x (bordered map) and dy, and compute Haar
// level 1 (and level 2 when the group has 4 rows and at least 4 columns) of
// both straight from registers.
template <typename T, int K, int VEC, bool TL = false>
WTC_HD WTC_INLINE void wtc_wgrad_stage(const WtcWgradArgs<T> &a, WtcWgradCtx<T, VEC> &ctx)
{
    constexpr int R = K / 2;
    const WtcWgradPlan &p = a.p;
    if (!ctx.gvalid) return;
    float xv[4][VEC], dv[4][VEC];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int t = 0; t < VEC; ++t) {
            const bool ok = q < p.gr;  // tiled loads return zeros outside the image
            xv[q][t] = ok ? wtc_to_float(ctx.prex[q][t]) : 0.0f;
            dv[q][t] = ok ? wtc_to_float(ctx.prey[q][t]) : 0.0f;
        }
    // (r0, c0): the group in the loaded region; tiled: (r0 - lh, c0 - lh) in
    // the tile, dy stored only for groups inside the tile
    const int lh = TL ? p.lh : 0;
    const int r0 = p.gr * ctx.grow - lh, c0 = VEC * ctx.gcol - lh;
    const bool dyin = !TL || (r0 >= 0 && r0 < p.h && c0 >= 0 && c0 < p.w);
    if constexpr (TL) {
        // x at the plan's origin; windows start 16-byte aligned, the stores
        // themselves are 4-byte
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < p.gr)
#pragma unroll
                for (int t = 0; t < VEC; ++t) WTC_LDS(ctx, p.x.off + wtc_wg_mul<TL>(r0 + q + p.xr, p.x.pitch) + c0 + t + p.xc) = xv[q][t];
        if (dyin) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q < p.gr)
                    wtc_lds_put<VEC, wtc_align_of(VEC, 0)>(ctx, p.dy.off + wtc_wg_mul<TL>(r0 + q, p.dy.pitch) + c0, dv[q]);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < p.gr) {
                wtc_lds_put<VEC, wtc_align_of(VEC, R)>(ctx, p.x.off + wtc_wg_mul<TL>(r0 + q + R, p.x.pitch) + c0 + R, xv[q]);
                wtc_lds_put<VEC, wtc_align_of(VEC, 0)>(ctx, p.dy.off + wtc_wg_mul<TL>(r0 + q, p.dy.pitch) + c0, dv[q]);
            }
        }
    }
    if constexpr (VEC >= 2) {
        if (p.levels < 1) return;
        constexpr int H1 = VEC / 2;
        const WtcMap u1 = p.u[1], d1 = p.d[1];
        const int su = u1.rows * u1.pitch, sd = d1.rows * d1.pitch;
        float llx[2][H1], lld[2][H1];
#pragma unroll
        for (int aa = 0; aa < 2; ++aa) {
            if (2 * aa < p.gr) {
                const int i = r0 / 2 + aa;
                float bx[4][H1], bd[4][H1];
                wtc_haar_rows<H1>(xv[2 * aa], xv[2 * aa + 1], bx);
                wtc_haar_rows<H1>(dv[2 * aa], dv[2 * aa + 1], bd);
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    // x side at the level-1 origin (u1r, u1c): (r, r) untiled,
                    // u1c = r (mod 4) tiled, so the alignment class is the same
                    const int u1r = TL ? p.u1r : R, u1c = TL ? p.u1c : R;
                    wtc_lds_put<H1, wtc_align_of(H1, R)>(ctx, u1.off + b * su + wtc_wg_mul<TL>(i + u1r, u1.pitch) + c0 / 2 + u1c,
                                                         bx[b]);
                    if (dyin)
                        wtc_lds_put<H1, wtc_align_of(H1, 0)>(ctx, d1.off + b * sd + wtc_wg_mul<TL>(i, d1.pitch) + c0 / 2,
                                                             bd[b]);
                }
#pragma unroll
                for (int j = 0; j < H1; ++j) {
                    llx[aa][j] = bx[0][j];
                    lld[aa][j] = bd[0][j];
                }
                if constexpr (TL) {
                    // the tile interior's level-1 low-pass values, (a + b + c + d) / 2
                    if (dyin && a.llx) {
                        const int64_t o = ctx.llo + (int64_t)i * (p.iw / 2) + c0 / 2;
#ifdef WTC_EMULATE
                        const int64_t all = (int64_t)p.n * p.c * (p.ih / 2) * (p.iw / 2);
                        for (int j = 0; j < H1; ++j) {
                            wtc_chk(a.llx, o + j, all, __LINE__) = 0.5f * bx[0][j];
                            wtc_chk(a.lld, o + j, all, __LINE__) = 0.5f * bd[0][j];
                        }
#else
#pragma unroll
                        for (int j = 0; j < H1; ++j) {
                            a.llx[o + j] = 0.5f * bx[0][j];
                            a.lld[o + j] = 0.5f * bd[0][j];
                        }
#endif
                    }
                }
            }
        }
        if constexpr (VEC >= 4 && !TL) {  // tiled plans carry levels 0 and 1 only
            if (p.first_deep != 3) return;
            constexpr int H2 = VEC / 4;
            const WtcMap u2 = p.u[2], d2 = p.d[2];
            const int su2 = u2.rows * u2.pitch, sd2 = d2.rows * d2.pitch;
            float bx[4][H2], bd[4][H2];
            wtc_haar_rows<H2>(llx[0], llx[1], bx);
            wtc_haar_rows<H2>(lld[0], lld[1], bd);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                wtc_lds_put<H2, wtc_align_of(H2, R)>(ctx, u2.off + b * su2 + wtc_wg_mul<TL>(ctx.grow + R, u2.pitch) + c0 / 4 + R,
                                                     bx[b]);
                wtc_lds_put<H2, wtc_align_of(H2, 0)>(ctx, d2.off + b * sd2 + wtc_wg_mul<TL>(ctx.grow, d2.pitch) + c0 / 4, bd[b]);
            }
        }
    }
}

// Haar level m (m >= first_deep) of both pyramids from level m - 1 in LDS:
// x side into the bordered maps, dy side into the interior maps.
template <typename T, int K, int VEC>
WTC_HD WTC_INLINE void wtc_wgrad_analysis(const WtcWgradArgs<T> &a, WtcWgradCtx<T, VEC> &ctx, int m)
{
    constexpr int R = K / 2;
    const WtcWgradPlan &p = a.p;
    const int Hm = p.h >> m, Wm = p.w >> m;
    const WtcMap ux = p.u[m], ud = p.d[m];
    const int sx = p.u[m - 1].off + R * p.u[m - 1].pitch + R, sxp = p.u[m - 1].pitch;
    const int sd = p.d[m - 1].off, sdp = p.d[m - 1].pitch;
    const int stx = ux.rows * ux.pitch, std_ = ud.rows * ud.pitch;
    const int total = Hm * Wm;
    for (int idx = ctx.tid; idx < total; idx += ctx.nth) {
        const int i = idx / Wm, j = idx - i * Wm;
        const int s0 = sx + (2 * i) * sxp + 2 * j, s1 = sd + (2 * i) * sdp + 2 * j;
        const float x00 = WTC_LDS(ctx, s0), x01 = WTC_LDS(ctx, s0 + 1);
        const float x10 = WTC_LDS(ctx, s0 + sxp), x11 = WTC_LDS(ctx, s0 + sxp + 1);
        const float y00 = WTC_LDS(ctx, s1), y01 = WTC_LDS(ctx, s1 + 1);
        const float y10 = WTC_LDS(ctx, s1 + sdp), y11 = WTC_LDS(ctx, s1 + sdp + 1);
        {
            const float sa = x00 + x01, sc = x10 + x11, da = x00 - x01, dc = x10 - x11;
            const int o = ux.off + (i + R) * ux.pitch + j + R;
            WTC_LDS(ctx, o) = sa + sc;
            WTC_LDS(ctx, o + stx) = sa - sc;
            WTC_LDS(ctx, o + 2 * stx) = da + dc;
            WTC_LDS(ctx, o + 3 * stx) = da - dc;
        }
        {
            const float sa = y00 + y01, sc = y10 + y11, da = y00 - y01, dc = y10 - y11;
            const int o = ud.off + i * ud.pitch + j;
            WTC_LDS(ctx, o) = sa + sc;
            WTC_LDS(ctx, o + std_) = sa - sc;
            WTC_LDS(ctx, o + 2 * std_) = da + dc;
            WTC_LDS(ctx, o + 3 * std_) = da - dc;
        }
    }
}

// Piece descriptors, two ints: (LDS index of the x-side window at row i0 - r,
// column j0 - r) | (LDS index of the dy-side piece) << 16, and x-side pitch |
// dy-side pitch << 8 | map index << 16.
template <typename T, int K, int VEC>
WTC_HD WTC_INLINE void wtc_wgrad_table(const WtcWgradArgs<T> &a, WtcWgradCtx<T, VEC> &ctx)
{
    constexpr int P = WTC_WG_P;
    const WtcWgradPlan &p = a.p;
    for (int it = ctx.tid; it < p.npieces; it += ctx.nth) {
        int g = 0;
        while (g + 1 < p.nmaps && it >= p.first[g + 1]) ++g;
        const int m = g == 0 ? 0 : (g - 1) / 4 + 1, b = g == 0 ? 0 : (g - 1) % 4;
        const int Wm = p.w >> m, npc = (Wm + P - 1) / P;
        const int rem = it - p.first[g];
        const int pr = rem / npc, pc = rem - pr * npc;
        int d0, d1, d2;
        if (m == 0) {
            // x map origin (xr, xc): element (i0 - r, j0 - r) sits at (i0 - r + xr, j0 - r + xc)
            d0 = p.x.off + (P * pr - K / 2 + p.xr) * p.x.pitch + P * pc - K / 2 + p.xc;
            d1 = p.dy.off + (P * pr) * p.dy.pitch + P * pc;
            d2 = p.x.pitch | (p.dy.pitch << 16);
        } else {
            const WtcMap ux = p.u[m], ud = p.d[m];
            const int orow = m == 1 ? p.u1r : K / 2, ocol = m == 1 ? p.u1c : K / 2;
            d0 = ux.off + b * ux.rows * ux.pitch + (P * pr - K / 2 + orow) * ux.pitch + P * pc - K / 2 + ocol;
            d1 = ud.off + b * ud.rows * ud.pitch + (P * pr) * ud.pitch + P * pc;
            d2 = ux.pitch | (ud.pitch << 16);
        }
        int *tab = (int *)&WTC_LDS(ctx, p.tab_off + 2 * it + 1) - 1;
        tab[0] = (int)((unsigned)d0 | ((unsigned)d1 << 16));
        tab[1] = (d2 & 0xff) | (((d2 >> 16) & 0xff) << 8) | (g << 16);
    }
    constexpr int per = WTC_WG_CHMAX + WTC_WG_NMAPS;
    for (int i = ctx.tid; i < WTC_WG_QMAX * per; i += ctx.nth) {
        const int s = i / per, j = i - s * per;
        const int v = j < WTC_WG_CHMAX ? p.chunk[s][j] : p.mapc[s][j - WTC_WG_CHMAX];
        *(int *)&WTC_LDS(ctx, p.ctab_off + i) = v;
    }
}

// Correlation of one 4x4 dy-side piece with its x-side window, added to acc
// (k*k taps, then, for a piece of the base map, the sum of the dy-side values:
// the bias gradient's; the level maps' partial rows have no such entry, so
// their pieces skip it).
template <typename T, int K, int VEC>
WTC_HD WTC_INLINE void wtc_wgrad_piece(WtcWgradCtx<T, VEC> &ctx, int d0, int d1, int xp, int dp, bool base,
                                      float (&acc)[K * K + 1])
{
    constexpr int P = WTC_WG_P;
    constexpr int NR = (P + K - 1 + 3) / 4 * 4;  // window row, as read (16-byte reads)
    float av[P][P];
#pragma unroll
    for (int r = 0; r < P; ++r) wtc_lds_row<T, P>(ctx, d1 + r * dp, av[r]);
    if (base) {
#pragma unroll
        for (int r = 0; r < P; ++r)
#pragma unroll
            for (int c = 0; c < P; ++c) acc[K * K] += av[r][c];
    }
    float row[NR];
    wtc_lds_row<T, NR>(ctx, d0, row);
#pragma unroll
    for (int t = 0; t < P + K - 1; ++t) {
        float nxt[NR];
        if (t + 1 < P + K - 1) wtc_lds_row<T, NR>(ctx, d0 + (t + 1) * xp, nxt);
#pragma unroll
        for (int r = 0; r < P; ++r) {
            const int u = t - r;
            if (u < 0 || u >= K) continue;
#pragma unroll
            for (int v = 0; v < K; ++v)
#pragma unroll
                for (int c = 0; c < P; ++c) acc[u * K + v] = wtc_fma(av[r][c], row[c + v], acc[u * K + v]);
        }
        if (t + 1 < P + K - 1) {
#pragma unroll
            for (int e = 0; e < NR; ++e) row[e] = nxt[e];
        }
    }
}

// One dy row of a piece (row r0) against its k rows of the x window.
template <typename T, int K, int VEC>
WTC_HD WTC_INLINE void wtc_wgrad_row_piece(WtcWgradCtx<T, VEC> &ctx, int d0, int d1, int xp, int dp, bool base,
                                          int r0, float (&acc)[K * K + 1])
{
    constexpr int P = WTC_WG_P;
    constexpr int NR = (P + K - 1 + 3) / 4 * 4;  // window row, as read (16-byte reads)
    float av[P];
    wtc_lds_row<T, P>(ctx, d1 + r0 * dp, av);
    if (base) {
#pragma unroll
        for (int c = 0; c < P; ++c) acc[K * K] += av[c];
    }
#pragma unroll
    for (int u = 0; u < K; ++u) {
        float row[NR];
        wtc_lds_row<T, NR>(ctx, d0 + (r0 + u) * xp, row);
#pragma unroll
        for (int v = 0; v < K; ++v)
#pragma unroll
            for (int c = 0; c < P; ++c) acc[u * K + v] = wtc_fma(av[c], row[c + v], acc[u * K + v]);
    }
}

// Piece descriptor `it`: x window, dy start, their pitches and the base flag.
template <typename T, int VEC>
WTC_HD WTC_INLINE void wtc_wgrad_desc(const WtcWgradPlan &p, WtcWgradCtx<T, VEC> &ctx, int it, unsigned &t0,
                                     unsigned &t1)
{
    const int *tab = (const int *)&WTC_LDS(ctx, p.tab_off + 2 * it + 1) - 1;
#ifdef WTC_EMULATE
    t0 = (unsigned)tab[0];
    t1 = (unsigned)tab[1];
#else
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    const u2 tv = *(const u2 *)tab;
    t0 = tv.x;
    t1 = tv.y;
#endif
}

// Q: accumulator sets the kernel holds (at least the plan's q).  TAIL =
// false: an instance whose plans have no tail (tiles, several sets),
// compiled without the one-row pieces.
template <typename T, int K, int VEC, int Q, bool TAIL = true>
WTC_HD WTC_INLINE void wtc_wgrad_correlate(const WtcWgradArgs<T> &a, WtcWgradCtx<T, VEC> &ctx,
                                          float (&acc)[Q][K * K + 1])
{
    const WtcWgradPlan &p = a.p;
    const int full = p.npieces - (TAIL ? p.tail : 0);
#pragma unroll
    for (int s = 0; s < Q; ++s) {
        const int it = s * ctx.nth + ctx.tid;
        if (s < p.q && it < full) {
            unsigned t0, t1;
            wtc_wgrad_desc<T, VEC>(p, ctx, it, t0, t1);
            wtc_wgrad_piece<T, K, VEC>(ctx, (int)(t0 & 0xffffu), (int)(t0 >> 16), (int)(t1 & 0xffu),
                                      (int)((t1 >> 8) & 0xffu), (t1 >> 16) == 0, acc[s]);
        }
    }
    if constexpr (TAIL) {
        // the tail's one-row pieces, on the threads after the full pieces
        // (tails exist only in one-set plans)
        const int j = ctx.tid - full;
        if (j >= 0 && j < WTC_WG_P * p.tail) {
            unsigned t0, t1;
            wtc_wgrad_desc<T, VEC>(p, ctx, full + j / WTC_WG_P, t0, t1);
            wtc_wgrad_row_piece<T, K, VEC>(ctx, (int)(t0 & 0xffffu), (int)(t0 >> 16), (int)(t1 & 0xffu),
                                          (int)((t1 >> 8) & 0xffu), (t1 >> 16) == 0, j % WTC_WG_P, acc[0]);
        }
    }
}

// After the last image, per set s of pieces (piece s nth + t on thread t):
// every thread parks its accumulators in LDS (park); first-stage jobs sum the
// parked values of up to CH consecutive threads of one map, in thread order
// (chunks); then every (map, tap) adds its chunk sums, in chunk order, to the
// per-map result (combine).  The order of every addition is fixed.
template <typename T, int K, int VEC>
WTC_HD WTC_INLINE void wtc_wgrad_park(const WtcWgradArgs<T> &a, WtcWgradCtx<T, VEC> &ctx,
                                     const float (&acc)[K * K + 1])
{
    constexpr int n1 = K * K + 1, n1p = n1 | 1;
    const WtcWgradPlan &p = a.p;
#pragma unroll
    for (int e = 0; e < n1; ++e) WTC_LDS(ctx, p.red_off + ctx.tid * n1p + e) = acc[e];
}

template <typename T, int K, int VEC>
WTC_HD WTC_INLINE void wtc_wgrad_chunks(const WtcWgradArgs<T> &a, WtcWgradCtx<T, VEC> &ctx, int s)
{
    constexpr int n1 = K * K + 1, n1p = n1 | 1, CH = WTC_WG_CH;
    const WtcWgradPlan &p = a.p;
    const int tab = p.ctab_off + s * (WTC_WG_CHMAX + WTC_WG_NMAPS);
    for (int j = ctx.tid; j < p.nchunks[s] * n1; j += ctx.nth) {
        const int c = j / n1, e = j - c * n1;
        const int word = *(const int *)&WTC_LDS(ctx, tab + c);
        const int t0 = word & 0xffff, t1 = word >> 16;
        float sum = 0.0f;
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int t = t0 + u;
            const float v = WTC_LDS(ctx, p.red_off + wtc_min(t, t1 - 1) * n1p + e);
            sum += t < t1 ? v : 0.0f;
        }
        WTC_LDS(ctx, p.csum_off + j) = sum;
    }
}

template <typename T, int K, int VEC>
WTC_HD WTC_INLINE void wtc_wgrad_combine(const WtcWgradArgs<T> &a, WtcWgradCtx<T, VEC> &ctx, int s)
{
    constexpr int n1 = K * K + 1;
    const WtcWgradPlan &p = a.p;
    const int tab = p.ctab_off + s * (WTC_WG_CHMAX + WTC_WG_NMAPS) + WTC_WG_CHMAX;
    for (int idx = ctx.tid; idx < p.nmaps * n1; idx += ctx.nth) {
        const int g = idx / n1, e = idx - g * n1;
        const int word = *(const int *)&WTC_LDS(ctx, tab + g);
        const int c0 = word & 0xffff, cnt = word >> 16;
        float sum = WTC_LDS(ctx, p.res_off + idx);
        for (int c = c0; c < c0 + cnt; ++c) sum += WTC_LDS(ctx, p.csum_off + c * n1 + e);
        WTC_LDS(ctx, p.res_off + idx) = sum;
    }
}

// Write the workgroup's per-map results: partial[group][c][plen] with
// G_0 (k*k), G_b, then G of every band of every level (k*k each).
template <typename T, int K, int VEC>
WTC_HD WTC_INLINE void wtc_wgrad_write(const WtcWgradArgs<T> &a, WtcWgradCtx<T, VEC> &ctx)
{
    constexpr int kk = K * K, n1 = kk + 1;
    const WtcWgradPlan &p = a.p;
#ifndef WTC_EMULATE
    float *dst = a.partial + ((int64_t)ctx.group * p.c + ctx.c) * p.plen;
#endif
    for (int e = ctx.tid; e < p.plen; e += ctx.nth) {
        float v;
        if (e < kk) v = WTC_LDS(ctx, p.res_off + e);
        else if (e == kk) v = WTC_LDS(ctx, p.res_off + kk);
        else {
            const int g = 1 + (e - kk - 1) / kk, t = (e - kk - 1) % kk;
            v = WTC_LDS(ctx, p.res_off + g * n1 + t);
        }
#ifdef WTC_EMULATE
        wtc_chk(a.partial, ((int64_t)ctx.group * p.c + ctx.c) * p.plen + e, (int64_t)p.groups * p.c * p.plen,
                __LINE__) = v;
#else
        dst[e] = v;
#endif
    }
}

// Second pass, one 64-lane wave per (channel c, map g): lane t < k*k sums tap
// t of the workgroup partials in group order (lane k*k the sum of dy for the
// base map), writes the weight (and bias) gradient, and returns its term of
// the scale gradient, which the caller adds up with a fixed xor butterfly
// over the wave (wtc_wgrad_finalize_store takes lane 0's total).
WTC_HD WTC_INLINE float wtc_wgrad_finalize_lane(int lane, int c, int g, int C, int k, int groups, int plen,
                                               const float *partial, const float *w_base, const float *bias,
                                               const float *s_base, const float *w_lvl, const float *s_lvl,
                                               float *dw_base, float *dbias, float *dw_lvl)
{
    const int kk = k * k;
    const int off = g == 0 ? 0 : kk + 1 + (g - 1) * kk;
    const int nval = g == 0 ? kk + 1 : kk;
    float gsum = 0.0f;
    if (lane < nval) {
        // eight groups' loads in flight at once, added in group order (the
        // order of the sum stays fixed; one load at a time made every group a
        // memory round trip)
        const float *src = partial + (int64_t)c * plen + off + lane;
        const int64_t stride = (int64_t)C * plen;
        for (int q = 0; q < groups; q += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = q + u < groups ? src[(q + u) * stride] : 0.0f;
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (q + u < groups) gsum += v[u];
        }
    }
    float term = 0.0f;
    if (g == 0) {
        const float s0 = s_base[c];
        if (lane < kk) {
            dw_base[c * kk + lane] = s0 * gsum;
            term = w_base[c * kk + lane] * gsum;
        } else if (lane == kk) {
            dbias[c] = s0 * gsum;
            term = (bias ? bias[c] : 0.0f) * gsum;
        }
    } else {
        const int m = (g - 1) / 4 + 1, b = (g - 1) % 4;
        const int64_t ch = (int64_t)(m - 1) * 4 * C + 4 * c + b;
        if (lane < kk) {
            const float gt = ldexpf(gsum, -2 * m);
            dw_lvl[ch * kk + lane] = s_lvl[ch] * gt;
            term = w_lvl[ch * kk + lane] * gt;
        }
    }
    return term;
}

WTC_HD WTC_INLINE void wtc_wgrad_finalize_store(int c, int g, int C, float total, float *ds_base, float *ds_lvl)
{
    if (g == 0) {
        ds_base[c] = total;
    } else {
        const int m = (g - 1) / 4 + 1, b = (g - 1) % 4;
        ds_lvl[(int64_t)(m - 1) * 4 * C + 4 * c + b] = total;
    }
}

#ifdef WTC_EMULATE
// The wave of the second pass on the host: the same per-lane work and the
// same xor butterfly as the kernel's shuffles.
static inline void wtc_wgrad_finalize_one(int c, int g, int C, int k, int levels, int groups, int plen,
                                          const float *partial, const float *w_base, const float *bias,
                                          const float *s_base, const float *w_lvl, const float *s_lvl,
                                          float *dw_base, float *dbias, float *ds_base, float *dw_lvl,
                                          float *ds_lvl)
{
    (void)levels;
    float t[64], u[64];
    for (int lane = 0; lane < 64; ++lane)
        t[lane] = wtc_wgrad_finalize_lane(lane, c, g, C, k, groups, plen, partial, w_base, bias, s_base, w_lvl,
                                          s_lvl, dw_base, dbias, dw_lvl);
    for (int d = 32; d >= 1; d >>= 1) {
        for (int lane = 0; lane < 64; ++lane) u[lane] = t[lane] + t[lane ^ d];
        for (int lane = 0; lane < 64; ++lane) t[lane] = u[lane];
    }
    wtc_wgrad_finalize_store(c, g, C, t[0], ds_base, ds_lvl);
}
#endif

#endif  // WTCONV_WGRAD_BODY_H
