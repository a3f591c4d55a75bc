// wtconv_plan.h -- launch geometry and LDS layout of the fused WTConv kernels.
//
// One workgroup owns one output tile of one (n, c) plane (the whole plane when
// it fits).  Inside the tile it keeps, in LDS:
//   * the low-pass maps U_m of levels m = 1..L over the tile plus the halo the
//     deeper levels need (r * 2^(L-m) pixels of level m), computed from the
//     input directly ("coarse" part);
//   * for the deep levels m >= 2: the three detail bands over the tile plus r,
//     and the four convolution outputs over the tile;
//   * for one row strip of the tile at a time ("fine" part): the staged input
//     with a 2r halo, the three level-1 detail bands of the strip plus r, and
//     the four level-1 convolution outputs of the strip;
//   * the folded weights of the channel.
// Everything here is plain integer arithmetic shared by the host (which picks
// the sizes) and the kernels (which read them).
#ifndef WTCONV_PLAN_H
#define WTCONV_PLAN_H

#include <stdint.h>

// The helpers below run on the host (planning) and in the kernels.
#if defined(__HIP__) && !defined(WTC_EMULATE)
#include <hip/hip_runtime.h>
#define WTC_PLAN_HD __host__ __device__
#else
#define WTC_PLAN_HD
#endif

#define WTC_MAXL 6
#define WTC_PR 2  // rows of a per-level convolution piece
#define WTC_PC 4  // columns of a per-level convolution piece

struct WtcMap {
    int32_t off;    // first float of the map in LDS
    int32_t pitch;  // floats between rows
    int32_t rows;   // allocated rows (maps of one group are rows * pitch apart)
};

struct WtcFusedPlan {
    int32_t n, c, h, w, k, levels;
    int32_t tile_h, tile_w, tiles_y, tiles_x;
    int32_t strip_h;   // output rows per strip, even, divides tile_h
    int32_t out_bw;    // output block width: 2, 4 or 8, divides tile_w
    int32_t nthreads;  // workgroup size
    int32_t rotate;    // 1: kernels turned by 180 degrees and no bias (data backward)
    WtcMap ll[WTC_MAXL + 1];    // U_m, m = 1..L
    WtcMap band[WTC_MAXL + 1];  // 3 detail bands of level m = 2..L
    WtcMap z[WTC_MAXL + 1];     // 4 conv outputs of level m = 2..L
    WtcMap xs;                  // staged input strip
    WtcMap b1s;                 // 3 level-1 detail bands of the strip
    WtcMap z1s;                 // 4 level-1 conv outputs of the strip
    int32_t wf_off;             // folded weights: (1 + 4L) k*k floats
    int32_t lds_floats;
};

WTC_PLAN_HD static inline int32_t wtc_roundup(int32_t a, int32_t b) { return (a + b - 1) / b * b; }
WTC_PLAN_HD static inline int32_t wtc_min(int32_t a, int32_t b) { return a < b ? a : b; }
WTC_PLAN_HD static inline int32_t wtc_max(int32_t a, int32_t b) { return a > b ? a : b; }

// Row pitch for a map of `cols` columns: a multiple of 4 floats (16-byte rows)
// that is 4 mod 8, so that vertically adjacent rows start in different banks.
WTC_PLAN_HD static inline int32_t wtc_pitch(int32_t cols)
{
    int32_t p = wtc_roundup(cols, 4);
    if (p % 8 == 0) p += 4;
    return p;
}

// Halo of the low-pass map of level m (1 <= m <= L): level m itself needs r
// pixels for its own convolution, and level m+1 needs twice the halo of level
// m+1 in level-m pixels.
WTC_PLAN_HD static inline int32_t wtc_halo(int32_t r, int32_t levels, int32_t m) { return r << (levels - m); }

// Fills the LDS layout of plan p from its sizes.  Returns the number of floats.
static inline int32_t wtc_fused_layout(WtcFusedPlan *p)
{
    const int32_t L = p->levels, r = p->k / 2, kk = p->k * p->k;
    const int32_t TH = p->tile_h, TW = p->tile_w, TS = p->strip_h;
    int32_t off = 0;
    p->wf_off = off;
    off += wtc_roundup((1 + 4 * L) * kk, 4);
    for (int32_t m = 0; m <= WTC_MAXL; ++m) {
        p->ll[m].off = p->ll[m].pitch = p->ll[m].rows = 0;
        p->band[m] = p->ll[m];
        p->z[m] = p->ll[m];
    }
    for (int32_t m = 1; m <= L; ++m) {
        const int32_t Hm = p->h >> m, Wm = p->w >> m, THm = TH >> m, TWm = TW >> m;
        const int32_t hal = wtc_halo(r, L, m);
        // written region, clipped to one r-wide zero border around the map, plus
        // room for the ragged last convolution piece and two spare rows
        int32_t rows = wtc_max(wtc_min(THm + 2 * hal, Hm + 2 * r), hal + wtc_roundup(THm, WTC_PR) + r) + 2;
        int32_t cols = wtc_max(wtc_min(TWm + 2 * hal, Wm + 2 * r), hal + wtc_roundup(TWm, WTC_PC) + r) + 4;
        p->ll[m].off = off;
        p->ll[m].pitch = wtc_pitch(cols);
        p->ll[m].rows = rows;
        off += p->ll[m].pitch * rows;
        if (m >= 2) {
            int32_t brows = wtc_roundup(THm, WTC_PR) + 2 * r + 2;
            int32_t bcols = wtc_roundup(TWm, WTC_PC) + 2 * r + 4;
            p->band[m].off = off;
            p->band[m].pitch = wtc_pitch(bcols);
            p->band[m].rows = brows;
            off += 3 * p->band[m].pitch * brows;
            p->z[m].off = off;
            p->z[m].pitch = wtc_pitch(TWm);
            p->z[m].rows = THm;
            off += 4 * p->z[m].pitch * THm;
        }
    }
    // strip buffers
    p->xs.off = off;
    p->xs.pitch = wtc_pitch(TW + 4 * r);
    p->xs.rows = TS + 4 * r;
    off += p->xs.pitch * p->xs.rows;
    const int32_t TS1 = TS / 2, TW1 = TW / 2;
    p->b1s.off = off;
    p->b1s.pitch = wtc_pitch(wtc_roundup(TW1, WTC_PC) + 2 * r + 4);
    p->b1s.rows = wtc_roundup(TS1, WTC_PR) + 2 * r + 2;
    off += 3 * p->b1s.pitch * p->b1s.rows;
    p->z1s.off = off;
    p->z1s.pitch = wtc_pitch(TW1);
    p->z1s.rows = TS1;
    off += 4 * p->z1s.pitch * p->z1s.rows;
    p->lds_floats = off;
    return off;
}

// Largest even divisor of `total` that is below `cur` (0 if none).
static inline int32_t wtc_next_smaller_even_divisor(int32_t total, int32_t cur)
{
    for (int32_t d = cur - 1; d >= 2; --d)
        if (d % 2 == 0 && total % d == 0) return d;
    return 0;
}

// Largest multiple of g below `cur` that divides `total` (0 if none).
static inline int32_t wtc_next_smaller_tile(int32_t total, int32_t cur, int32_t g)
{
    for (int32_t d = cur - g; d >= g; d -= g)
        if (total % d == 0) return d;
    return 0;
}

// Chooses tile and strip sizes so that the layout fits in `budget_floats`.
// Preference: whole plane, then shorter strips (down to 8 rows), then smaller
// tiles.  Returns 0 on success, -1 if nothing fits.
static inline int wtc_make_fused_plan(WtcFusedPlan *p, int32_t n, int32_t c, int32_t h, int32_t w, int32_t k,
                                      int32_t levels, int32_t rotate, int32_t nthreads, int32_t budget_floats)
{
    p->n = n;
    p->c = c;
    p->h = h;
    p->w = w;
    p->k = k;
    p->levels = levels;
    p->rotate = rotate;
    p->nthreads = nthreads;
    if (levels < 1 || levels > WTC_MAXL) return -1;
    const int32_t g = 1 << levels;
    if (h % g || w % g) return -1;
    int32_t th = h, tw = w;
    for (;;) {
        int32_t ts = th;
        for (;;) {
            p->tile_h = th;
            p->tile_w = tw;
            p->strip_h = ts;
            wtc_fused_layout(p);
            if (p->lds_floats <= budget_floats) {
                p->tiles_y = h / th;
                p->tiles_x = w / tw;
                p->out_bw = (tw % 8 == 0) ? 8 : (tw % 4 == 0) ? 4 : 2;
                return 0;
            }
            int32_t nts = wtc_next_smaller_even_divisor(th, ts);
            if (nts < 8 || nts == 0) break;
            ts = nts;
        }
        // shrink the tile: the longer side goes to the next smaller multiple of
        // 2^L that divides the plane side
        int32_t ntw = wtc_next_smaller_tile(w, tw, g), nth = wtc_next_smaller_tile(h, th, g);
        if (ntw && (tw >= th || !nth)) {
            tw = ntw;
        } else if (nth) {
            th = nth;
        } else {
            return -1;
        }
    }
}

// Images per workgroup for a grid of C x ceil(N / planes) workgroups of
// which `slots` run at once: the planes that minimise rounds x (planes +
// fixed), where fixed is a workgroup's set-up and reduction cost in units of
// one image's work and rounds = ceil(workgroups / slots).  Ties go to fewer
// images per workgroup.
static inline int wtc_choose_planes(int64_t n, int64_t c, int64_t slots, double fixed)
{
    if (slots < 1) slots = 1;
    int best = 1;
    double best_cost = 0.0;
    for (int64_t p = 1; p <= n; ++p) {
        const int64_t groups = (n + p - 1) / p;
        if (p > 1 && (n + p - 2) / (p - 1) == groups) continue;  // same grid as p - 1
        const int64_t rounds = (c * groups + slots - 1) / slots;
        const double cost = (double)rounds * ((double)p + fixed);
        if (p == 1 || cost < best_cost) {
            best = (int)p;
            best_cost = cost;
        }
    }
    return best;
}

#endif  // WTCONV_PLAN_H
