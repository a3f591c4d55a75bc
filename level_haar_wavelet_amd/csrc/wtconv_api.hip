// wtconv_api.hip -- the C ABI of libwtconv (include/wtconv.h): argument
// validation, launch planning and dispatch.  Validation happens before any HIP
// call; nothing is allocated; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/wtconv.h"
#include "wtconv_launch.h"

int wtc_dwconv_max_width(int k);
hipError_t wtc_launch_dwconv(int dtype, int k, const void *in, void *out, const float *w_base, const float *bias,
                             const float *s_base, int N, int C, int H, int W, int rotate, hipStream_t stream);

namespace {

constexpr int kFusedThreads = 256;
constexpr int kWholeThreads = 256;     // whole-plane forward / data backward: 256 or 512 threads
constexpr int kWholeWideItems = 384;  // convolution pieces per image from which 512 threads pay
constexpr int kStackItems = 192;      // at most this many pieces per image: two images per pass
constexpr int kMaxLdsFloats = 160 * 1024 / 4;

// LDS budget of one fused workgroup.  The default keeps two workgroups per
// compute unit; WTCONV_LDS_KB (16..160) overrides it for tuning.
int env_int(const char *name, int dflt, int lo, int hi)
{
    if (const char *e = std::getenv(name)) {
        int v = std::atoi(e);
        if (v >= lo && v <= hi) return v;
    }
    return dflt;
}

int lds_budget_floats() { return env_int("WTCONV_LDS_KB", 64, 16, 160) * 1024 / 4; }

// WTCONV_NO_STRIPS=1 takes the strip and level-step fallbacks away (tests: a
// call whose plan needs them is refused with WTCONV_ERR_UNSUPPORTED).
bool no_strips() { return env_int("WTCONV_NO_STRIPS", 0, 0, 1) != 0; }

// LDS budget of the whole-plane kernel: all of a compute unit's 160 KB.  Planes
// up to 80 KB still run two workgroups per compute unit (the images per
// workgroup follow the occupancy); larger ones run one rather than being
// tiled (one per CU measured about 10 % faster than tiles plus a nested call
// on the 64 x 64 planes of a 128 x 128 layer).  WTCONV_WHOLE_LDS_KB overrides.
int whole_budget_floats() { return env_int("WTCONV_WHOLE_LDS_KB", 160, 8, 160) * 1024 / 4; }

// Set-up and reduction cost of one workgroup, in units of one image's work
// (measured on the 56 x 56 and 28 x 28 planes of the stage workloads).
constexpr double kWholeFixed = 1.0;
constexpr double kWgradFixed = 1.0;

// Images per workgroup: WTCONV_PLANES overrides; otherwise as many as keep
// the rounds of resident workgroups few (wtc_choose_planes), with the
// resident count from HIP's occupancy query (two per compute unit of 256 when
// that fails).
int pick_planes(const wtconv_desc_t *d, int resident, double fixed, const char *env)
{
    int forced = env_int(env, 0, 1, 1 << 20);
    if (forced) return forced;
    if (resident < 1) resident = 2 * 256;
    return wtc_choose_planes(d->n, d->c, resident, fixed);
}

wtconv_status_t check_desc(const wtconv_desc_t *d)
{
    if (!d) return WTCONV_ERR_NULL;
    if (d->n < 1 || d->c < 1 || d->h < 1 || d->w < 1) return WTCONV_ERR_SHAPE;
    if (d->h > WTCONV_MAX_SIDE || d->w > WTCONV_MAX_SIDE) return WTCONV_ERR_SHAPE;
    if (d->levels < 0 || d->levels > WTCONV_MAX_LEVELS) return WTCONV_ERR_SHAPE;
    if (d->k != 1 && d->k != 3 && d->k != 5 && d->k != 7) return WTCONV_ERR_UNSUPPORTED;
    if (d->dtype != WTCONV_F32 && d->dtype != WTCONV_F16) return WTCONV_ERR_UNSUPPORTED;
    if (d->n * d->c > (int64_t)1 << 24) return WTCONV_ERR_SHAPE;  // grid size
    if (d->levels == 0 && d->w > wtc_dwconv_max_width(d->k)) return WTCONV_ERR_UNSUPPORTED;
    return WTCONV_OK;
}

size_t act_bytes(const wtconv_desc_t *d)
{
    return (size_t)(d->n * d->c * d->h * d->w) * (d->dtype == WTCONV_F32 ? 4 : 2);
}

// Sides that 2^L does not divide: the layer is computed on copies zero-padded
// at the bottom and right to multiples of 2^L (equal to padding every odd level
// map by one zero before its analysis and cropping that level's synthesis),
// kept in the workspace ahead of the padded layer's own workspace.
bool ragged(const wtconv_desc_t *d)
{
    const int64_t g = (int64_t)1 << d->levels;
    return d->h % g || d->w % g;
}

wtconv_desc_t padded_desc(const wtconv_desc_t *d)
{
    const int64_t g = (int64_t)1 << d->levels;
    wtconv_desc_t s = *d;
    s.h = (d->h + g - 1) / g * g;
    s.w = (d->w + g - 1) / g * g;
    return s;
}

bool overlaps(const void *a, const void *b, size_t bytes)
{
    const char *pa = (const char *)a, *pb = (const char *)b;
    return pa < pb + bytes && pb < pa + bytes;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

wtconv_status_t check_params(const wtconv_desc_t *d, const float *w_base, const float *s_base, const float *w_lvl,
                             const float *s_lvl)
{
    if (!w_base || !s_base) return WTCONV_ERR_NULL;
    if (d->levels > 0 && (!w_lvl || !s_lvl)) return WTCONV_ERR_NULL;
    return WTCONV_OK;
}

// Whole-plane plan for d (256 threads, or 512 when a plane has enough
// convolution pieces to keep them busy: more waves in flight hide the latency
// of the staging and output passes; WTCONV_WHOLE_THREADS overrides), with its
// images per workgroup; false if a plane does not fit one workgroup.
bool whole_choice(const wtconv_desc_t *d, int rotate, WtcWholePlan *wp, int nobase = 0)
{
    if (env_int("WTCONV_NO_WHOLE", 0, 0, 1)) return false;
    const int eb = d->dtype == WTCONV_F32 ? 4 : 2;
    int wth = env_int("WTCONV_WHOLE_THREADS", 0, 64, 512);
    // the thread count follows the pieces of the layer with its base path
    // (without it, the 64 x 64 nested planes of L = 3 measured 2 % slower
    // on the 256 threads their fewer pieces would pick)
    if (wtc_make_whole_plan(wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, rotate,
                            wth ? wth : kWholeThreads, 1, eb, whole_budget_floats()) &&
        (!nobase || wtc_make_whole_plan(wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, rotate,
                                        wth ? wth : kWholeThreads, 1, eb, whole_budget_floats(), nobase)))
        return false;
    // small planes (few pieces per image): two images per pass, stacked down
    // one plane with zero rows between them, so that a pass fills more of
    // the workgroup's waves and its barriers are paid once for both
    // (WTCONV_STACK=1 switches it off)
    int stack = 1;
    if (!nobase && d->levels >= 1 && wp->items <= kStackItems && env_int("WTCONV_STACK", 2, 1, 2) == 2) {
        if (wtc_make_whole_plan(wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, rotate,
                                wth ? wth : kWholeThreads, 1, eb, whole_budget_floats(), 0, 2) == 0)
            stack = 2;
        else  // back to the one-image plan the thread count is chosen from
            wtc_make_whole_plan(wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, rotate,
                                wth ? wth : kWholeThreads, 1, eb, whole_budget_floats());
    }
    if (!wth) wth = wp->items >= kWholeWideItems ? 2 * kWholeThreads : kWholeThreads;
    if (wtc_make_whole_plan(wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, rotate, wth, 1, eb,
                            whole_budget_floats(), nobase, stack))
        return false;
    wtconv_desc_t units = *d;  // the units of work: images, or stacks of two
    units.n = wp->units;
    const int planes = pick_planes(&units, wtc_whole_resident(d->dtype, wp[0]), kWholeFixed, "WTCONV_PLANES");
    wtc_make_whole_plan(wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, rotate, wth, planes, eb,
                        whole_budget_floats(), nobase, stack);
    return true;
}

// Tile shapes tried in order for planes too large for one workgroup; wide
// tiles first (fewer halo columns, whole cache lines per row): measured on the
// 128 x 128 and 256 x 256 planes, 32 x 64 tiles are fastest for the forward
// and data backward (sweep L = 1 fp32: 184 -> 172 us against 64 x 32), 16 x 128
// for the weight backward (265 -> 214 us).  WTCONV_TILE=<rows>x<cols> puts one
// shape first (tuning).
// Threads of a tiled workgroup (WTCONV_TILE_THREADS: 256 or 512).
int tile_threads() { return env_int("WTCONV_TILE_THREADS", kFusedThreads, 256, 512) >= 512 ? 512 : 256; }

struct TileShapes {
    int n;
    int s[10][2];
};

TileShapes tile_shapes(bool wgrad)
{
    static const int pass[][2] = {{32, 64}, {16, 128}, {64, 32}, {32, 32}, {16, 64}, {16, 32}, {32, 16}, {16, 16}};
    static const int corr[][2] = {{16, 128}, {32, 64}, {64, 32}, {32, 32}, {16, 64}, {16, 32}, {32, 16}, {16, 16}};
    const int(*base)[2] = wgrad ? corr : pass;
    const int nb = 8;
    TileShapes t;
    t.n = 0;
    int fr = 0, fc = 0;
    if (const char *e = std::getenv("WTCONV_TILE")) {
        if (std::sscanf(e, "%dx%d", &fr, &fc) == 2 && fr >= 8 && fc >= 8 && fr <= 256 && fc <= 256) {
            t.s[0][0] = fr;
            t.s[0][1] = fc;
            t.n = 1;
        }
    }
    for (int i = 0; i < nb; ++i) {
        if (t.n == 1 && base[i][0] == fr && base[i][1] == fc) continue;
        t.s[t.n][0] = base[i][0];
        t.s[t.n][1] = base[i][1];
        ++t.n;
    }
    return t;
}

// Tiled plan for planes too large for one workgroup: the base and level-1
// convolutions on tiles, the deeper levels from the level-1 low-pass map by a
// separate call (L = 0: the base convolution alone).  Tile shapes are tried
// in the order of tile_shapes(); false if none fits or WTCONV_NO_TILES is set.
bool tile_choice(const wtconv_desc_t *d, int rotate, WtcWholePlan *tp, int nobase = 0)
{
    if (env_int("WTCONV_NO_TILES", 0, 0, 1)) return false;
    const int eb = d->dtype == WTCONV_F32 ? 4 : 2;
    // the tiles carry the base convolution and level 1; deeper levels are the
    // nested call on the level-1 low-pass map
    const int tl = d->levels >= 1 ? 1 : 0;
    const TileShapes shapes = tile_shapes(false);
    for (int si = 0; si < shapes.n; ++si) {
        const int *sh = shapes.s[si];
        if (d->h % sh[0] || d->w % sh[1] || (sh[0] == d->h && sh[1] == d->w)) continue;
        if (wtc_make_whole_tile_plan(tp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, sh[0], sh[1], d->k, tl,
                                     rotate, tile_threads(), 1, eb, whole_budget_floats(), nobase))
            continue;
        const int resident = wtc_whole_resident(d->dtype, tp[0]);
        int planes = env_int("WTCONV_PLANES", 0, 1, 1 << 20);
        if (!planes) planes = wtc_choose_planes(tp->units, d->c, resident > 0 ? resident : 512, kWholeFixed);
        wtc_make_whole_tile_plan(tp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, sh[0], sh[1], d->k, tl, rotate,
                                 tile_threads(), planes, eb, whole_budget_floats(), nobase);
        return true;
    }
    return false;
}

// Fused large-plane plan (planes too large for one workgroup whose level-1
// low-pass map fits one, L >= 2): the deeper levels staged from x and kept on
// chip, the base and level 1 on tiles, in one kernel with no workspace; also
// without the base path (the nested deeper-levels call of a larger plane).
// Tile shapes in the order of tile_shapes(); WTCONV_NO_LARGE=1 takes it away
// (the tiles plus a nested call on a stored low-pass map).
bool large_choice(const wtconv_desc_t *d, int rotate, WtcLargePlan *lp, int nobase)
{
    if (d->levels < 2 || env_int("WTCONV_NO_LARGE", 0, 0, 1) || env_int("WTCONV_NO_TILES", 0, 0, 1))
        return false;
    const int eb = d->dtype == WTCONV_F32 ? 4 : 2;
    // 32 x 64 tiles first, as for the tiled pass (against 16 x 128 since the
    // staging specialisation: 128 x 128 fp16 forward 2-3 % faster, fp32 within
    // 1 %)
    const TileShapes shapes = tile_shapes(false);
    for (int si = 0; si < shapes.n; ++si) {
        const int *sh = shapes.s[si];
        if (wtc_make_large_plan(lp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, sh[0], sh[1], d->k, d->levels,
                                rotate, kFusedThreads, 1, eb, whole_budget_floats(), nobase))
            continue;
        const int resident = wtc_large_resident(d->dtype, *lp);
        int planes = env_int("WTCONV_PLANES", 0, 1, 1 << 20);
        if (!planes) planes = wtc_choose_planes(d->n, d->c, resident > 0 ? resident : 512, kWholeFixed);
        return wtc_make_large_plan(lp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, sh[0], sh[1], d->k, d->levels,
                                   rotate, kFusedThreads, planes, eb, whole_budget_floats(), nobase) == 0;
    }
    return false;
}

// The deeper levels (L >= 2) of a tiled pass are the layer with L - 1 levels
// on the level-1 low-pass map, with the level weights and scales from level 2
// on and a zero base scale.  That map and the nested call's output are fp32
// whatever the activation type (intermediates; the layer's outputs are rounded
// once, at their store).
wtconv_desc_t deeper_desc(const wtconv_desc_t *d)
{
    wtconv_desc_t s = *d;
    s.h = d->h / 2;
    s.w = d->w / 2;
    s.levels = d->levels - 1;
    s.dtype = WTCONV_F32;
    return s;
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Workspace of a forward / data-backward pass; nobase: the pass runs without
// the base path (the nested call for the deeper levels of a larger layer), so
// that the plans sized here are the ones fused_pass launches.
size_t pass_workspace(const wtconv_desc_t *d, int rotate, int nobase)
{
    if (ragged(d)) {
        const wtconv_desc_t pd = padded_desc(d);
        return 2 * align256(act_bytes(&pd)) + pass_workspace(&pd, rotate, nobase);
    }
    WtcWholePlan wp;
    if (whole_choice(d, rotate, &wp, nobase) || d->levels < 2 || !tile_choice(d, rotate, &wp, nobase)) return 0;
    WtcLargePlan lp;
    if (large_choice(d, rotate, &lp, nobase)) return 0;
    const wtconv_desc_t sd = deeper_desc(d);
    const size_t quarter = align256(act_bytes(&sd));
    return 2 * quarter + align256((size_t)d->c * 4) + pass_workspace(&sd, rotate, 1);
}

// zero_base (C floats of scratch, or null): the base path is zero, as in the
// nested call for the deeper levels of a larger layer (w_base, bias and
// s_base are then not read); the whole-plane and tiled kernels skip it, the
// other paths run with a zero base scale written there.
// launch = false: a dry run that takes every decision and check of the pass,
// nested and ragged calls included, and enqueues nothing; the entry points run
// it first, so that a call that fails enqueues no work at all.
wtconv_status_t fused_pass(const wtconv_desc_t *d, const void *in, const float *w_base, const float *bias,
                           const float *s_base, const float *w_lvl, const float *s_lvl, void *out, int rotate,
                           void *workspace, size_t workspace_bytes, wtconv_stream_t stream, float *zero_base,
                           bool launch)
{
    wtconv_status_t st = check_desc(d);
    if (st != WTCONV_OK) return st;
    if (!in || !out) return WTCONV_ERR_NULL;
    if ((st = check_params(d, w_base, s_base, w_lvl, s_lvl)) != WTCONV_OK) return st;
    if (!aligned16(in) || !aligned16(out)) return WTCONV_ERR_UNSUPPORTED;
    if (overlaps(in, out, act_bytes(d))) return WTCONV_ERR_ALIAS;
    const int nobase = zero_base != nullptr && d->levels >= 1;
    hipStream_t s = (hipStream_t)stream;
    if (ragged(d)) {
        // zero-padded copy in, the padded layer, crop out
        const wtconv_desc_t pd = padded_desc(d);
        if ((st = check_desc(&pd)) != WTCONV_OK) return st;
        const size_t a = align256(act_bytes(&pd)), inner = pass_workspace(&pd, rotate, nobase);
        if (!workspace || workspace_bytes < 2 * a + inner) return WTCONV_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return WTCONV_ERR_UNSUPPORTED;
        char *ws = (char *)workspace;
        if (launch && wtc_launch_repack(d->dtype, in, ws, d->n * d->c, (int)d->h, (int)d->w, (int)pd.h, (int)pd.w,
                                        s) != hipSuccess)
            return WTCONV_ERR_HIP;
        st = fused_pass(&pd, ws, w_base, bias, s_base, w_lvl, s_lvl, ws + a, rotate, ws + 2 * a, inner, stream,
                        zero_base, launch);
        if (st != WTCONV_OK || !launch) return st;
        return wtc_launch_repack(d->dtype, ws + a, out, d->n * d->c, (int)pd.h, (int)pd.w, (int)d->h, (int)d->w,
                                 s) == hipSuccess
                   ? WTCONV_OK
                   : WTCONV_ERR_HIP;
    }
    // the whole-plane kernel when a plane fits one workgroup (any L, even
    // sides for L = 0); else tiles where a tile shape divides the plane; else
    // the row-band kernel for L = 0 and the strip kernel for L >= 1
    hipError_t e = hipSuccess;
    WtcWholePlan wp;
    if (whole_choice(d, rotate, &wp, nobase)) {
        if (launch) e = wtc_launch_whole(d->dtype, wp, in, out, w_base, bias, s_base, w_lvl, s_lvl, s);
    } else if (WtcLargePlan lp; tile_choice(d, rotate, &wp, nobase) && large_choice(d, rotate, &lp, nobase)) {
        if (launch) e = wtc_launch_large(d->dtype, lp, in, out, w_base, bias, s_base, w_lvl, s_lvl, s);
    } else if (tile_choice(d, rotate, &wp, nobase)) {
        const void *low = nullptr;
        if (d->levels >= 2) {
            const size_t need = pass_workspace(d, rotate, nobase);
            if (!workspace || workspace_bytes < need) return WTCONV_ERR_WORKSPACE;
            if (((uintptr_t)workspace & 255u) != 0) return WTCONV_ERR_UNSUPPORTED;
            const wtconv_desc_t sd = deeper_desc(d);
            const size_t quarter = align256(act_bytes(&sd));
            char *ws = (char *)workspace;
            float *ll = (float *)ws;
            void *deep = ws + quarter;
            float *zeros = (float *)(ws + 2 * quarter);
            char *sub = ws + 2 * quarter + align256((size_t)d->c * 4);
            const int64_t kk = (int64_t)d->k * d->k;
            if (launch && wtc_launch_lowpass(d->dtype, in, ll, d->n * d->c, (int)d->h, (int)d->w, s) != hipSuccess)
                return WTCONV_ERR_HIP;
            // the deeper levels: the layer with L - 1 levels and no base path,
            // in fp32
            const float *wl2 = w_lvl + 4 * d->c * kk, *sl2 = s_lvl + 4 * d->c;
            st = fused_pass(&sd, ll, w_base, nullptr, zeros, wl2, sl2, deep, rotate, sub, need - (sub - ws), stream,
                            zeros, launch);
            if (st != WTCONV_OK) return st;
            low = deep;
        }
        if (launch) e = wtc_launch_whole(d->dtype, wp, in, out, w_base, bias, s_base, w_lvl, s_lvl, s, low);
    } else if (d->levels == 0) {
        if (launch)
            e = wtc_launch_dwconv(d->dtype, d->k, in, out, w_base, bias, s_base, (int)d->n, (int)d->c, (int)d->h,
                                  (int)d->w, rotate, s);
    } else {
        WtcFusedPlan p;
        if (no_strips()) return WTCONV_ERR_UNSUPPORTED;
        if (wtc_make_fused_plan(&p, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, rotate,
                                kFusedThreads, lds_budget_floats()) &&
            wtc_make_fused_plan(&p, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, rotate,
                                kFusedThreads, kMaxLdsFloats))
            return WTCONV_ERR_UNSUPPORTED;
        if (!launch) return WTCONV_OK;
        if (nobase) {
            if (wtc_launch_fill(zero_base, d->c, 0.0f, s) != hipSuccess) return WTCONV_ERR_HIP;
            s_base = zero_base;
            bias = nullptr;
        }
        e = wtc_launch_fused(d->dtype, p, in, out, w_base, bias, s_base, w_lvl, s_lvl, s);
    }
    return e == hipSuccess ? WTCONV_OK : WTCONV_ERR_HIP;
}

// A forward / data-backward entry point: the dry run, then the launches.
wtconv_status_t run_pass(const wtconv_desc_t *d, const void *in, const float *w_base, const float *bias,
                         const float *s_base, const float *w_lvl, const float *s_lvl, void *out, int rotate,
                         void *workspace, size_t workspace_bytes, wtconv_stream_t stream)
{
    wtconv_status_t st = fused_pass(d, in, w_base, bias, s_base, w_lvl, s_lvl, out, rotate, workspace,
                                    workspace_bytes, stream, nullptr, false);
    if (st != WTCONV_OK) return st;
    return fused_pass(d, in, w_base, bias, s_base, w_lvl, s_lvl, out, rotate, workspace, workspace_bytes, stream,
                      nullptr, true);
}

// Weight-gradient plan: the whole-plane kernel when the plane fits in LDS,
// otherwise the level-by-level tiled steps.  Both write partial rows
// [groups][C][plen] that the finalize pass reduces.
struct WgradChoice {
    bool whole;        // one plane per workgroup
    bool tiles;        // planes too large: base and level 1 on tiles (wp), deeper levels nested
    WtcWgradPlan wp;
    int groups;
    int plen;          // partial-row length of the kernel that writes them
    WtcWtileCarve cv;
    size_t part_bytes; // partial rows (tiles: at the start of the workspace)
    size_t quarter;    // tiles, L >= 2: bytes of one level-1 low-pass map
    size_t sub_bytes;  // tiles, L >= 2: the nested call's workspace
    size_t total_bytes;
};

int wgrad_groups(const wtconv_desc_t *d)
{
    int forced = env_int("WTCONV_WGRAD_GROUPS", 0, 1, 4096);
    if (forced) return forced;
    // enough workgroups to fill the chip a few times over
    int g = (int)((2048 + d->c - 1) / d->c);
    return g < 1 ? 1 : g;
}

wtconv_status_t wgrad_workspace(const wtconv_desc_t *d, int nobase, size_t *bytes);

// nobase: the base gradients are not wanted (the nested call for the deeper
// levels of a larger layer); its workspace is sized with the same choice.
wtconv_status_t choose_wgrad(const wtconv_desc_t *d, WgradChoice *ch, int nobase = 0)
{
    const int kk = d->k * d->k;
    ch->plen = kk + 1 + 4 * d->levels * kk;
    const int eb = d->dtype == WTCONV_F32 ? 4 : 2;
    // 256 threads, 512 when a plane has more than two pieces per thread of 256
    // (64 x 64 planes: 3 % faster; at the 56 x 56 and 28 x 28 planes 512
    // threads measured slower); WTCONV_WGRAD_THREADS overrides
    const int forced_wth = env_int("WTCONV_WGRAD_THREADS", 0, 64, 512);
    int wth = forced_wth ? forced_wth : kFusedThreads;
    ch->whole = !env_int("WTCONV_NO_WHOLE", 0, 0, 1) &&
                wtc_make_wgrad_plan(&ch->wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, wth, 1,
                                    eb, whole_budget_floats(), nobase) == 0;
    if (ch->whole && !forced_wth && ch->wp.npieces > 2 * kFusedThreads &&
        wtc_make_wgrad_plan(&ch->wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels,
                            2 * kFusedThreads, 1, eb, whole_budget_floats(), nobase) == 0)
        wth = 2 * kFusedThreads;
    ch->tiles = false;
    // levels carried by the tiles (base and level 1; L = 0: the base alone)
    const int tl = d->levels >= 1 ? 1 : 0;
    if (!ch->whole && !env_int("WTCONV_NO_TILES", 0, 0, 1)) {
        // planes too large for one workgroup: base and level-1 correlations on
        // tiles (L = 1 partial rows); levels 2..L are the layer with L - 1
        // levels on the level-1 low-pass maps of x and dy, a nested call
        // 64 x 64 tiles on 512 threads first (128 x 128 weight backward: fp16
        // L = 1 145.7 -> 141.3 us, L = 3 189.7 -> 186.9 us, fp32 L = 1 1-4 %
        // faster, the other points within 1 %), unless the tile knobs are
        // set; then fp32: 16 x 128 tiles first; fp16: 32 x 64 (128 x 128 fp16
        // weight backward 3.5 % faster, fp32 within 1 %), on tile_threads()
        // threads
        const TileShapes shapes = tile_shapes(d->dtype == WTCONV_F32);
        int cand[12][3], nc = 0;
        if (!std::getenv("WTCONV_TILE") && !std::getenv("WTCONV_TILE_THREADS")) {
            cand[nc][0] = 64;
            cand[nc][1] = 64;
            cand[nc++][2] = 2 * kFusedThreads;
        }
        for (int si = 0; si < shapes.n && nc < 12; ++si, ++nc) {
            cand[nc][0] = shapes.s[si][0];
            cand[nc][1] = shapes.s[si][1];
            cand[nc][2] = tile_threads();
        }
        for (int ci = 0; ci < nc; ++ci) {
            const int *sh = cand[ci];
            if (d->h % sh[0] || d->w % sh[1] || (sh[0] == d->h && sh[1] == d->w)) continue;
            if (wtc_make_wgrad_tile_plan(&ch->wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, sh[0], sh[1], d->k,
                                         tl, sh[2], 1, eb, whole_budget_floats(), nobase))
                continue;
            const int resident = wtc_wgrad_resident(d->dtype, ch->wp);
            int planes = env_int("WTCONV_WGRAD_PLANES", 0, 1, 1 << 20);
            if (!planes) planes = wtc_choose_planes(ch->wp.units, d->c, resident > 0 ? resident : 512, kWgradFixed);
            wtc_make_wgrad_tile_plan(&ch->wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, sh[0], sh[1], d->k,
                                     tl, sh[2], planes, eb, whole_budget_floats(), nobase);
            ch->tiles = true;
            break;
        }
    }
    if (ch->tiles) {
        ch->groups = ch->wp.groups;
        ch->plen = (1 + 4 * tl) * kk + 1;
        ch->part_bytes = align256((size_t)ch->groups * d->c * ch->plen * 4);
        ch->quarter = ch->sub_bytes = 0;
        if (d->levels >= 2) {
            const wtconv_desc_t sd = deeper_desc(d);  // fp32 low-pass maps
            ch->quarter = align256(act_bytes(&sd));
            size_t sub = 0;
            wtconv_status_t st = wgrad_workspace(&sd, 1, &sub);
            if (st != WTCONV_OK) return st;
            ch->sub_bytes = sub;
        }
        // partials | LL(x) | LL(dy) | scratch base gradients (C k^2 + 2C floats) | nested workspace
        ch->total_bytes = ch->part_bytes + 2 * ch->quarter +
                          (d->levels >= 2 ? align256((size_t)d->c * (kk + 2) * 4) + ch->sub_bytes : 0);
        return WTCONV_OK;
    }
    if (ch->whole) {
        wtc_make_wgrad_plan(&ch->wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, wth, 1, eb,
                            whole_budget_floats(), nobase);
        const int planes = pick_planes(d, wtc_wgrad_resident(d->dtype, ch->wp), kWgradFixed,
                                       "WTCONV_WGRAD_PLANES");
        wtc_make_wgrad_plan(&ch->wp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, wth, planes, eb,
                            whole_budget_floats(), nobase);
        ch->groups = ch->wp.groups;
    } else {
        if (no_strips()) return WTCONV_ERR_UNSUPPORTED;
        ch->groups = (int)wgrad_groups(d);
        for (int j = 0; j <= d->levels; ++j) {
            WtcWtilePlan tp;
            if (wtc_make_wtile_plan(&tp, (int)d->n, (int)d->c, d->k, d->levels, j, (int)(d->h >> j),
                                    (int)(d->w >> j), kFusedThreads, ch->groups, kMaxLdsFloats))
                return WTCONV_ERR_UNSUPPORTED;
        }
    }
    wtc_wtile_carve(&ch->cv, d->n, d->c, d->h, d->w, ch->whole ? 0 : d->levels, ch->groups, ch->plen);
    ch->total_bytes = ch->cv.total;
    return WTCONV_OK;
}

// Workspace of the weight backward (nobase: see choose_wgrad).
wtconv_status_t wgrad_workspace(const wtconv_desc_t *d, int nobase, size_t *bytes)
{
    WgradChoice ch;
    const wtconv_desc_t pd = padded_desc(d);
    wtconv_status_t st = check_desc(&pd);
    if (st != WTCONV_OK) return st;
    if ((st = choose_wgrad(&pd, &ch, nobase)) != WTCONV_OK) return st;
    // ragged sides: zero-padded copies of x and dy ahead of the padded call's workspace
    *bytes = (ragged(d) ? 2 * align256(act_bytes(&pd)) : 0) + ch.total_bytes;
    return WTCONV_OK;
}

// Fused single-pass backward plan (512 threads; WTCONV_BWD_THREADS=256
// overrides), with its images per workgroup; false where it does not apply or
// is not selected.  It is correct but measured slower than the two calls on
// MI355X (stage1 151.5 against 126.3 us, stage2 125.6 against 83.1 us: with
// both pyramids, the convolution outputs and the accumulators a compute unit
// holds one 512-thread workgroup, where the two calls keep 16 and 8 waves in
// flight), so the two calls are the default and WTCONV_FUSED_BWD=1 selects it.
bool bwd_choice(const wtconv_desc_t *d, WtcBwdPlan *bp)
{
    if (!env_int("WTCONV_FUSED_BWD", 0, 0, 1) || d->levels < 1 || ragged(d) || env_int("WTCONV_NO_WHOLE", 0, 0, 1))
        return false;
    const int eb = d->dtype == WTCONV_F32 ? 4 : 2;
    const int nth = env_int("WTCONV_BWD_THREADS", 512, 256, 512) >= 512 ? 512 : 256;
    if (wtc_make_bwd_plan(bp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, nth, 1, eb,
                          whole_budget_floats()))
        return false;
    const int planes = pick_planes(d, wtc_bwd_resident(d->dtype, *bp), kWgradFixed, "WTCONV_BWD_PLANES");
    return wtc_make_bwd_plan(bp, (int)d->n, (int)d->c, (int)d->h, (int)d->w, d->k, d->levels, nth, planes, eb,
                             whole_budget_floats()) == 0;
}

size_t bwd_partial_bytes(const wtconv_desc_t *d, const WtcBwdPlan &bp)
{
    return align256((size_t)bp.g.groups * d->c * bp.g.plen * 4);
}

// Workspace of wtconv_backward: the fused pass's partial rows, else the larger
// of the two calls' workspaces (they run one after the other).
wtconv_status_t bwd_workspace(const wtconv_desc_t *d, size_t *bytes)
{
    WtcBwdPlan bp;
    if (bwd_choice(d, &bp)) {
        *bytes = bwd_partial_bytes(d, bp);
        return WTCONV_OK;
    }
    size_t wb = 0;
    wtconv_status_t st = wgrad_workspace(d, 0, &wb);
    if (st != WTCONV_OK) return st;
    const size_t pb = pass_workspace(d, 1, 0);
    *bytes = wb > pb ? wb : pb;
    return WTCONV_OK;
}

}  // namespace

int wtc_resident_blocks(const void *fn, int nthreads, size_t lds)
{
    struct Entry {
        const void *fn;
        int dev, nthreads;
        size_t lds;
        int resident;
    };
    static std::mutex mu;
    static Entry cache[64];
    static int used = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; ++i)
            if (cache[i].fn == fn && cache[i].dev == dev && cache[i].nthreads == nthreads && cache[i].lds == lds)
                return cache[i].resident;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, nthreads, lds) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();  // leave no error for the next launch check to report
        return 0;
    }
    const int resident = per_cu * cus;
    std::lock_guard<std::mutex> lock(mu);
    if (used < 64) cache[used++] = Entry{fn, dev, nthreads, lds, resident};
    return resident;
}

// ---- The weight backward without a caller's workspace ---------------------
// Its partial rows live in this file-scope device array, one copy per GPU; in
// host code `scratch` only names the symbol, so the kernels get the per-device
// address that hipGetSymbolAddress returns (looked up once per device, with
// that device current).
static __device__ __align__(256) unsigned char scratch[WTCONV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

void *scratch_address(int dev)
{
    static std::mutex mu;
    static void *ptr[kMaxDevices];
    static bool done[kMaxDevices];
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!done[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        ptr[dev] = p;
        done[dev] = true;
    }
    return ptr[dev];
}

}  // namespace

extern "C" {

wtconv_status_t wtconv_workspace_size(const wtconv_desc_t *desc, wtconv_op_t op, size_t *bytes)
{
    wtconv_status_t st = check_desc(desc);
    if (st != WTCONV_OK) return st;
    if (!bytes) return WTCONV_ERR_NULL;
    switch (op) {
    case WTCONV_OP_FWD: *bytes = pass_workspace(desc, 0, 0); return WTCONV_OK;
    case WTCONV_OP_BWD_DATA: *bytes = pass_workspace(desc, 1, 0); return WTCONV_OK;
    case WTCONV_OP_BWD_WEIGHT: return wgrad_workspace(desc, 0, bytes);
    case WTCONV_OP_BWD: return bwd_workspace(desc, bytes);
    default: return WTCONV_ERR_UNSUPPORTED;
    }
}

// The weight backward; nobase: the base gradients are not wanted (the nested
// call for the deeper levels of a larger layer, which writes them to
// scratch): the whole-plane and tiled kernels skip them and write 0.
// launch = false: the dry run (see fused_pass).
// fin: the partial-row sets of the calls above this one (null for the
// outermost call).  Every call adds its own; the outermost call finalizes all
// of them with one launch after the last correlation kernel.
static wtconv_status_t wgrad_pass(const wtconv_desc_t *desc, const void *x, const void *dy, const float *w_base,
                                  const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
                                  float *dw_base, float *dbias, float *ds_base, float *dw_lvl, float *ds_lvl,
                                  void *workspace, size_t workspace_bytes, wtconv_stream_t stream, int nobase,
                                  bool launch, WtcFinalizeSets *fin = nullptr)
{
    WtcFinalizeSets own;
    const bool outer = fin == nullptr;
    if (outer) {
        own.C = (int)desc->c;
        own.k = desc->k;
        own.n = 0;
        fin = &own;
    }
    // this call's set (levels of its partial rows, their layout), and the
    // outermost call's single finalize launch
    auto add_set = [&](int levels, int groups, int plen, const float *partial) -> bool {
        if (fin->n >= WTC_FIN_MAX) return false;
        fin->s[fin->n++] = WtcFinalizeSet{levels, groups, plen, partial, w_base, bias, s_base, w_lvl, s_lvl,
                                          dw_base, dbias, ds_base, dw_lvl, ds_lvl};
        return true;
    };
    auto finish = [&](hipStream_t hs) -> wtconv_status_t {
        if (!outer || !launch) return WTCONV_OK;
        return wtc_launch_wgrad_finalize_sets(*fin, hs) == hipSuccess ? WTCONV_OK : WTCONV_ERR_HIP;
    };
    wtconv_status_t st = check_desc(desc);
    if (st != WTCONV_OK) return st;
    if (!x || !dy || !dw_base || !dbias || !ds_base) return WTCONV_ERR_NULL;
    if ((st = check_params(desc, w_base, s_base, w_lvl, s_lvl)) != WTCONV_OK) return st;
    if (desc->levels > 0 && (!dw_lvl || !ds_lvl)) return WTCONV_ERR_NULL;
    if (!aligned16(x) || !aligned16(dy)) return WTCONV_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    if (ragged(desc)) {
        // the gradients of the layer on zero-padded copies of x and dy
        const wtconv_desc_t pd = padded_desc(desc);
        if ((st = check_desc(&pd)) != WTCONV_OK) return st;
        size_t need = 0;
        if ((st = wgrad_workspace(desc, nobase, &need)) != WTCONV_OK) return st;
        if (!workspace || workspace_bytes < need) return WTCONV_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return WTCONV_ERR_UNSUPPORTED;
        const size_t a = align256(act_bytes(&pd));
        char *ws = (char *)workspace;
        const int64_t planes = desc->n * desc->c;
        if (launch &&
            (wtc_launch_repack(desc->dtype, x, ws, planes, (int)desc->h, (int)desc->w, (int)pd.h, (int)pd.w, s) !=
                 hipSuccess ||
             wtc_launch_repack(desc->dtype, dy, ws + a, planes, (int)desc->h, (int)desc->w, (int)pd.h, (int)pd.w,
                               s) != hipSuccess))
            return WTCONV_ERR_HIP;
        return wgrad_pass(&pd, ws, ws + a, w_base, bias, s_base, w_lvl, s_lvl, dw_base, dbias, ds_base, dw_lvl,
                          ds_lvl, ws + 2 * a, workspace_bytes - 2 * a, stream, nobase, launch,
                          outer ? nullptr : fin);
    }
    WgradChoice ch;
    if ((st = choose_wgrad(desc, &ch, nobase)) != WTCONV_OK) return st;
    if (!workspace || workspace_bytes < ch.total_bytes) return WTCONV_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return WTCONV_ERR_UNSUPPORTED;
    char *ws = (char *)workspace;
    float *partial = (float *)ws;
    hipError_t e = hipSuccess;
    if (ch.tiles) {
        // with L >= 2 the tiles also write the level-1 low-pass maps of x and
        // dy (every tile its interior, fp32), the inputs of the nested call
        char *llx = desc->levels >= 2 ? ws + ch.part_bytes : nullptr;
        char *lld = desc->levels >= 2 ? llx + ch.quarter : nullptr;
        if (desc->levels >= 2) {
            // levels 2..L: the layer with L - 1 levels on the low-pass maps,
            // its base gradients not wanted (written to scratch); checked here,
            // launched after the tiles
            const wtconv_desc_t sd = deeper_desc(desc);
            float *scratch = (float *)(lld + ch.quarter);
            char *sub = (char *)scratch + align256((size_t)desc->c * (desc->k * desc->k + 2) * 4);
            const int64_t kk = (int64_t)desc->k * desc->k, C = desc->c;
            if (launch && wtc_launch_wgrad(desc->dtype, ch.wp, x, dy, partial, s, llx, lld) != hipSuccess)
                return WTCONV_ERR_HIP;
            if (!add_set(1, ch.groups, ch.plen, partial)) return WTCONV_ERR_UNSUPPORTED;
            st = wgrad_pass(&sd, llx, lld, w_base, nullptr, s_base, w_lvl + 4 * C * kk, s_lvl + 4 * C, scratch,
                            scratch + C * kk, scratch + C * kk + C, dw_lvl + 4 * C * kk, ds_lvl + 4 * C, sub,
                            ch.sub_bytes, stream, 1, launch, fin);
            return st != WTCONV_OK ? st : finish(s);
        }
        if (!add_set(desc->levels >= 1 ? 1 : 0, ch.groups, ch.plen, partial)) return WTCONV_ERR_UNSUPPORTED;
        if (launch && wtc_launch_wgrad(desc->dtype, ch.wp, x, dy, partial, s) != hipSuccess) return WTCONV_ERR_HIP;
        return finish(s);
    }
    if (!add_set(desc->levels, ch.groups, ch.plen, partial)) return WTCONV_ERR_UNSUPPORTED;
    if (!launch) return WTCONV_OK;
    if (ch.whole) {
        e = wtc_launch_wgrad(desc->dtype, ch.wp, x, dy, partial, s);
    } else {
        float *bx[2] = {(float *)(ws + ch.cv.off_ux[0]), (float *)(ws + ch.cv.off_ux[1])};
        float *bd[2] = {(float *)(ws + ch.cv.off_ud[0]), (float *)(ws + ch.cv.off_ud[1])};
        const void *cx = x, *cd = dy;
        int dt = desc->dtype;
        for (int j = 0; j <= desc->levels && e == hipSuccess; ++j) {
            WtcWtilePlan tp;
            wtc_make_wtile_plan(&tp, (int)desc->n, (int)desc->c, desc->k, desc->levels, j, (int)(desc->h >> j),
                                (int)(desc->w >> j), kFusedThreads, ch.groups, kMaxLdsFloats);
            float *ux = j < desc->levels ? bx[j % 2] : nullptr;
            float *ud = j < desc->levels ? bd[j % 2] : nullptr;
            e = wtc_launch_wgrad_tile(dt, tp, cx, cd, ux, ud, partial, s);
            cx = ux;
            cd = ud;
            dt = WTCONV_F32;
        }
    }
    if (e != hipSuccess) return WTCONV_ERR_HIP;
    return finish(s);
}

wtconv_status_t wtconv_backward_weight_noalloc(const wtconv_desc_t *desc, const void *x, const void *dy,
                                               const float *w_base, const float *bias, const float *s_base,
                                               const float *w_lvl, const float *s_lvl, float *dw_base, float *dbias,
                                               float *ds_base, float *dw_lvl, float *ds_lvl, wtconv_stream_t stream)
{
    size_t need = 0;
    wtconv_status_t st = check_desc(desc);
    if (st != WTCONV_OK) return st;
    if ((st = wgrad_workspace(desc, 0, &need)) != WTCONV_OK) return st;
    if (need > (size_t)WTCONV_NOALLOC_SCRATCH_BYTES) return WTCONV_ERR_WORKSPACE;
    // the whole call checked with a stand-in address before anything else
    void *const probe = (void *)(uintptr_t)256;
    st = wgrad_pass(desc, x, dy, w_base, bias, s_base, w_lvl, s_lvl, dw_base, dbias, ds_base, dw_lvl, ds_lvl, probe,
                    WTCONV_NOALLOC_SCRATCH_BYTES, stream, 0, false);
    if (st != WTCONV_OK) return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return WTCONV_ERR_HIP;
    }
    void *ws = scratch_address(dev);
    if (!ws) return WTCONV_ERR_HIP;
    return wgrad_pass(desc, x, dy, w_base, bias, s_base, w_lvl, s_lvl, dw_base, dbias, ds_base, dw_lvl, ds_lvl, ws,
                      WTCONV_NOALLOC_SCRATCH_BYTES, stream, 0, true);
}

wtconv_status_t wtconv_backward_weight(const wtconv_desc_t *desc, const void *x, const void *dy,
                                       const float *w_base, const float *bias, const float *s_base,
                                       const float *w_lvl, const float *s_lvl, float *dw_base, float *dbias,
                                       float *ds_base, float *dw_lvl, float *ds_lvl, void *workspace,
                                       size_t workspace_bytes, wtconv_stream_t stream)
{
    wtconv_status_t st = wgrad_pass(desc, x, dy, w_base, bias, s_base, w_lvl, s_lvl, dw_base, dbias, ds_base,
                                    dw_lvl, ds_lvl, workspace, workspace_bytes, stream, 0, false);
    if (st != WTCONV_OK) return st;
    return wgrad_pass(desc, x, dy, w_base, bias, s_base, w_lvl, s_lvl, dw_base, dbias, ds_base, dw_lvl, ds_lvl,
                      workspace, workspace_bytes, stream, 0, true);
}

wtconv_status_t wtconv_backward(const wtconv_desc_t *desc, const void *x, const void *dy, const float *w_base,
                                const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
                                void *dx, float *dw_base, float *dbias, float *ds_base, float *dw_lvl, float *ds_lvl,
                                void *workspace, size_t workspace_bytes, wtconv_stream_t stream)
{
    wtconv_status_t st = check_desc(desc);
    if (st != WTCONV_OK) return st;
    if (!x || !dy || !dx || !dw_base || !dbias || !ds_base) return WTCONV_ERR_NULL;
    if ((st = check_params(desc, w_base, s_base, w_lvl, s_lvl)) != WTCONV_OK) return st;
    if (desc->levels > 0 && (!dw_lvl || !ds_lvl)) return WTCONV_ERR_NULL;
    if (!aligned16(x) || !aligned16(dy) || !aligned16(dx)) return WTCONV_ERR_UNSUPPORTED;
    if (overlaps(dx, dy, act_bytes(desc)) || overlaps(dx, x, act_bytes(desc))) return WTCONV_ERR_ALIAS;
    WtcBwdPlan bp;
    if (!bwd_choice(desc, &bp)) {
        // the two calls, each checked in full before anything is enqueued
        st = fused_pass(desc, dy, w_base, nullptr, s_base, w_lvl, s_lvl, dx, 1, workspace, workspace_bytes, stream,
                        nullptr, false);
        if (st == WTCONV_OK)
            st = wgrad_pass(desc, x, dy, w_base, bias, s_base, w_lvl, s_lvl, dw_base, dbias, ds_base, dw_lvl, ds_lvl,
                            workspace, workspace_bytes, stream, 0, false);
        if (st != WTCONV_OK) return st;
        st = fused_pass(desc, dy, w_base, nullptr, s_base, w_lvl, s_lvl, dx, 1, workspace, workspace_bytes, stream,
                        nullptr, true);
        if (st != WTCONV_OK) return st;
        return wgrad_pass(desc, x, dy, w_base, bias, s_base, w_lvl, s_lvl, dw_base, dbias, ds_base, dw_lvl, ds_lvl,
                          workspace, workspace_bytes, stream, 0, true);
    }
    if (!workspace || workspace_bytes < bwd_partial_bytes(desc, bp)) return WTCONV_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return WTCONV_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    float *partial = (float *)workspace;
    hipError_t e = wtc_launch_bwd(desc->dtype, bp, x, dy, dx, w_base, s_base, w_lvl, s_lvl, partial, s);
    if (e == hipSuccess)
        e = wtc_launch_wgrad_finalize((int)desc->c, desc->k, desc->levels, bp.g.groups, bp.g.plen, partial, w_base,
                                      bias, s_base, w_lvl, s_lvl, dw_base, dbias, ds_base, dw_lvl, ds_lvl, s);
    return e == hipSuccess ? WTCONV_OK : WTCONV_ERR_HIP;
}

wtconv_status_t wtconv_forward(const wtconv_desc_t *desc, const void *x, const float *w_base, const float *bias,
                               const float *s_base, const float *w_lvl, const float *s_lvl, void *y,
                               void *workspace, size_t workspace_bytes, wtconv_stream_t stream)
{
    return run_pass(desc, x, w_base, bias, s_base, w_lvl, s_lvl, y, 0, workspace, workspace_bytes, stream);
}

wtconv_status_t wtconv_backward_data(const wtconv_desc_t *desc, const void *dy, const float *w_base,
                                     const float *s_base, const float *w_lvl, const float *s_lvl, void *dx,
                                     void *workspace, size_t workspace_bytes, wtconv_stream_t stream)
{
    return run_pass(desc, dy, w_base, nullptr, s_base, w_lvl, s_lvl, dx, 1, workspace, workspace_bytes, stream);
}

const char *wtconv_status_string(wtconv_status_t status)
{
    switch (status) {
    case WTCONV_OK: return "ok";
    case WTCONV_ERR_NULL: return "a required pointer is NULL";
    case WTCONV_ERR_SHAPE: return "invalid shape, level count or divisibility";
    case WTCONV_ERR_UNSUPPORTED: return "unsupported kernel size, dtype, alignment or size";
    case WTCONV_ERR_WORKSPACE: return "workspace missing or too small";
    case WTCONV_ERR_HIP: return "HIP launch error";
    case WTCONV_ERR_ALIAS: return "an output overlaps an input";
    default: return "unknown status";
    }
}

const char *wtconv_version(void) { return "0.1.0"; }

}  // extern "C"
