// wtconv_emu.cpp -- CPU emulation of the fused WTConv kernels (test tool).
//
// Runs the very phase functions the GPU kernels run (wtconv_fused_body.h),
// one workgroup after another and, inside a phase, one thread after another,
// with every LDS, input and output access bounds-checked (an out-of-range
// index aborts the process with its line number).  Barriers fall between
// phases, so this ordering is one legal interleaving of the workgroup.  Used
// by the CPU test suite to check the tiling, strip and LDS-layout logic against
// the oracle before any GPU run; it is never part of the product library.
#define WTC_EMULATE 1
#include <cstdint>
#include <cstring>
#include <algorithm>
#include <array>
#include <vector>

#include "../../level_haar_wavelet_amd/csrc/wtconv_bwd_body.h"
#include "../../level_haar_wavelet_amd/csrc/wtconv_fused_body.h"
#include "../../level_haar_wavelet_amd/csrc/wtconv_large_body.h"
#include "../../level_haar_wavelet_amd/csrc/wtconv_whole_body.h"
#include "../../level_haar_wavelet_amd/csrc/wtconv_wgrad_body.h"
#include "../../level_haar_wavelet_amd/csrc/wtconv_wgrad_tile_body.h"

template <typename T, int K, int BW>
static void run_fused(const WtcFusedArgs<T> &a)
{
    const WtcFusedPlan &p = a.p;
    const int nblocks = p.n * p.c * p.tiles_y * p.tiles_x;
    std::vector<float> lds((size_t)p.lds_floats);
    const int nth = p.nthreads;
    for (int bid = 0; bid < nblocks; ++bid) {
        // poison LDS so that a read of a value no phase wrote shows up as NaN
        for (auto &v : lds) v = __builtin_nanf("");
        std::vector<WtcCtx<T>> ctx((size_t)nth);
        for (int t = 0; t < nth; ++t) {
            ctx[t].lds = lds.data();
            ctx[t].tid = t;
            ctx[t].nth = nth;
            ctx[t].lds_n = p.lds_floats;
            ctx[t].plane_n = (int64_t)p.h * p.w;
            wtc_fused_setup<T>(a, ctx[t], bid, nblocks);
        }
        for (int t = 0; t < nth; ++t) wtc_phase_fold<T, K>(a, ctx[t]);
        for (int t = 0; t < nth; ++t) wtc_phase_coarse<T, K>(a, ctx[t]);
        for (int m = 2; m <= p.levels; ++m)
            for (int t = 0; t < nth; ++t) wtc_phase_deep_level<T, K>(a, ctx[t], m);
        for (int t = 0; t < nth; ++t) wtc_phase_deep_conv<T, K>(a, ctx[t]);
        const int ty0 = ctx[0].ty0;
        for (int s0 = ty0; s0 < ty0 + p.tile_h; s0 += p.strip_h) {
            for (int t = 0; t < nth; ++t) wtc_phase_stage<T, K>(a, ctx[t], s0);
            for (int t = 0; t < nth; ++t) wtc_phase_strip_bands<T, K>(a, ctx[t], s0);
            for (int t = 0; t < nth; ++t) wtc_phase_strip_conv1<T, K>(a, ctx[t], s0);
            for (int t = 0; t < nth; ++t) wtc_phase_strip_out<T, K, BW>(a, ctx[t], s0);
        }
    }
}

template <typename T, int K>
static void run_k(const WtcFusedArgs<T> &a)
{
    switch (a.p.out_bw) {
    case 8: run_fused<T, K, 8>(a); break;
    case 4: run_fused<T, K, 4>(a); break;
    default: run_fused<T, K, 2>(a); break;
    }
}

template <typename T>
static int run_t(const WtcFusedArgs<T> &a)
{
    switch (a.p.k) {
    case 1: run_k<T, 1>(a); return 0;
    case 3: run_k<T, 3>(a); return 0;
    case 5: run_k<T, 5>(a); return 0;
    case 7: run_k<T, 7>(a); return 0;
    default: return -1;
    }
}

// Haar level 3 across lane quads (the kernel exchanges the quad's level-2 sums
// by DPP right after staging; here every thread has staged first).
template <typename T>
static void emu_stage_l3(const WtcWholeArgs<T> &a, std::vector<WtcWholeCtx<T>> &ctx)
{
    for (size_t t = 0; t < ctx.size(); ++t) {
        if (!ctx[t].gvalid) continue;
        float v[4];
        for (int j = 0; j < 4; ++j) {
            const WtcWholeCtx<T> &o = ctx[(t & ~(size_t)3) | (size_t)j];
            if (!o.gvalid) abort();  // quads are whole
            v[j] = o.u2;
        }
        wtc_whole_stage_l3(a, ctx[t], v);
    }
}

template <typename T, int K, int BW, bool TL, bool ST = false, bool G4 = TL || ST, int LV = 0>
static void run_whole(const WtcWholeArgs<T> &a)
{
    const WtcWholePlan &p = a.p;
    const int groups = (p.units + p.planes - 1) / p.planes;
    const int nblocks = groups * p.c;
    std::vector<float> lds((size_t)p.lds_floats);
    const int nth = p.nthreads;
    if (TL && p.tail) {  // as the launch: the tiled instances carry no tail loop
        fprintf(stderr, "wtconv emulation: a tiled plan with a piece tail\n");
        abort();
    }
    for (int bid = 0; bid < nblocks; ++bid) {
        // poison LDS: the kernel must zero it before use
        for (auto &v : lds) v = __builtin_nanf("");
        std::vector<WtcWholeCtx<T>> ctx((size_t)nth);
        for (int t = 0; t < nth; ++t) {
            ctx[t].lds = lds.data();
            ctx[t].tid = t;
            ctx[t].nth = nth;
            ctx[t].lds_n = p.lds_floats;
            // stacked plans address outputs from the tensor base
            ctx[t].img_n = ST ? (int64_t)p.n * p.c * p.sh * p.iw : (int64_t)p.ih * p.iw;
            wtc_whole_setup<T>(a, ctx[t], bid);
        }
        for (int t = 0; t < nth; ++t) wtc_whole_load<T, K, BW, TL, ST, G4>(a, ctx[t], 0);
        for (int t = 0; t < nth; ++t) wtc_whole_init<T, K>(a, ctx[t]);
        for (int t = 0; t < nth; ++t) wtc_whole_fold<T, K>(a, ctx[t]);
        for (int t = 0; t < nth; ++t) wtc_whole_table<T, K, BW>(a, ctx[t]);
        // the kernel's software pipeline: image i+1 is staged in the same
        // barrier interval as image i's output pass (here every staging runs
        // first, so a staging write that the output pass reads would show)
        for (int t = 0; t < nth; ++t) wtc_whole_stage<T, K, BW, TL, ST, G4>(a, ctx[t]);
        if (p.stage_l3) emu_stage_l3(a, ctx);
        for (int t = 0; t < nth; ++t)
            if (ctx[t].nimg > 1) wtc_whole_load<T, K, BW, TL, ST, G4>(a, ctx[t], 1);
        for (int img = 0; img < ctx[0].nimg; ++img) {
            for (int m = wtc_whole_first_deep(p); m <= p.levels; ++m)
                for (int t = 0; t < nth; ++t) wtc_whole_analysis<T, K>(a, ctx[t], m);
            for (int t = 0; t < nth; ++t) wtc_whole_conv<T, K, BW, !TL>(a, ctx[t]);
            for (int t = 0; t < nth; ++t) {
                if (img + 1 < ctx[t].nimg) wtc_whole_stage<T, K, BW, TL, ST, G4>(a, ctx[t]);
                if (img + 2 < ctx[t].nimg) wtc_whole_load<T, K, BW, TL, ST, G4>(a, ctx[t], img + 2);
            }
            if (p.stage_l3 && img + 1 < ctx[0].nimg) emu_stage_l3(a, ctx);
            for (int t = 0; t < nth; ++t) {
                wtc_whole_select<T, ST>(a, ctx[t], img);
                wtc_whole_out<T, K, BW, TL, ST, 0, LV>(a, ctx[t]);
            }
        }
    }
}

template <typename T, int K>
static void run_whole_k(const WtcWholeArgs<T> &a)
{
    if (a.p.tiled) {
        switch (a.p.out_bw) {
        case 8: run_whole<T, K, 8, true>(a); break;
        case 4:
            // as the launch: L = 1 tiles take the instance that knows it
            if (a.p.levels == 1)
                run_whole<T, K, 4, true, false, true, 1>(a);
            else
                run_whole<T, K, 4, true>(a);
            break;
        default: run_whole<T, K, 2, true>(a); break;
        }
        return;
    }
    if (a.p.stack > 1) {
        switch (a.p.out_bw) {
        case 8: run_whole<T, K, 8, false, true>(a); break;
        case 4: run_whole<T, K, 4, false, true>(a); break;
        default: run_whole<T, K, 2, false, true>(a); break;
        }
        return;
    }
    switch (a.p.out_bw) {
    case 8: run_whole<T, K, 8, false>(a); break;
    case 4: run_whole<T, K, 4, false>(a); break;
    default: run_whole<T, K, 2, false>(a); break;
    }
}

template <typename T>
static int run_whole_t(const WtcWholeArgs<T> &a)
{
    switch (a.p.k) {
    case 1: run_whole_k<T, 1>(a); return 0;
    case 3: run_whole_k<T, 3>(a); return 0;
    case 5: run_whole_k<T, 5>(a); return 0;
    case 7: run_whole_k<T, 7>(a); return 0;
    default: return -1;
    }
}

// The fused large-plane kernel, phase by phase.  After the deeper levels'
// output pass and after every image's tiles, the aliased map region is
// poisoned with NaN: the tiles must write every element they read (their
// staging covers the halos), and the deeper levels must zero their own maps.
// DL: the deeper-levels plan's level count, as the kernel instance has it
// (0: read from the plan)
template <typename T, int K, int BW, int DL, bool HALF = false>
static void run_large(const WtcLargeArgs<T> &A)
{
    if (HALF && !A.t.p.halves) abort();
    if (DL && (wtc_whole_first_deep(A.d.p) != (DL >= 3 ? 4 : (DL >= 2 ? 3 : 2)) || A.d.p.levels != DL)) {
        fprintf(stderr, "wtconv emulation: deeper-levels plan does not match its instance\n");
        abort();
    }
    if (A.d.p.tail || A.t.p.tail) {  // the kernel carries no tail loop
        fprintf(stderr, "wtconv emulation: a large-plane plan with a piece tail\n");
        abort();
    }
    if (A.t.p.levels != 1) {  // as the launch: the tiles' output pass assumes level 1
        fprintf(stderr, "wtconv emulation: a large-plane tile plan without level 1\n");
        abort();
    }
    const WtcLargeArgs<T> &lp = A;
    const WtcWholeArgs<T> &ad = A.d, &at = A.t;
    const int groups = (lp.n + lp.planes - 1) / lp.planes;
    const int nblocks = groups * lp.c;
    std::vector<float> lds((size_t)lp.lds_floats);
    const int nth = at.p.nthreads;
    const int tiles = at.p.tiles_x * at.p.tiles_y;
    auto poison_maps = [&]() {
        for (int i = lp.maps_off; i < lp.maps_off + lp.maps_floats; ++i) lds[(size_t)i] = __builtin_nanf("");
    };
    for (int bid = 0; bid < nblocks; ++bid) {
        for (auto &v : lds) v = __builtin_nanf("");
        std::vector<WtcWholeCtx<T>> cd((size_t)nth), ct((size_t)nth);
        for (int t = 0; t < nth; ++t) {
            for (auto *c : {&cd[t], &ct[t]}) {
                c->lds = lds.data();
                c->tid = t;
                c->nth = nth;
                c->lds_n = lp.lds_floats;
                c->img_n = (int64_t)lp.h * lp.w;
            }
            wtc_whole_setup<T>(ad, cd[t], bid);
            wtc_whole_setup<T>(at, ct[t], bid);
        }
        for (int i = 0; i < lp.lds_floats; ++i) lds[(size_t)i] = 0.0f;
        for (int t = 0; t < nth; ++t) {
            wtc_whole_fold<T, K>(ad, cd[t]);
            wtc_whole_fold<T, K>(at, ct[t]);
            wtc_whole_table<T, K, BW>(ad, cd[t]);
            wtc_whole_table<T, K, BW>(at, ct[t]);
        }
        for (int img = 0; img < cd[0].nimg; ++img) {
            std::vector<std::array<std::array<float, 4>, 4>> ll((size_t)nth);
            for (int t = 0; t < nth; ++t) {
                WtcLargeRaw<T> raw;
                wtc_large_fetch_d<T>(A, cd[t], img, raw);
                float v[4][4];
                wtc_large_reduce_d<T>(raw, v);
                for (int i = 0; i < 4; ++i)
                    for (int j = 0; j < 4; ++j) ll[(size_t)t][(size_t)i][(size_t)j] = v[i][j];
            }
            if (img > 0)
                for (int t = 0; t < nth; ++t) wtc_large_zero_d<T>(A, cd[t]);
            for (int t = 0; t < nth; ++t) {
                float v[4][4];
                for (int i = 0; i < 4; ++i)
                    for (int j = 0; j < 4; ++j) v[i][j] = ll[(size_t)t][(size_t)i][(size_t)j];
                wtc_whole_stage_vals<T, K, BW, false, false, true, DL>(ad, cd[t], v);
            }
            if (ad.p.stage_l3) emu_stage_l3(ad, cd);
            const int u0 = img * tiles;
            for (int t = 0; t < nth; ++t) wtc_whole_load<T, K, BW, true, false>(at, ct[t], u0);
            for (int m = DL ? (DL >= 3 ? 4 : (DL >= 2 ? 3 : 2)) : wtc_whole_first_deep(ad.p);
                 m <= (DL ? DL : ad.p.levels); ++m)
                for (int t = 0; t < nth; ++t) wtc_whole_analysis<T, K>(ad, cd[t], m);
            for (int t = 0; t < nth; ++t) wtc_whole_conv<T, K, BW, false>(ad, cd[t]);
            for (int t = 0; t < nth; ++t) wtc_whole_out<T, K, BW, false, false, 2, DL>(ad, cd[t]);
            poison_maps();
            for (int t = 0; t < nth; ++t) wtc_whole_stage<T, K, BW, true, false>(at, ct[t]);
            for (int t = 0; t < nth; ++t)
                if (tiles > 1) wtc_whole_load<T, K, BW, true, false>(at, ct[t], u0 + 1);
            for (int tt = 0; tt < tiles; ++tt) {
                for (int t = 0; t < nth; ++t) wtc_whole_conv<T, K, BW, false, HALF>(at, ct[t]);
                for (int t = 0; t < nth; ++t) {
                    if (tt + 1 < tiles) wtc_whole_stage<T, K, BW, true, false>(at, ct[t]);
                    if (tt + 2 < tiles) wtc_whole_load<T, K, BW, true, false>(at, ct[t], u0 + tt + 2);
                }
                for (int t = 0; t < nth; ++t) {
                    wtc_whole_select<T, false>(at, ct[t], u0 + tt);
                    wtc_whole_out<T, K, BW, true, false, 1, 1>(at, ct[t]);
                }
            }
            poison_maps();
        }
    }
}

template <typename T, int K>
static int run_large_k(const WtcLargeArgs<T> &a)
{
    if constexpr (sizeof(T) == 4 && K == 5) {
        if (a.t.p.halves) {
            switch (a.d.p.levels) {
            case 1: run_large<T, K, 4, 1, true>(a); return 0;
            case 2: run_large<T, K, 4, 2, true>(a); return 0;
            case 3: run_large<T, K, 4, 3, true>(a); return 0;
            default: run_large<T, K, 4, 0, true>(a); return 0;
            }
        }
    }
    switch (a.d.p.levels) {
    case 1: run_large<T, K, 4, 1>(a); return 0;
    case 2: run_large<T, K, 4, 2>(a); return 0;
    case 3: run_large<T, K, 4, 3>(a); return 0;
    default: run_large<T, K, 4, 0>(a); return 0;
    }
}

template <typename T>
static int run_large_t(const WtcLargeArgs<T> &a)
{
    switch (a.t.p.k) {
    case 1: return run_large_k<T, 1>(a);
    case 3: return run_large_k<T, 3>(a);
    case 5: return run_large_k<T, 5>(a);
    case 7: return run_large_k<T, 7>(a);
    default: return -1;
    }
}

// The fused single-pass backward, phase by phase (the data plan's lane-quad
// exchange for Haar level 3 after every thread has staged).
template <typename T, int K, int Q>
static void run_bwd(const WtcBwdArgs<T> &A, float *partial)
{
    const WtcWholeArgs<T> &ad = A.d;
    WtcWgradArgs<T> ag = A.g;
    ag.partial = partial;
    const int nblocks = ag.p.groups * ag.p.c;
    std::vector<float> lds((size_t)A.lds_floats);
    const int nth = ad.p.nthreads;
    for (int bid = 0; bid < nblocks; ++bid) {
        for (auto &v : lds) v = __builtin_nanf("");
        std::vector<WtcWholeCtx<T>> cw((size_t)nth);
        std::vector<WtcWgradCtx<T, 4>> cg((size_t)nth);
        std::vector<std::array<std::array<float, K * K + 1>, Q>> acc((size_t)nth);
        for (int t = 0; t < nth; ++t) {
            cw[t].lds = cg[t].lds = lds.data();
            cw[t].tid = cg[t].tid = t;
            cw[t].nth = cg[t].nth = nth;
            cw[t].lds_n = cg[t].lds_n = A.lds_floats;
            cw[t].img_n = (int64_t)ad.p.h * ad.p.w;
            wtc_whole_setup<T>(ad, cw[t], bid);
            wtc_wgrad_setup<T, 4>(ag, cg[t], bid);
            cg[t].grow = cw[t].grow;
            cg[t].gcol = cw[t].gcol;
            cg[t].gvalid = cw[t].gvalid;
            for (auto &a1 : acc[(size_t)t])
                for (auto &v : a1) v = 0.0f;
        }
        for (int t = 0; t < nth; ++t) wtc_wgrad_load<T, 4, false>(ag, cg[t], 0);
        for (int i = 0; i < A.lds_floats; ++i) lds[(size_t)i] = 0.0f;
        for (int t = 0; t < nth; ++t) {
            wtc_whole_fold<T, K>(ad, cw[t]);
            wtc_whole_table<T, K, 4>(ad, cw[t]);
            wtc_wgrad_table<T, K, 4>(ag, cg[t]);
        }
        auto stage = [&]() {
            for (int t = 0; t < nth; ++t) {
                wtc_wgrad_stage<T, K, 4, false>(ag, cg[t]);
                wtc_bwd_stage_dy<T, K, 4>(ad, cw[t], cg[t]);
            }
            if (ad.p.stage_l3) emu_stage_l3(ad, cw);
        };
        stage();
        for (int t = 0; t < nth; ++t)
            if (cw[t].nimg > 1) wtc_wgrad_load<T, 4, false>(ag, cg[t], 1);
        for (int img = 0; img < cw[0].nimg; ++img) {
            for (int m = ag.p.first_deep; m <= ag.p.levels; ++m)
                for (int t = 0; t < nth; ++t) wtc_wgrad_analysis<T, K, 4>(ag, cg[t], m);
            for (int m = wtc_whole_first_deep(ad.p); m <= ad.p.levels; ++m)
                for (int t = 0; t < nth; ++t) wtc_whole_analysis<T, K>(ad, cw[t], m);
            for (int t = 0; t < nth; ++t) {
                float a2[Q][K * K + 1];
                for (int q = 0; q < Q; ++q)
                    for (int e = 0; e < K * K + 1; ++e) a2[q][e] = acc[(size_t)t][(size_t)q][(size_t)e];
                wtc_wgrad_correlate<T, K, 4, Q>(ag, cg[t], a2);
                for (int q = 0; q < Q; ++q)
                    for (int e = 0; e < K * K + 1; ++e) acc[(size_t)t][(size_t)q][(size_t)e] = a2[q][e];
            }
            for (int t = 0; t < nth; ++t) wtc_whole_conv<T, K, 4>(ad, cw[t]);
            if (img + 1 < cw[0].nimg) stage();
            for (int t = 0; t < nth; ++t)
                if (img + 2 < cw[t].nimg) wtc_wgrad_load<T, 4, false>(ag, cg[t], img + 2);
            for (int t = 0; t < nth; ++t) {
                wtc_whole_select<T, false>(ad, cw[t], img);
                wtc_whole_out<T, K, 4, false, false>(ad, cw[t]);
            }
        }
        for (int q = 0; q < Q; ++q) {
            if (q >= ag.p.q) continue;
            for (int t = 0; t < nth; ++t) {
                float a1[K * K + 1];
                for (int e = 0; e < K * K + 1; ++e) a1[e] = acc[(size_t)t][(size_t)q][(size_t)e];
                wtc_wgrad_park<T, K, 4>(ag, cg[t], a1);
            }
            for (int t = 0; t < nth; ++t) wtc_wgrad_chunks<T, K, 4>(ag, cg[t], q);
            for (int t = 0; t < nth; ++t) wtc_wgrad_combine<T, K, 4>(ag, cg[t], q);
        }
        for (int t = 0; t < nth; ++t) wtc_wgrad_write<T, K, 4>(ag, cg[t]);
    }
}

template <typename T, int K>
static void run_bwd_k(const WtcBwdArgs<T> &a, float *partial)
{
    if (a.g.p.q == 1)
        run_bwd<T, K, 1>(a, partial);
    else
        run_bwd<T, K, WTC_WG_QMAX>(a, partial);
}

template <typename T, int K, int VEC, bool TL = false>
static void run_wgrad(const WtcWgradArgs<T> &a)
{
    const WtcWgradPlan &p = a.p;
    const int nblocks = p.groups * p.c;
    std::vector<float> lds((size_t)p.lds_floats);
    const int nth = p.nthreads;
    for (int bid = 0; bid < nblocks; ++bid) {
        for (auto &v : lds) v = __builtin_nanf("");
        std::vector<WtcWgradCtx<T, VEC>> ctx((size_t)nth);
        std::vector<float> acc((size_t)nth * WTC_WG_QMAX * (K * K + 1), 0.0f);
        auto A = [&](int t) -> float(&)[WTC_WG_QMAX][K * K + 1] {
            return *reinterpret_cast<float(*)[WTC_WG_QMAX][K * K + 1]>(&acc[(size_t)t * WTC_WG_QMAX * (K * K + 1)]);
        };
        for (int t = 0; t < nth; ++t) {
            ctx[t].lds = lds.data();
            ctx[t].tid = t;
            ctx[t].nth = nth;
            ctx[t].lds_n = p.lds_floats;
            wtc_wgrad_setup<T, VEC>(a, ctx[t], bid);
        }
        for (int t = 0; t < nth; ++t) wtc_wgrad_load<T, VEC, TL>(a, ctx[t], 0);
        for (int t = 0; t < nth; ++t) wtc_wgrad_zero<T, VEC>(a, ctx[t]);
        for (int t = 0; t < nth; ++t) wtc_wgrad_table<T, K, VEC>(a, ctx[t]);
        for (int img = 0; img < ctx[0].nimg; ++img) {
            for (int t = 0; t < nth; ++t) wtc_wgrad_stage<T, K, VEC, TL>(a, ctx[t]);
            for (int t = 0; t < nth; ++t)
                if (img + 1 < ctx[t].nimg) wtc_wgrad_load<T, VEC, TL>(a, ctx[t], img + 1);
            for (int m = p.first_deep; m <= p.levels; ++m)
                for (int t = 0; t < nth; ++t) wtc_wgrad_analysis<T, K, VEC>(a, ctx[t], m);
            for (int t = 0; t < nth; ++t) wtc_wgrad_correlate<T, K, VEC, WTC_WG_QMAX>(a, ctx[t], A(t));
        }
        for (int s = 0; s < p.q; ++s) {
            for (int t = 0; t < nth; ++t) wtc_wgrad_park<T, K, VEC>(a, ctx[t], A(t)[s]);
            for (int t = 0; t < nth; ++t) wtc_wgrad_chunks<T, K, VEC>(a, ctx[t], s);
            for (int t = 0; t < nth; ++t) wtc_wgrad_combine<T, K, VEC>(a, ctx[t], s);
        }
        for (int t = 0; t < nth; ++t) wtc_wgrad_write<T, K, VEC>(a, ctx[t]);
    }
}

template <typename T, int K>
static void run_wgrad_k(const WtcWgradArgs<T> &a)
{
    switch (a.p.vec) {
    case 4:
        if (a.p.tiled)
            run_wgrad<T, K, 4, true>(a);
        else
            run_wgrad<T, K, 4>(a);
        break;
    case 2: run_wgrad<T, K, 2>(a); break;
    default: run_wgrad<T, K, 1>(a); break;
    }
}

template <typename T>
static int run_wgrad_t(const WtcWgradArgs<T> &a)
{
    switch (a.p.k) {
    case 1: run_wgrad_k<T, 1>(a); return 0;
    case 3: run_wgrad_k<T, 3>(a); return 0;
    case 5: run_wgrad_k<T, 5>(a); return 0;
    case 7: run_wgrad_k<T, 7>(a); return 0;
    default: return -1;
    }
}

template <typename TI, int K>
static void run_wtile(const WtcWtileArgs<TI> &a)
{
    const WtcWtilePlan &p = a.p;
    const int nblocks = p.groups * p.c;
    std::vector<float> lds((size_t)p.lds_floats);
    const int nth = p.nthreads;
    const int units = p.n * p.tiles_y * p.tiles_x;
    for (int bid = 0; bid < nblocks; ++bid) {
        for (auto &v : lds) v = __builtin_nanf("");
        std::vector<WtcWtileCtx> ctx((size_t)nth);
        std::vector<float> acc((size_t)nth * WTC_WT_QMAX * (K * K + 1), 0.0f);
        auto A = [&](int t) -> float(&)[WTC_WT_QMAX][K * K + 1] {
            return *reinterpret_cast<float(*)[WTC_WT_QMAX][K * K + 1]>(&acc[(size_t)t * WTC_WT_QMAX * (K * K + 1)]);
        };
        for (int t = 0; t < nth; ++t) {
            ctx[t].lds = lds.data();
            ctx[t].tid = t;
            ctx[t].nth = nth;
            ctx[t].lds_n = p.lds_floats;
            ctx[t].c = bid % p.c;
            ctx[t].group = bid / p.c;
        }
        const int u0 = ctx[0].group * p.units_per_wg, u1 = std::min(units, u0 + p.units_per_wg);
        for (int t = 0; t < nth; ++t) wtc_wtile_zero<TI>(a, ctx[t]);
        for (int t = 0; t < nth; ++t) wtc_wtile_table<TI, K>(a, ctx[t]);
        for (int u = u0; u < u1; ++u) {
            for (int t = 0; t < nth; ++t) wtc_wtile_stage<TI, K>(a, ctx[t], u);
            if (p.step < p.levels)
                for (int t = 0; t < nth; ++t) wtc_wtile_analysis<TI, K>(a, ctx[t], u);
            for (int t = 0; t < nth; ++t) wtc_wtile_correlate<TI, K>(a, ctx[t], A(t));
        }
        for (int s = 0; s < p.q; ++s) {
            for (int t = 0; t < nth; ++t) wtc_wtile_park<TI, K>(a, ctx[t], A(t)[s]);
            for (int t = 0; t < nth; ++t) wtc_wtile_gather<TI, K>(a, ctx[t], s);
        }
        for (int t = 0; t < nth; ++t) wtc_wtile_write<TI, K>(a, ctx[t]);
    }
}

template <typename TI>
static int run_wtile_t(const WtcWtileArgs<TI> &a)
{
    switch (a.p.k) {
    case 1: run_wtile<TI, 1>(a); return 0;
    case 3: run_wtile<TI, 3>(a); return 0;
    case 5: run_wtile<TI, 5>(a); return 0;
    case 7: run_wtile<TI, 7>(a); return 0;
    default: return -1;
    }
}

extern "C" {

// Parameter gradients through the level-by-level tiled steps and the finalize.
int emu_wgrad_tiled(int dtype, const void *x, const void *dy, int n, int c, int h, int w, int k, int levels,
                    const float *w_base, const float *bias, const float *s_base, const float *w_lvl,
                    const float *s_lvl, float *dw_base, float *dbias, float *ds_base, float *dw_lvl, float *ds_lvl,
                    int nthreads, int groups, int budget_floats)
{
    const int kk = k * k, plen = kk + 1 + 4 * levels * kk;
    // one workspace carved exactly as the library carves it; NaN-filled so a
    // read of something no step wrote shows up
    WtcWtileCarve cv;
    wtc_wtile_carve(&cv, n, c, h, w, levels, groups, plen);
    std::vector<float> wsbuf(cv.total / sizeof(float) + 64, __builtin_nanf(""));
    char *ws = (char *)wsbuf.data();
    float *partialp = (float *)ws;
    const void *curx = x, *curd = dy;
    int curdt = dtype;
    for (int j = 0; j <= levels; ++j) {
        WtcWtilePlan p;
        if (wtc_make_wtile_plan(&p, n, c, k, levels, j, h >> j, w >> j, nthreads, groups, budget_floats)) return -1;
        float *ux = nullptr, *ud = nullptr;
        if (j < levels) {
            ux = (float *)(ws + cv.off_ux[j % 2]);
            ud = (float *)(ws + cv.off_ud[j % 2]);
        }
        int rc;
        if (curdt == 0) {
            WtcWtileArgs<float> a{(const float *)curx, (const float *)curd, ux, ud, partialp, p};
            rc = run_wtile_t<float>(a);
        } else {
            WtcWtileArgs<_Float16> a{(const _Float16 *)curx, (const _Float16 *)curd, ux, ud, partialp, p};
            rc = run_wtile_t<_Float16>(a);
        }
        if (rc) return rc;
        curx = ux;
        curd = ud;
        curdt = 0;
    }
    for (int cc = 0; cc < c; ++cc)
        for (int g = 0; g < 1 + 4 * levels; ++g)
            wtc_wgrad_finalize_one(cc, g, c, k, levels, groups, plen, partialp, w_base, bias, s_base, w_lvl,
                                   s_lvl, dw_base, dbias, ds_base, dw_lvl, ds_lvl);
    return 0;
}

// Parameter gradients through the fused weight-gradient phases and the
// fixed-order finalize.  Outputs overwritten, fp32.  nobase: the base
// gradients are skipped (written as 0), as in the nested call for deeper levels.
int emu_wgrad(int dtype, const void *x, const void *dy, int n, int c, int h, int w, int k, int levels,
              const float *w_base, const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
              float *dw_base, float *dbias, float *ds_base, float *dw_lvl, float *ds_lvl, int nthreads, int planes,
              int budget_floats, int nobase)
{
    WtcWgradPlan p;
    if (wtc_make_wgrad_plan(&p, n, c, h, w, k, levels, nthreads, planes, dtype == 0 ? 4 : 2, budget_floats, nobase))
        return -1;
    std::vector<float> partial((size_t)p.groups * p.c * p.plen, __builtin_nanf(""));
    int rc;
    if (dtype == 0) {
        WtcWgradArgs<float> a{(const float *)x, (const float *)dy, partial.data(), p};
        rc = run_wgrad_t<float>(a);
    } else {
        WtcWgradArgs<_Float16> a{(const _Float16 *)x, (const _Float16 *)dy, partial.data(), p};
        rc = run_wgrad_t<_Float16>(a);
    }
    if (rc) return rc;
    for (int cc = 0; cc < c; ++cc)
        for (int g = 0; g < 1 + 4 * levels; ++g)
            wtc_wgrad_finalize_one(cc, g, c, k, levels, p.groups, p.plen, partial.data(), w_base, bias, s_base,
                                   w_lvl, s_lvl, dw_base, dbias, ds_base, dw_lvl, ds_lvl);
    return 0;
}

// The tiled weight-gradient pass (base and level-1 correlations on th x tw
// tiles of ih x iw images, L = 1) on host arrays, with its finalize; llx and
// lld (both or neither) receive the level-1 low-pass maps of x and dy.
int emu_wgrad_tiles(int dtype, const void *x, const void *dy, int n, int c, int ih, int iw, int th, int tw, int k,
                    int levels, const float *w_base, const float *bias, const float *s_base, const float *w_lvl,
                    const float *s_lvl, float *dw_base, float *dbias, float *ds_base, float *dw_lvl, float *ds_lvl,
                    void *llx, void *lld, int nthreads, int planes, int budget_floats, int nobase)
{
    WtcWgradPlan p;
    if (wtc_make_wgrad_tile_plan(&p, n, c, ih, iw, th, tw, k, levels, nthreads, planes, dtype == 0 ? 4 : 2,
                                 budget_floats, nobase))
        return -1;
    std::vector<float> partial((size_t)p.groups * p.c * p.plen, __builtin_nanf(""));
    int rc;
    if (dtype == 0) {
        WtcWgradArgs<float> a{(const float *)x, (const float *)dy, partial.data(), p, (float *)llx, (float *)lld};
        rc = run_wgrad_t<float>(a);
    } else {
        WtcWgradArgs<_Float16> a{(const _Float16 *)x, (const _Float16 *)dy, partial.data(), p, (float *)llx,
                                 (float *)lld};
        rc = run_wgrad_t<_Float16>(a);
    }
    if (rc) return rc;
    for (int cc = 0; cc < c; ++cc)
        for (int g = 0; g < 1 + 4 * levels; ++g)
            wtc_wgrad_finalize_one(cc, g, c, k, levels, p.groups, p.plen, partial.data(), w_base, bias, s_base, w_lvl,
                                   s_lvl, dw_base, dbias, ds_base, dw_lvl, ds_lvl);
    return 0;
}

int emu_wgrad_plan(int n, int c, int h, int w, int k, int levels, int nthreads, int planes, int ebytes,
                   int budget_floats, int *out)
{
    WtcWgradPlan p;
    int rc = wtc_make_wgrad_plan(&p, n, c, h, w, k, levels, nthreads, planes, ebytes, budget_floats);
    out[0] = p.lds_floats;
    out[1] = p.npieces;
    out[2] = p.q;
    out[3] = p.groups;
    out[4] = p.plen;
    out[5] = p.vec;
    out[6] = p.tail;
    return rc;
}

// Images per workgroup chosen for a grid of c x ceil(n / planes) workgroups.
int emu_choose_planes(int n, int c, int slots, double fixed) { return wtc_choose_planes(n, c, slots, fixed); }

// Whole-plane plan: out[0..11] = planes, vec, out_bw, lds_floats, pieces, nthreads, ok, stage_l3, plane rows,
// rows between stacked images, units, pieces run as one-row pieces.
int emu_whole_plan(int n, int c, int h, int w, int k, int levels, int rotate, int nthreads, int planes, int ebytes,
                   int budget_floats, int stack, int *out)
{
    WtcWholePlan p;
    int rc = wtc_make_whole_plan(&p, n, c, h, w, k, levels, rotate, nthreads, planes, ebytes, budget_floats, 0, stack);
    out[0] = p.planes;
    out[1] = p.vec;
    out[2] = p.out_bw;
    out[3] = p.lds_floats;
    out[4] = p.items;
    out[5] = p.nthreads;
    out[6] = rc == 0;
    out[7] = p.stage_l3;
    out[8] = p.h;
    out[9] = p.sgap;
    out[10] = p.units;
    out[11] = p.tail;
    return rc;
}

int emu_whole(int dtype, const void *in, void *out, int n, int c, int h, int w, int k, int levels, int rotate,
              const float *w_base, const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
              int nthreads, int planes, int budget_floats, int nobase, int stack)
{
    WtcWholePlan p;
    if (wtc_make_whole_plan(&p, n, c, h, w, k, levels, rotate, nthreads, planes, dtype == 0 ? 4 : 2,
                            budget_floats, nobase, stack))
        return -1;
    if (dtype == 0) {
        WtcWholeArgs<float> a{(const float *)in, (float *)out, w_base, bias, s_base, w_lvl, s_lvl, p};
        return run_whole_t<float>(a);
    }
    WtcWholeArgs<_Float16> a{(const _Float16 *)in, (_Float16 *)out, w_base, bias, s_base, w_lvl, s_lvl, p};
    return run_whole_t<_Float16>(a);
}

// The tiled whole-plane pass (L = 1 plus the deeper levels' low-pass term
// `low`, (N, C, ih/2, iw/2), or null) on host arrays.  nobase: without the
// base path (both entry points; w_base, bias and s_base may then be null).
int emu_whole_tiled(int dtype, const void *in, void *out, const void *low, int n, int c, int ih, int iw, int th,
                    int tw, int k, int levels, int rotate, const float *w_base, const float *bias, const float *s_base,
                    const float *w_lvl, const float *s_lvl, int nthreads, int planes, int budget_floats, int nobase)
{
    WtcWholePlan p;
    if (wtc_make_whole_tile_plan(&p, n, c, ih, iw, th, tw, k, levels, rotate, nthreads, planes, dtype == 0 ? 4 : 2,
                                 budget_floats, nobase))
        return -1;
    if (dtype == 0) {
        WtcWholeArgs<float> a{(const float *)in, (float *)out, w_base, bias, s_base, w_lvl, s_lvl, p,
                              (const float *)low};
        return run_whole_t<float>(a);
    }
    WtcWholeArgs<_Float16> a{(const _Float16 *)in, (_Float16 *)out, w_base, bias, s_base, w_lvl, s_lvl, p,
                             (const float *)low};
    return run_whole_t<_Float16>(a);
}

// Plan of a fused launch, for inspection by the tests: fills out[0..7] with
// tile_h, tile_w, strip_h, out_bw, tiles_y, tiles_x, lds_floats, nthreads.
int emu_fused_plan(int n, int c, int h, int w, int k, int levels, int rotate, int nthreads, int budget_floats,
                   int *out)
{
    WtcFusedPlan p;
    if (wtc_make_fused_plan(&p, n, c, h, w, k, levels, rotate, nthreads, budget_floats)) return -1;
    out[0] = p.tile_h;
    out[1] = p.tile_w;
    out[2] = p.strip_h;
    out[3] = p.out_bw;
    out[4] = p.tiles_y;
    out[5] = p.tiles_x;
    out[6] = p.lds_floats;
    out[7] = p.nthreads;
    return 0;
}

// The fused pass on host arrays.  dtype 0: float in/out, 1: _Float16 in/out.
int emu_fused(int dtype, const void *in, void *out, int n, int c, int h, int w, int k, int levels, int rotate,
              const float *w_base, const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
              int nthreads, int budget_floats)
{
    WtcFusedPlan p;
    if (wtc_make_fused_plan(&p, n, c, h, w, k, levels, rotate, nthreads, budget_floats)) return -1;
    if (dtype == 0) {
        WtcFusedArgs<float> a{(const float *)in, (float *)out, w_base, bias, s_base, w_lvl, s_lvl, p};
        return run_t<float>(a);
    }
    WtcFusedArgs<_Float16> a{(const _Float16 *)in, (_Float16 *)out, w_base, bias, s_base, w_lvl, s_lvl, p};
    return run_t<_Float16>(a);
}

// The fused large-plane pass (every level on chip) on host arrays: th x tw
// tiles, nobase: without the base path; out[0..3] of `info` = images per
// workgroup, LDS floats, deeper-levels plan's LDS-map floats, tiles per image
// (info may be null).
int emu_large(int dtype, const void *in, void *out, int n, int c, int h, int w, int th, int tw, int k, int levels,
              int rotate, const float *w_base, const float *bias, const float *s_base, const float *w_lvl,
              const float *s_lvl, int planes, int budget_floats, int nobase, int *info)
{
    WtcLargePlan p;
    if (wtc_make_large_plan(&p, n, c, h, w, th, tw, k, levels, rotate, 256, planes, dtype == 0 ? 4 : 2,
                            budget_floats, nobase))
        return -1;
    if (info) {
        info[0] = p.planes;
        info[1] = p.lds_floats;
        info[2] = p.dmaps_floats;
        info[3] = p.t.tiles_x * p.t.tiles_y;
        info[4] = p.d.items;
        info[5] = p.d.tail;
        info[6] = p.t.items;
        info[7] = p.t.tail;
        info[8] = p.t.halves;
    }
    if (!in) return 0;
    if (dtype == 0)
        return run_large_t<float>(
            wtc_large_args<float>(p, (const float *)in, (float *)out, w_base, bias, s_base, w_lvl, s_lvl));
    return run_large_t<_Float16>(
        wtc_large_args<_Float16>(p, (const _Float16 *)in, (_Float16 *)out, w_base, bias, s_base, w_lvl, s_lvl));
}

// The fused single-pass backward on host arrays: dx and the five gradients
// (through the weight backward's finalize).  Returns -1 where the plan does
// not apply.
int emu_bwd(int dtype, const void *x, const void *dy, void *dx, int n, int c, int h, int w, int k, int levels,
            const float *w_base, const float *bias, const float *s_base, const float *w_lvl, const float *s_lvl,
            float *dw_base, float *dbias, float *ds_base, float *dw_lvl, float *ds_lvl, int nthreads, int planes,
            int budget_floats)
{
    WtcBwdPlan p;
    if (wtc_make_bwd_plan(&p, n, c, h, w, k, levels, nthreads, planes, dtype == 0 ? 4 : 2, budget_floats)) return -1;
    std::vector<float> partial((size_t)p.g.groups * c * p.g.plen, __builtin_nanf(""));
    auto run = [&](auto tag) {
        using T = decltype(tag);
        const WtcBwdArgs<T> a = wtc_bwd_args<T>(p, (const T *)x, (const T *)dy, (T *)dx, w_base, s_base, w_lvl,
                                                s_lvl, partial.data());
        switch (k) {
        case 1: run_bwd_k<T, 1>(a, partial.data()); break;
        case 3: run_bwd_k<T, 3>(a, partial.data()); break;
        case 5: run_bwd_k<T, 5>(a, partial.data()); break;
        default: run_bwd_k<T, 7>(a, partial.data()); break;
        }
    };
    if (dtype == 0)
        run(float{});
    else
        run(_Float16{});
    for (int cc = 0; cc < c; ++cc)
        for (int g = 0; g < 1 + 4 * levels; ++g)
            wtc_wgrad_finalize_one(cc, g, c, k, levels, p.g.groups, p.g.plen, partial.data(), w_base, bias, s_base,
                                   w_lvl, s_lvl, dw_base, dbias, ds_base, dw_lvl, ds_lvl);
    return 0;
}

}  // extern "C"
