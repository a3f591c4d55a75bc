// sanitize_main.cpp -- the CPU emulation of the kernels and the oracle, built
// together with AddressSanitizer and UndefinedBehaviorSanitizer (test tool):
// runs the whole-plane, strip, large-plane, weight-gradient and fused
// backward emulations on small cases and compares each with the oracle.
// Exit status 0 when every case is within its tolerance and the sanitizers
// report nothing (they abort on the first error).
#include "wtconv_emu.cpp"

#include <cmath>
#include <cstdio>
#include <vector>

extern "C" {
int oracle_wtconv_forward(int64_t n, int64_t c, int64_t h, int64_t w, int k, int levels, const double *x,
                          const double *w_base, const double *bias, const double *s_base, const double *w_lvl,
                          const double *s_lvl, double *y, int nthreads);
int oracle_wtconv_backward_data(int64_t n, int64_t c, int64_t h, int64_t w, int k, int levels, const double *dy,
                                const double *w_base, const double *s_base, const double *w_lvl,
                                const double *s_lvl, double *dx, int nthreads);
int oracle_wtconv_backward_weight(int64_t n, int64_t c, int64_t h, int64_t w, int k, int levels, const double *x,
                                  const double *dy, const double *w_base, const double *bias, const double *s_base,
                                  const double *w_lvl, const double *s_lvl, double *dw_base, double *dbias,
                                  double *ds_base, double *dw_lvl, double *ds_lvl, int nthreads);
}

namespace {

// Test inputs: multiples of 1/64 in [-2, 2) from a 64-bit xorshift (exact in
// fp16 and fp32), and small weights.
struct Gen {
    uint64_t s;
    double next(double scale)
    {
        s ^= s << 13;
        s ^= s >> 7;
        s ^= s << 17;
        return scale * ((double)(int64_t)(s % 256) - 128.0) / 64.0;
    }
};

struct Case {
    int n, c, h, w, k, L;
    std::vector<float> x, dy, w0, b0, s0, wl, sl;
    Case(int n_, int c_, int h_, int w_, int k_, int L_, uint64_t seed) : n(n_), c(c_), h(h_), w(w_), k(k_), L(L_)
    {
        Gen g{seed * 2654435761u + 1};
        const size_t e = (size_t)n * c * h * w, kk = (size_t)k * k;
        x.resize(e);
        dy.resize(e);
        for (auto &v : x) v = (float)g.next(1.0);
        for (auto &v : dy) v = (float)g.next(1.0);
        w0.resize(c * kk);
        b0.resize(c);
        s0.resize(c);
        wl.resize((size_t)(L > 0 ? L : 1) * 4 * c * kk);
        sl.resize((size_t)(L > 0 ? L : 1) * 4 * c);
        for (auto &v : w0) v = (float)g.next(0.05);
        for (auto &v : b0) v = (float)g.next(0.01);
        for (auto &v : s0) v = 1.0f + (float)g.next(0.01);
        for (auto &v : wl) v = (float)g.next(0.05);
        for (auto &v : sl) v = 0.1f + (float)g.next(0.01);
    }
    size_t elems() const { return (size_t)n * c * h * w; }
};

std::vector<double> wide(const std::vector<float> &v) { return std::vector<double>(v.begin(), v.end()); }

std::vector<_Float16> half(const std::vector<float> &v)
{
    std::vector<_Float16> o(v.size());
    for (size_t i = 0; i < v.size(); ++i) o[i] = (_Float16)v[i];
    return o;
}

int failures = 0;

void check_elem(const char *what, const std::vector<double> &got, const std::vector<double> &ref, double tol)
{
    double worst = 0.0;
    for (size_t i = 0; i < ref.size(); ++i) {
        const double e = std::fabs(got[i] - ref[i]) / (1.0 + std::fabs(ref[i]));
        if (!(e <= worst)) worst = e;  // NaN propagates
    }
    const bool ok = worst <= tol;
    std::printf("%-44s max scaled err %.3e %s\n", what, worst, ok ? "ok" : "FAIL");
    failures += !ok;
}

void check_l2(const char *what, const std::vector<float> &got, const std::vector<double> &ref, double tol)
{
    double num = 0.0, den = 0.0;
    for (size_t i = 0; i < ref.size(); ++i) {
        num += (got[i] - ref[i]) * (got[i] - ref[i]);
        den += ref[i] * ref[i];
    }
    const double rel = std::sqrt(num / (den > 0 ? den : 1e-300));
    const bool ok = rel <= tol;
    std::printf("%-44s rel L2 %.3e %s\n", what, rel, ok ? "ok" : "FAIL");
    failures += !ok;
}

std::vector<double> ref_forward(const Case &t)
{
    std::vector<double> y(t.elems());
    oracle_wtconv_forward(t.n, t.c, t.h, t.w, t.k, t.L, wide(t.x).data(), wide(t.w0).data(), wide(t.b0).data(),
                          wide(t.s0).data(), wide(t.wl).data(), wide(t.sl).data(), y.data(), 1);
    return y;
}

std::vector<double> ref_backward_data(const Case &t)
{
    std::vector<double> dx(t.elems());
    oracle_wtconv_backward_data(t.n, t.c, t.h, t.w, t.k, t.L, wide(t.dy).data(), wide(t.w0).data(),
                                wide(t.s0).data(), wide(t.wl).data(), wide(t.sl).data(), dx.data(), 1);
    return dx;
}

void ref_grads(const Case &t, std::vector<double> (&g)[5])
{
    const size_t kk = (size_t)t.k * t.k;
    g[0].resize(t.c * kk);
    g[1].resize(t.c);
    g[2].resize(t.c);
    g[3].resize((size_t)t.L * 4 * t.c * kk);
    g[4].resize((size_t)t.L * 4 * t.c);
    oracle_wtconv_backward_weight(t.n, t.c, t.h, t.w, t.k, t.L, wide(t.x).data(), wide(t.dy).data(),
                                  wide(t.w0).data(), wide(t.b0).data(), wide(t.s0).data(), wide(t.wl).data(),
                                  wide(t.sl).data(), g[0].data(), g[1].data(), g[2].data(), g[3].data(),
                                  g[4].data(), 1);
}

template <typename O>
std::vector<double> widen(const std::vector<O> &v)
{
    std::vector<double> o(v.size());
    for (size_t i = 0; i < v.size(); ++i) o[i] = (double)v[i];
    return o;
}

}  // namespace

int main()
{
    const double f16tol = 4.0 / 2048.0;
    {  // whole-plane forward, fp32
        Case t(2, 3, 16, 16, 5, 2, 1);
        std::vector<float> y(t.elems());
        emu_whole(0, t.x.data(), y.data(), t.n, t.c, t.h, t.w, t.k, t.L, 0, t.w0.data(), t.b0.data(), t.s0.data(),
                  t.wl.data(), t.sl.data(), 256, 2, 40960, 0, 1);
        check_elem("whole-plane forward fp32 2x3x16x16 L=2", widen(y), ref_forward(t), 1e-4);
    }
    {  // whole-plane data backward, fp16, stacked images
        Case t(3, 2, 28, 28, 5, 2, 2);
        auto dyh = half(t.dy);
        std::vector<_Float16> dx(t.elems());
        emu_whole(1, dyh.data(), dx.data(), t.n, t.c, t.h, t.w, t.k, t.L, 1, t.w0.data(), nullptr, t.s0.data(),
                  t.wl.data(), t.sl.data(), 256, 2, 40960, 0, 2);
        check_elem("whole-plane data backward fp16 3x2x28x28", widen(dx), ref_backward_data(t), f16tol);
    }
    {  // strip fallback, small LDS budget
        Case t(1, 1, 64, 96, 3, 3, 3);
        std::vector<float> y(t.elems());
        emu_fused(0, t.x.data(), y.data(), t.n, t.c, t.h, t.w, t.k, t.L, 0, t.w0.data(), t.b0.data(), t.s0.data(),
                  t.wl.data(), t.sl.data(), 256, 4000);
        check_elem("strip forward fp32 1x1x64x96 L=3", widen(y), ref_forward(t), 1e-4);
    }
    {  // fused large-plane forward, every level on chip
        Case t(3, 1, 64, 64, 5, 3, 4);
        std::vector<float> y(t.elems());
        emu_large(0, t.x.data(), y.data(), t.n, t.c, t.h, t.w, 32, 64, t.k, t.L, 0, t.w0.data(), t.b0.data(),
                  t.s0.data(), t.wl.data(), t.sl.data(), 2, 40960, 0, nullptr);
        check_elem("large-plane forward fp32 3x1x64x64 L=3", widen(y), ref_forward(t), 1e-4);
    }
    {  // weight gradients
        Case t(2, 2, 24, 40, 3, 3, 5);
        std::vector<float> g[5] = {std::vector<float>(t.w0.size()), std::vector<float>(t.c),
                                   std::vector<float>(t.c), std::vector<float>(t.wl.size()),
                                   std::vector<float>(t.sl.size())};
        emu_wgrad(0, t.x.data(), t.dy.data(), t.n, t.c, t.h, t.w, t.k, t.L, t.w0.data(), t.b0.data(), t.s0.data(),
                  t.wl.data(), t.sl.data(), g[0].data(), g[1].data(), g[2].data(), g[3].data(), g[4].data(), 256, 2,
                  40960, 0);
        std::vector<double> r[5];
        ref_grads(t, r);
        const char *names[5] = {"weight backward dw_base", "weight backward dbias", "weight backward ds_base",
                                "weight backward dw_lvl", "weight backward ds_lvl"};
        for (int i = 0; i < 5; ++i) check_l2(names[i], g[i], r[i], 1e-4);
    }
    {  // fused single-pass backward
        Case t(3, 2, 16, 16, 5, 2, 6);
        std::vector<float> dx(t.elems());
        std::vector<float> g[5] = {std::vector<float>(t.w0.size()), std::vector<float>(t.c),
                                   std::vector<float>(t.c), std::vector<float>(t.wl.size()),
                                   std::vector<float>(t.sl.size())};
        emu_bwd(0, t.x.data(), t.dy.data(), dx.data(), t.n, t.c, t.h, t.w, t.k, t.L, t.w0.data(), t.b0.data(),
                t.s0.data(), t.wl.data(), t.sl.data(), g[0].data(), g[1].data(), g[2].data(), g[3].data(),
                g[4].data(), 256, 2, 40960);
        check_elem("fused backward dx fp32 3x2x16x16 L=2", widen(dx), ref_backward_data(t), 1e-4);
        std::vector<double> r[5];
        ref_grads(t, r);
        for (int i = 0; i < 5; ++i) check_l2("fused backward gradient", g[i], r[i], 1e-4);
    }
    std::printf("%s\n", failures ? "FAILED" : "all cases ok");
    return failures ? 1 : 0;
}
