// Accuracy of the tree-construction kernel's table exponentials (exp_tab.h,
// the same source the kernel compiles), on the CPU against the C library's
// exp. The table is filled with the C library's exp2, as the kernel fills it
// with the device library's. exp_tab over its whole range: the largest error
// in ulps of the result (normal results) and in subnormal steps (subnormal
// results). exp_tab_nonpos over x <= 0, with its own table (exp_tab_adjust): the
// largest relative error for -40 <= x <= 0 and for -700 <= x < -40, and its special
// inputs (NaN, -inf and x <= -700 give exp(-700), zero gives exactly 1). Prints
// the figures and the points checked.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "exp_tab.h"

static double ulp_of(double v) {
    const double a = std::fabs(v);
    return std::nextafter(a, INFINITY) - a;
}

int main() {
    double tab[256], tab_adj[256];
    for (int j = 0; j < 256; ++j) {
        tab[j] = std::exp2((double)j / 256.0);
        tab_adj[j] = jf::exp_tab_adjust(tab[j], j);
    }
    double max_ulp = 0.0, max_sub = 0.0, worst = 0.0;
    long points = 0;
    uint64_t state = 0x9e3779b97f4a7c15ull;   // splitmix64
    auto next = [&]() {
        uint64_t z = (state += 0x9e3779b97f4a7c15ull);
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        return z ^ (z >> 31);
    };
    bool nonpos = false;
    double rel_near = 0.0, rel_far = 0.0;
    auto check = [&](double x) {
        if (nonpos) {
            if (!(x <= 0.0)) return;
            ++points;
            const double ref = std::exp(x);
            const double got = jf::exp_tab_nonpos(x, tab_adj);
            if (x >= -700.0) {
                const double rel = std::fabs(got - ref) / ref;
                double& slot = x >= -40.0 ? rel_near : rel_far;
                if (rel > slot) slot = rel;
            } else if (!(std::fabs(got - std::exp(-700.0)) <= 1e-13 * std::exp(-700.0))) {
                rel_far = 1.0;                  // below -700: exp(-700)
            }
            return;
        }
        const double ref = std::exp(x);
        const double got = jf::exp_tab(x, tab);
        ++points;
        if (ref == 0.0) {
            if (got != 0.0 && got > 4.9406564584124654e-324 * 1.5) {
                std::printf("x=%.17g: expected 0, got %.17g\n", x, got);
                max_sub = 1e9;
            }
            return;
        }
        const double err = std::fabs(got - ref);
        if (ref < 2.2250738585072014e-308) {
            const double steps = err / 4.9406564584124654e-324;
            if (steps > max_sub) max_sub = steps;
        } else {
            const double u = err / ulp_of(ref);
            if (u > max_ulp) {
                max_ulp = u;
                worst = x;
            }
        }
    };
    // a dense grid over the whole range, every table slot at many offsets, and random
    // points; then the same points (those <= 0) for exp_tab_nonpos, with the special
    // inputs it reads (NaN and -inf give exp(-700), the clamp at -700, zero gives 1)
    for (int pass = 0; pass < 2; ++pass) {
        nonpos = pass == 1;
        for (long i = 0; i <= 4000000; ++i) check(-745.0 + (709.0 + 745.0) * (double)i / 4000000.0);
        for (int k = -256 * 1075; k <= 256 * 1023; k += 7)
            for (int f = -3; f <= 3; ++f) check((double)k * (0.6931471805599453 / 256.0) + f * 1e-4);
        for (int i = 0; i < 2000000; ++i) {
            const double u = (double)(next() >> 11) * 0x1.0p-53;
            check(-745.0 + 1454.0 * u);
            check((u - 0.5) * 1e-3);            // around zero
        }
        for (double x : {-745.5, -746.0, -746.5, -800.0, -1e300}) check(x);
    }
    long special_bad = 0;
    for (double x : {(double)NAN, -(double)INFINITY, -700.0, -746.0, -1e300})
        special_bad += !(std::fabs(jf::exp_tab_nonpos(x, tab_adj) - std::exp(-700.0)) <= 1e-13 * std::exp(-700.0));
    special_bad += jf::exp_tab_nonpos(0.0, tab_adj) != 1.0;
    special_bad += jf::exp_tab_nonpos(-0.0, tab_adj) != 1.0;
    for (long i = 0; i <= 4000000; ++i) {                   // exp_tab_nonpos where the scan's terms live
        nonpos = true;
        check(-40.0 * (double)i / 4000000.0);
    }
    std::printf("points %ld max_ulp %.4f at x=%.17g max_subnormal_steps %.4f special_bad %ld nonpos_rel_near %.3e "
                "nonpos_rel_far %.3e\n", points, max_ulp, worst, max_sub, special_bad, rel_near, rel_far);
    return 0;
}
