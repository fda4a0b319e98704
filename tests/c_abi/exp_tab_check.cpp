// Accuracy of the tree-construction kernel's table exponential exp_tab_nonpos
// (exp_tab.h, the same source the kernel compiles), on the CPU against the C
// library's exp. The table is filled as the kernel fills it: the library's exp2
// of j/256, adjusted by exp_tab_adjust. Over x <= 0: the largest relative error
// for -40 <= x <= 0 and for -700 <= x < -40; below -700 the result must be
// exp(-700); special inputs: NaN, -inf and x <= -700 give exp(-700), +0 and -0
// give exactly 1. Points: a dense grid, every table slot at several offsets, and
// random points (splitmix64). Prints the figures and the points checked.
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "exp_tab.h"

int main() {
    double tab[256];
    for (int j = 0; j < 256; ++j) tab[j] = jf::exp_tab_adjust(std::exp2((double)j / 256.0), j);
    const double floor700 = std::exp(-700.0);
    double rel_near = 0.0, rel_far = 0.0;
    long points = 0, below_bad = 0;
    uint64_t state = 0x9e3779b97f4a7c15ull;   // splitmix64
    auto next = [&]() {
        uint64_t z = (state += 0x9e3779b97f4a7c15ull);
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        return z ^ (z >> 31);
    };
    auto check = [&](double x) {
        if (!(x <= 0.0)) return;
        ++points;
        const double got = jf::exp_tab_nonpos(x, tab);
        if (x >= -700.0) {
            const double ref = std::exp(x);
            const double rel = std::fabs(got - ref) / ref;
            double& slot = x >= -40.0 ? rel_near : rel_far;
            if (rel > slot) slot = rel;
        } else if (!(std::fabs(got - floor700) <= 1e-13 * floor700)) {
            ++below_bad;
        }
    };
    for (long i = 0; i <= 4000000; ++i) check(-745.0 * (double)i / 4000000.0);
    for (long i = 0; i <= 4000000; ++i) check(-40.0 * (double)i / 4000000.0);   // where the scan's terms live
    for (int k = -256 * 1010; k <= 0; k += 3)
        for (int f = -3; f <= 3; ++f) check((double)k * (0.6931471805599453 / 256.0) + f * 1e-4);
    for (int i = 0; i < 2000000; ++i) {
        const double u = (double)(next() >> 11) * 0x1.0p-53;
        check(-745.0 * u);
        check(-u * 1e-3);                     // next to zero
    }
    for (double x : {-700.5, -745.5, -746.0, -800.0, -1e300}) check(x);
    long special_bad = 0;
    for (double x : {(double)NAN, -(double)INFINITY, -700.0, -746.0, -1e300})
        special_bad += !(std::fabs(jf::exp_tab_nonpos(x, tab) - floor700) <= 1e-13 * floor700);
    special_bad += jf::exp_tab_nonpos(0.0, tab) != 1.0;
    special_bad += jf::exp_tab_nonpos(-0.0, tab) != 1.0;
    std::printf("points %ld rel_near %.3e rel_far %.3e below_bad %ld special_bad %ld\n", points, rel_near, rel_far,
                below_bad, special_bad);
    return 0;
}
