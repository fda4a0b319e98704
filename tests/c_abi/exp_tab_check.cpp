// Accuracy of the tree-construction kernel's table exponential (exp_tab.h,
// the same source the kernel compiles), on the CPU against the C library's
// exp. The table is filled with the C library's exp2, as the kernel fills it
// with the device library's. Prints the largest error in ulps of the result
// (normal results) and in subnormal steps (subnormal results), and the
// number of points checked.
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
    double tab[256];
    for (int j = 0; j < 256; ++j) tab[j] = std::exp2((double)j / 256.0);
    double max_ulp = 0.0, max_sub = 0.0, worst = 0.0;
    long points = 0;
    uint64_t state = 0x9e3779b97f4a7c15ull;   // splitmix64
    auto next = [&]() {
        uint64_t z = (state += 0x9e3779b97f4a7c15ull);
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        return z ^ (z >> 31);
    };
    auto check = [&](double x) {
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
    // a dense grid over the whole range, every table slot at many offsets, and random points
    for (long i = 0; i <= 4000000; ++i) check(-745.0 + (709.0 + 745.0) * (double)i / 4000000.0);
    for (int k = -256 * 1075; k <= 256 * 1023; k += 7)
        for (int f = -3; f <= 3; ++f) check((double)k * (0.6931471805599453 / 256.0) + f * 1e-4);
    for (int i = 0; i < 2000000; ++i) {
        const double u = (double)(next() >> 11) * 0x1.0p-53;
        check(-745.0 + 1454.0 * u);
        check((u - 0.5) * 1e-3);            // around zero
    }
    std::printf("points %ld max_ulp %.4f at x=%.17g max_subnormal_steps %.4f\n", points, max_ulp, worst, max_sub);
    return 0;
}
