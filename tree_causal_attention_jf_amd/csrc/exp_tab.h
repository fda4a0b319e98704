// exp(x) in fp64 from a 256-entry table of 2^(j/256), for the tree
// construction kernel's per-value exponentials. Host and device: the same
// source is checked against the C library's exp on the CPU
// (tests/c_abi/exp_tab_check.cpp).
#pragma once

#include <hip/hip_runtime.h>

namespace jf {

// exp(x) for x <= 709 (0 below -745.2). x = k ln2/256 + r with k integer
// (Cody-Waite: ln2/256 split into a 31-bit head, so k * head is exact for
// |k| < 2^22, and a tail), |r| <= ln2/512; e^r = 1 + p(r) with p the degree-4
// Taylor polynomial (remainder r^5/120 < 4e-17); e^x = 2^(k>>8) * tab[k&255] * e^r
// with tab[j] = 2^(j/256). Measured error, with the table from the C library's
// exp2: at most 1 ulp against the C library's exp over [-745, 709] (normal
// results; subnormal results within one subnormal step). Four fused
// multiply-adds instead of the dozen of a general-purpose exp.
__host__ __device__ inline double exp_tab(double x, const double* __restrict__ tab) {
    constexpr double kInvStep = 369.3299304675746;          // 256 / ln 2
    constexpr double kStepHi = 0x1.62e42fec00000p-9;         // ln 2 / 256, leading 31 bits
    constexpr double kStepLo = 0x1.d1cf79abc9e3bp-40;        // ln 2 / 256 - kStepHi
    const double xc = x > -746.0 ? x : -746.0;
    const double kd = __builtin_rint(xc * kInvStep);
    const int k = (int)kd;
    const double r = __builtin_fma(-kd, kStepLo, __builtin_fma(-kd, kStepHi, xc));
    const double p = r * (1.0 + r * (0.5 + r * (1.0 / 6.0 + r * (1.0 / 24.0))));
    const double t = tab[k & 255];
    const double e = __builtin_ldexp(__builtin_fma(t, p, t), k >> 8);
    return x > -745.2 ? e : 0.0;
}

}  // namespace jf
