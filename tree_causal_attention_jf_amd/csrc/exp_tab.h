// exp(x) in fp64 for x <= 0 from a 256-entry table of 2^(j/256), for the tree
// construction kernel's per-value exponentials. Host and device: the same
// source is checked against the C library's exp on the CPU
// (tests/c_abi/exp_tab_check.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace jf {

// Entry j of the table exp_tab_nonpos reads: 2^(j/256) with j << 44 taken from its
// bit pattern (j << 12 from the high word), so that adding k << 12 to the high
// word, where k & 255 == j, gives 2^(k >> 8) * 2^(j/256) exactly.
__host__ __device__ inline double exp_tab_adjust(double t, int j) {
    return __builtin_bit_cast(double, __builtin_bit_cast(unsigned long long, t) - ((unsigned long long)j << 44));
}

// exp(x) for x <= 0 (results down to exp(-700)): the scan's terms exp(z - m)
// against a reference m no smaller than any z, where each term only has to be
// good to a relative 1e-13 (they are summed into a logsumexp whose decisions need
// far less). x = k ln2/256 + r with k an integer and |r| <= ln2/512, and
// e^x = 2^(k >> 8) * tab[k & 255] * e^r with tab[j] = 2^(j/256):
//  * a max clamps x at -700 (and turns a NaN into -700): a NaN, -inf or x < -700
//    gives exp(-700) ~ 1e-304, which vanishes beside the reference term, 1;
//  * k = rint(x * 256/ln2) comes from one fused multiply-add with the rounding
//    constant 1.5 * 2^52 (the sum's unit in the last place is 1, so k sits in the
//    low word of its bit pattern, and k itself is the sum minus the constant);
//  * r = x - k * ln2/256 with ln2/256 rounded to one double: an error of at most
//    |k| * 2.2e-19 in r (3.2e-15 relative for |x| <= 40);
//  * e^r - 1 by r (c1 + c2 r + c3 r^2), the minimax polynomial of that form on
//    |r| <= ln2/512 (relative error 2.4e-14; fitted as a linear program over a
//    dense grid). It vanishes at r = 0, so exp(0) is exactly 1: a row with one
//    finite logit gives that token a log-probability of exactly 0, and rows with
//    equal maxima tie exactly;
//  * 2^(k >> 8) by an integer add to the table entry's high word (tab holds
//    exp_tab_adjust(2^(j/256), j)): no ldexp, and at x >= -700 the exponent
//    stays normal.
// Measured relative error (tests/c_abi/exp_tab_check.cpp): at most 4e-14 for
// -40 <= x <= 0, 1e-13 down to -700.
__host__ __device__ inline double exp_tab_nonpos(double x, const double* __restrict__ tab) {
    constexpr double kInvStep = 369.3299304675746;           // 256 / ln 2
    constexpr double kStep = 0x1.62e42fefa39efp-9;           // ln 2 / 256
    constexpr double kShift = 0x1.8p52;
    constexpr double c1 = 0x1.00000000000d1p+0, c2 = 0x1.0000021f6e2c6p-1, c3 = 0x1.5555523a6aed1p-3;
    const double xc = __builtin_fmax(x, -700.0);
    const double y = __builtin_fma(xc, kInvStep, kShift);
    const unsigned k = (unsigned)__builtin_bit_cast(unsigned long long, y);
    const double kd = y - kShift;
    const double r = __builtin_fma(-kd, kStep, xc);
    const double p = r * __builtin_fma(r, __builtin_fma(r, c3, c2), c1);
    typedef unsigned words2 __attribute__((ext_vector_type(2)));   // (low word, high word)
    words2 tw = __builtin_bit_cast(words2, tab[k & 255]);
    tw.y += k << 12;                                               // one 32-bit add on the high word
    const double t = __builtin_bit_cast(double, tw);
    return __builtin_fma(t, p, t);
}

}  // namespace jf
