// Order-independent sums across workgroups without fences or a second kernel.
//
// A sum travels in one 64-bit word: the top 8 bits count the contributions,
// the low 56 bits hold the sum of the contributions as fixed point with 24
// fraction bits, each biased by 2^47 so that every term is non-negative and no
// carry reaches the count (at most 255 terms below 2^48 each).  Contributors
// add with one device-scope integer atomic; integer addition makes the total
// exact and independent of arrival order, and the adder that sees S-1 earlier
// contributions in the returned word holds the complete sum, writes the result
// and clears the word (so the buffer is zero again when the kernel ends).
// Terms are clamped to |v| < 2^23.
#pragma once
#include "aqd_internal.h"

namespace aqd {

constexpr int FIX_FRAC = 24;
constexpr int FIX_COUNT_SHIFT = 56;
constexpr unsigned long long FIX_BIAS = 1ull << 47;
constexpr double FIX_LIMIT = (double)((1ll << 47) - 1);
constexpr int FIX_MAX_TERMS = 255;

__device__ __forceinline__ unsigned long long fix_term(float v) {
    double d = (double)v * (double)(1 << FIX_FRAC);
    d = d > FIX_LIMIT ? FIX_LIMIT : (d < -FIX_LIMIT ? -FIX_LIMIT : d);
    return (unsigned long long)(__double2ll_rn(d) + (long long)FIX_BIAS);
}

// The word to add for term v.
__device__ __forceinline__ unsigned long long fix_add_word(unsigned long long term) {
    return (1ull << FIX_COUNT_SHIFT) + term;
}

// True when the returned word `old` shows that this adder completed the count.
__device__ __forceinline__ bool fix_is_last(unsigned long long old, int terms) {
    return (int)(old >> FIX_COUNT_SHIFT) == terms - 1;
}

// The complete sum, from the returned word and this adder's own term.
__device__ __forceinline__ double fix_total(unsigned long long old, unsigned long long term, int terms) {
    const unsigned long long biased = (old & ((1ull << FIX_COUNT_SHIFT) - 1)) + term;
    const long long total = (long long)biased - (long long)terms * (long long)FIX_BIAS;
    return (double)total * (1.0 / (double)(1 << FIX_FRAC));
}

}  // namespace aqd
