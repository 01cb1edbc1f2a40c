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
constexpr int FIX_MAX_TERMS = 255;

// The biased term of v: round-to-nearest-even(v * 2^24), saturated at
// +-(2^47 - 1), plus 2^47.  Computed in fp32 and 32-bit integers without
// rounding error: a = |v| * 2^24 is exact in fp32; its high word
// h = floor(a * 2^-32) and the remainder a - h * 2^32 (a multiple of the ulp
// of a below 2^32, so exact in fp32) are integers below 2^32 except for the
// fraction bits of a < 2^24, which rintf rounds; round-to-nearest-even is
// symmetric, so the sign is applied to the rounded magnitude.
__device__ __forceinline__ unsigned long long fix_term(float v) {
    const float a = __builtin_fabsf(v) * (float)(1 << FIX_FRAC);
    unsigned long long n = FIX_BIAS - 1;                         // saturated magnitude
    if (a < (float)FIX_BIAS) {
        const float h = __builtin_floorf(a * (1.0f / 4294967296.0f));
        const float r = __builtin_fmaf(h, -4294967296.0f, a);
        n = ((unsigned long long)(uint32_t)h << 32) + (uint32_t)__builtin_rintf(r);
    }
    return v < 0.f ? FIX_BIAS - n : FIX_BIAS + n;
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
