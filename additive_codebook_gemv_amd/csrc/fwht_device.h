// Block Walsh-Hadamard butterflies on one 64-wide wavefront (Drop-by-Drop,
// section 5: block-wise Walsh-Hadamard rotation of the activation, online).
//
// Lane l holds the elements l, l + 64, l + 128, ... of a block of B inputs
// (B/64 per lane).  The six stages whose partners are 1..32 apart cross lanes,
// the stages 64 and 128 apart stay in registers.  Sums are fp32; the result is
// scaled by 1/sqrt(B).  The network gives the Sylvester-order matrix
// H[r][c] = (-1)^popcount(r & c).  Shared by the standalone rotation and the
// GEMV that rotates its own input, so both produce the same bits.
#pragma once
#include "aqd_internal.h"

namespace aqd {

template <int B>
__device__ __forceinline__ float inv_sqrt_block() {
    return B == 64 ? 0.125f : (B == 128 ? 0.0883883476483184405f : 0.0625f);
}

template <int B>
__device__ __forceinline__ void fwht_block(float (&v)[B / 64], int lane) {
    constexpr int E = B / 64;
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
        const bool upper = (lane & h) != 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float o = __shfl_xor(v[e], h);
            v[e] = upper ? (o - v[e]) : (v[e] + o);
        }
    }
#pragma unroll
    for (int hb = 1; hb < E; hb <<= 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if ((e & hb) == 0) {
                const float a = v[e], c = v[e | hb];
                v[e] = a + c;
                v[e | hb] = a - c;
            }
        }
    }
    const float sc = inv_sqrt_block<B>();
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] *= sc;
}

}  // namespace aqd
