// Encode side: greedy residual code assignment for fixed codebooks.
//
// Drop-by-Drop, section 3.2, defines the decoder: a weight group is the sum of
// one codeword from each codebook.  Section 5 fixes the order: a model uses a
// prefix of the codebooks.  The search that picks the codes (AQLM's appendix)
// is not on the pages; this is the greedy stand-in that respects the prefix
// order.  Codebook m = 0, 1, ... in turn takes the codeword nearest (squared
// Euclidean distance) to the residual the earlier codebooks left, and the
// residual loses it.
//
// The decision is an index, so it is taken in float32 with one fixed order of
// operations: e_t = r_t - C[c][t], d = fma(e_t, e_t, d) for t = 0..7 starting
// from d = 0, the smallest d wins and equal d go to the lower index, then
// r_t = r_t - C[c*][t].
//
// One thread per group of 8 targets.  The codebooks, widened to fp32 (exact),
// sit in LDS; every lane of a wave reads the same codeword at the same time,
// so each read is a broadcast.  The work is plain fp32 ALU: 8 subtractions, 8
// fmas and a compare per codeword.
#include "aqd_internal.h"

namespace aqd {

template <int M>
__global__ __launch_bounds__(256) void encode_greedy_kernel(const float* __restrict__ target,
                                                            const uint16_t* __restrict__ codebooks,
                                                            uint8_t* __restrict__ codes, int64_t n_groups) {
    __shared__ __align__(16) float cbf[M * CODEWORDS * GROUP];
    for (int i = threadIdx.x; i < M * CODEWORDS * GROUP; i += 256) cbf[i] = h2f(codebooks[i]);
    __syncthreads();
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= n_groups) return;
    const float4 t0 = reinterpret_cast<const float4*>(target)[2 * q];
    const float4 t1 = reinterpret_cast<const float4*>(target)[2 * q + 1];
    float r[GROUP] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
    uint8_t out[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float4* cm = reinterpret_cast<const float4*>(cbf + m * CODEWORDS * GROUP);
        int best = 0;
        float best_d = 0.f;
#pragma unroll 4
        for (int c = 0; c < CODEWORDS; ++c) {
            const float4 a = cm[2 * c], b = cm[2 * c + 1];
            const float cw[GROUP] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            float d = 0.f;
#pragma unroll
            for (int t = 0; t < GROUP; ++t) {
                const float e = r[t] - cw[t];
                d = __builtin_fmaf(e, e, d);
            }
            if (c == 0 || d < best_d) {
                best = c;
                best_d = d;
            }
        }
        out[m] = (uint8_t)best;
        const float* cb = cbf + (m * CODEWORDS + best) * GROUP;
#pragma unroll
        for (int t = 0; t < GROUP; ++t) r[t] = r[t] - cb[t];
    }
#pragma unroll
    for (int m = 0; m < M; ++m) codes[q * M + m] = out[m];
}

hipError_t launch_encode_greedy(const float* target, const uint16_t* codebooks, int M, int64_t d_out,
                                int64_t d_in, uint8_t* codes, hipStream_t s) {
    const int64_t n = d_out * (d_in / GROUP);
    if (n == 0) return hipSuccess;
    const dim3 gd((unsigned)((n + 255) / 256)), bd(256);
    switch (M) {
        case 1: hipLaunchKernelGGL(encode_greedy_kernel<1>, gd, bd, 0, s, target, codebooks, codes, n); break;
        case 2: hipLaunchKernelGGL(encode_greedy_kernel<2>, gd, bd, 0, s, target, codebooks, codes, n); break;
        case 3: hipLaunchKernelGGL(encode_greedy_kernel<3>, gd, bd, 0, s, target, codebooks, codes, n); break;
        case 4: hipLaunchKernelGGL(encode_greedy_kernel<4>, gd, bd, 0, s, target, codebooks, codes, n); break;
        case 5: hipLaunchKernelGGL(encode_greedy_kernel<5>, gd, bd, 0, s, target, codebooks, codes, n); break;
        case 6: hipLaunchKernelGGL(encode_greedy_kernel<6>, gd, bd, 0, s, target, codebooks, codes, n); break;
        case 7: hipLaunchKernelGGL(encode_greedy_kernel<7>, gd, bd, 0, s, target, codebooks, codes, n); break;
        default: hipLaunchKernelGGL(encode_greedy_kernel<8>, gd, bd, 0, s, target, codebooks, codes, n); break;
    }
    return hipGetLastError();
}

}  // namespace aqd
