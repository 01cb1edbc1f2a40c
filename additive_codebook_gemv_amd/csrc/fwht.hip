// Online block Walsh-Hadamard rotation of the activation (Drop-by-Drop,
// section 5: block-wise Walsh-Hadamard rotation; applied online at inference).
// One 64-wide wavefront transforms one block of b inputs (fwht_device.h) and
// rounds the result once to the output type.  With a sign mask the inputs are
// first multiplied by eps = +-1 (the randomized Hadamard transform
// H diag(eps) of ApexQuant, section 3); a negation is exact, so the result is
// the unsigned rotation of the sign-flipped input, bit for bit.
#include "fwht_device.h"

namespace aqd {

template <int DT>
__device__ __forceinline__ float load_as_f32(const void* p, int64_t i) {
    if (DT == AQD_F16) return h2f(static_cast<const uint16_t*>(p)[i]);
    if (DT == AQD_BF16) return bf2f(static_cast<const uint16_t*>(p)[i]);
    return static_cast<const float*>(p)[i];
}

template <int DT>
__device__ __forceinline__ void store_from_f32(void* p, int64_t i, int64_t plane, float v) {
    if (DT == AQD_F16) {
        static_cast<uint16_t*>(p)[i] = f2h(v);
    } else if (DT == AQD_BF16) {
        static_cast<uint16_t*>(p)[i] = f2bf(v);
    } else if (DT == AQD_F32) {
        static_cast<float*>(p)[i] = v;
    } else {  // AQD_BF16X2: hi plane then lo plane
        const uint16_t hi = f2bf(v);
        static_cast<uint16_t*>(p)[i] = hi;
        static_cast<uint16_t*>(p)[plane + i] = f2bf(v - bf2f(hi));
    }
}

// Grid: x covers the blocks of one row, four per workgroup (one per wave);
// y strides over the rows.  The block and row indices are wave-uniform.
template <int B, int IN, int OUT>
__global__ __launch_bounds__(256) void hadamard_kernel(const void* x, void* y, const uint64_t* signs,
                                                       int32_t blocks_per_row, int64_t batch, int64_t d_in,
                                                       int64_t plane) {
    constexpr int E = B / 64;
    const int lane = threadIdx.x & 63;
    const int blk = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    if (blk >= blocks_per_row) return;
    const int64_t col = (int64_t)blk * B;                      // first input of the block in its row
    for (int64_t row = blockIdx.y; row < batch; row += gridDim.y) {
        const int64_t base = row * d_in + col;
        float v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = load_as_f32<IN>(x, base + e * 64 + lane);
        if (signs) {                                           // uniform: bit `lane` of word (col + 64e) / 64
#pragma unroll
            for (int e = 0; e < E; ++e)
                if ((signs[col / 64 + e] >> lane) & 1ull) v[e] = -v[e];
        }
        fwht_block<B>(v, lane);
#pragma unroll
        for (int e = 0; e < E; ++e) store_from_f32<OUT>(y, base + e * 64 + lane, plane, v[e]);
    }
}

template <int B, int IN>
static hipError_t launch_out(const void* x, void* y, const uint64_t* sg, int out_dt, int64_t batch, int64_t d_in,
                             hipStream_t s) {
    const int32_t per_row = (int32_t)(d_in / B);
    const int64_t plane = batch * d_in;
    const dim3 grid((unsigned)((per_row + 3) / 4), (unsigned)(batch < 65535 ? batch : 65535)), block(256);
    switch (out_dt) {
        case AQD_F16: hipLaunchKernelGGL((hadamard_kernel<B, IN, AQD_F16>), grid, block, 0, s, x, y, sg, per_row, batch, d_in, plane); break;
        case AQD_BF16: hipLaunchKernelGGL((hadamard_kernel<B, IN, AQD_BF16>), grid, block, 0, s, x, y, sg, per_row, batch, d_in, plane); break;
        case AQD_F32: hipLaunchKernelGGL((hadamard_kernel<B, IN, AQD_F32>), grid, block, 0, s, x, y, sg, per_row, batch, d_in, plane); break;
        default: hipLaunchKernelGGL((hadamard_kernel<B, IN, AQD_BF16X2>), grid, block, 0, s, x, y, sg, per_row, batch, d_in, plane); break;
    }
    return hipGetLastError();
}

template <int B>
static hipError_t launch_in(const void* x, void* y, const uint64_t* sg, int in_dt, int out_dt, int64_t batch,
                            int64_t d_in, hipStream_t s) {
    switch (in_dt) {
        case AQD_F16: return launch_out<B, AQD_F16>(x, y, sg, out_dt, batch, d_in, s);
        case AQD_BF16: return launch_out<B, AQD_BF16>(x, y, sg, out_dt, batch, d_in, s);
        default: return launch_out<B, AQD_F32>(x, y, sg, out_dt, batch, d_in, s);
    }
}

hipError_t launch_hadamard(const void* x, void* y, int in_dt, int out_dt, int64_t batch, int64_t d_in, int block,
                           const uint8_t* signs, hipStream_t s) {
    const uint64_t* sg = reinterpret_cast<const uint64_t*>(signs);
    if (block == 64) return launch_in<64>(x, y, sg, in_dt, out_dt, batch, d_in, s);
    if (block == 128) return launch_in<128>(x, y, sg, in_dt, out_dt, batch, d_in, s);
    return launch_in<256>(x, y, sg, in_dt, out_dt, batch, d_in, s);
}

}  // namespace aqd
