// Decode GEMV, batch 1..8: lookup-and-accumulate over the packed code tiles
// (batch 1 and 2 through the table kernels, batch 3 and 4 at k <= 2 on small
// slot counts through the four-column tables, otherwise batch 2..8 with
// batch * k > 4 through the fp16 matrix-core kernel, the rest here).
//
// Drop-by-Drop ("Multi-Bitwidth Quantization for LLMs Using Additive
// Codebooks"), section 3.2: every 8-wide group of a weight row is the sum of
// one codeword per codebook; section 5: only the first k codebooks are used.
// So  y[n][i] = s_i * sum_j sum_{m<k} < C_m[code(i,j,m)], xrot[n][8j..8j+8) >.
//
// One workgroup owns one tile of 16 rows.  The k codebooks (k x 4 KiB fp16)
// sit in LDS.  Each wave walks a share of the (codebook, group tile) pairs;
// per pair, lane l loads the 16 codes of group l for the 16 rows (one 1 KiB
// tile per wave, a single coalesced 16-byte load per lane), reads the 8-wide
// activation slice of its group once, and for every row gathers the codeword
// from LDS and accumulates its dot product with the activation in fp32
// (v_dot2 on fp16 pairs).  The 16 row sums of every lane are folded across the
// wave with a transposing butterfly, then across the waves in LDS, scaled and
// rounded to fp16.
#include "aqd_internal.h"

namespace aqd {

constexpr int GEMV_WAVES = 8;

__device__ __forceinline__ float dot8(const uint4& w, const uint4& x, float acc) {
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.x), __builtin_bit_cast(half2_t, x.x), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.y), __builtin_bit_cast(half2_t, x.y), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.z), __builtin_bit_cast(half2_t, x.z), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w.w), __builtin_bit_cast(half2_t, x.w), acc, false);
    return acc;
}

// Fold v[16][NB] (one value per row and column in every lane) across the 64
// lanes.  After the four halving steps lane l holds row
// r = 8*b5 + 4*b4 + 2*b3 + b2 (b = bits of l); the last two steps finish the
// sum over the four lanes that share r.
template <int NB>
__device__ __forceinline__ void wave_fold_rows(float (&v)[16][NB], int lane, float (&out)[NB]) {
    float a[8][NB];
    {
        const bool hi = (lane & 32) != 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float send = hi ? v[i][b] : v[i + 8][b];
                const float keep = hi ? v[i + 8][b] : v[i][b];
                a[i][b] = keep + __shfl_xor(send, 32);
            }
    }
    float c[4][NB];
    {
        const bool hi = (lane & 16) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float send = hi ? a[i][b] : a[i + 4][b];
                const float keep = hi ? a[i + 4][b] : a[i][b];
                c[i][b] = keep + __shfl_xor(send, 16);
            }
    }
    float d[2][NB];
    {
        const bool hi = (lane & 8) != 0;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float send = hi ? c[i][b] : c[i + 2][b];
                const float keep = hi ? c[i + 2][b] : c[i][b];
                d[i][b] = keep + __shfl_xor(send, 8);
            }
    }
    {
        const bool hi = (lane & 4) != 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float send = hi ? d[0][b] : d[1][b];
            const float keep = hi ? d[1][b] : d[0][b];
            float e = keep + __shfl_xor(send, 4);
            e += __shfl_xor(e, 2);
            e += __shfl_xor(e, 1);
            out[b] = e;
        }
    }
}

template <int NB>
__global__ __launch_bounds__(64 * GEMV_WAVES) void gemv_direct_kernel(
    const uint8_t* __restrict__ packed, const uint4* __restrict__ codebooks, const uint16_t* __restrict__ scales,
    int k, const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int64_t d_out, int64_t d_in, int64_t G,
    int64_t n_rt, int64_t n_gt, int64_t plane_bytes) {
    extern __shared__ uint4 cb_lds[];              // [k][256] codewords, 16 bytes each
    __shared__ float red[GEMV_WAVES][16][NB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t it = blockIdx.x;

    if (n_gt > 0)
        for (int i = tid; i < k * CODEWORDS; i += 64 * GEMV_WAVES) cb_lds[i] = codebooks[i];
    __syncthreads();

    float acc[16][NB];
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;

    const int64_t n_items = (int64_t)k * n_gt;
    for (int64_t item = wave; item < n_items; item += GEMV_WAVES) {
        const int m = (int)(item / n_gt);
        const int64_t jt = item % n_gt;
        const int64_t j = jt * TILE_GROUPS + lane;
        if (j >= G) continue;                       // padding group: contributes nothing
        const uint4 codes = *reinterpret_cast<const uint4*>(packed + m * plane_bytes +
                                                            (jt * n_rt + it) * TILE_BYTES + lane * TILE_ROWS);
        uint4 xv[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) xv[b] = *reinterpret_cast<const uint4*>(x + b * d_in + j * GROUP);
        const uint4* cb = cb_lds + m * CODEWORDS;
        const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t c = (cw[r >> 2] >> (8 * (r & 3))) & 0xFFu;
            const uint4 w = cb[c];
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[r][b] = dot8(w, xv[b], acc[r][b]);
        }
    }

    float part[NB];
    wave_fold_rows<NB>(acc, lane, part);
    if ((lane & 3) == 0) {
        const int r = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
#pragma unroll
        for (int b = 0; b < NB; ++b) red[wave][r][b] = part[b];
    }
    __syncthreads();
    if (tid < 16 * NB) {
        const int r = tid / NB, b = tid % NB;
        const int64_t i = it * TILE_ROWS + r;
        if (i < d_out) {
            float s = 0.f;
#pragma unroll
            for (int w = 0; w < GEMV_WAVES; ++w) s += red[w][r][b];
            y[b * d_out + i] = f2h(h2f(scales[i]) * s);
        }
    }
}

// Batch 2..8 with batch * k > 4 goes to the fp16 matrix-core kernel: there its cost
// (about the same for any batch up to 16) undercuts the 4 * batch dot products
// per code of the direct kernel.
static bool gemv_use_mfma(int batch, int k) { return batch >= 2 && batch * k > 4; }

// The lookup-table accumulators of batch 1..4 (which must stay zero between
// calls) come first; the matrix-core route's partial sums (overwritten by every
// call) follow.
static size_t lut_region(const Geometry& g) {
    size_t b = gemv_lut_workspace_bytes(g);
    const size_t b2 = gemv_lut2_workspace_bytes(g), b4 = gemv_lut4_workspace_bytes(g);
    b = b2 > b ? b2 : b;
    b = b4 > b ? b4 : b;
    return (b + 255) & ~(size_t)255;
}

size_t gemv_zeroed_bytes(const Geometry& g) { return lut_region(g); }

size_t gemv_workspace_bytes(const Geometry& g, int batch) {
    return lut_region(g) + (batch >= 2 ? gemm_sb_workspace_bytes(g, batch) : 0);
}

template <int NB>
static hipError_t launch_nb(const uint8_t* packed, const uint16_t* cb, const uint16_t* scales, int k,
                            const uint16_t* x, uint16_t* y, const Geometry& g, hipStream_t s) {
    const size_t lds = (size_t)k * CODEWORDS * 16;
    hipLaunchKernelGGL((gemv_direct_kernel<NB>), dim3((unsigned)g.n_rt), dim3(64 * GEMV_WAVES), lds, s, packed,
                       reinterpret_cast<const uint4*>(cb), scales, k, x, y, g.d_out, g.d_in, g.G, g.n_rt, g.n_gt,
                       g.plane_bytes);
    return hipGetLastError();
}

hipError_t launch_gemv(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                       const uint16_t* x, uint16_t* y, int batch, const Geometry& g, void* ws, hipStream_t s) {
    if (gemv_lut_supported(g, batch, k)) return launch_gemv_lut(packed, codebooks, scales, k, x, y, g, ws, s);
    if (gemv_lut2_supported(g, batch, k)) return launch_gemv_lut2(packed, codebooks, scales, k, x, y, g, ws, s);
    if (gemv_lut4_supported(g, batch, k)) return launch_gemv_lut4(packed, codebooks, scales, k, x, y, batch, g, ws, s);
    if (gemv_use_mfma(batch, k))
        return launch_gemm_sb_f16out(packed, codebooks, scales, k, x, y, batch, g,
                                     ws ? static_cast<uint8_t*>(ws) + lut_region(g) : nullptr, s);
    switch (batch) {
        case 1: return launch_nb<1>(packed, codebooks, scales, k, x, y, g, s);
        case 2: return launch_nb<2>(packed, codebooks, scales, k, x, y, g, s);
        case 3: return launch_nb<3>(packed, codebooks, scales, k, x, y, g, s);
        case 4: return launch_nb<4>(packed, codebooks, scales, k, x, y, g, s);
        case 5: return launch_nb<5>(packed, codebooks, scales, k, x, y, g, s);
        case 6: return launch_nb<6>(packed, codebooks, scales, k, x, y, g, s);
        case 7: return launch_nb<7>(packed, codebooks, scales, k, x, y, g, s);
        default: return launch_nb<8>(packed, codebooks, scales, k, x, y, g, s);
    }
}

}  // namespace aqd
