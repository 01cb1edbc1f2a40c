// Small-batch product (batch 1..64) on the bf16 matrix cores.
//
// Same operation as the GEMV (Drop-by-Drop, section 3.2 reconstruction from
// the first k codebooks, section 5), but with enough activation columns that
// the work is a dense contraction: each wave rebuilds a 16-row x 32-input
// slice of the weights from the codes (codeword sums in fp32), splits it into
// bf16 hi + lo, and feeds it to v_mfma_f32_16x16x32_bf16 against 16-column
// tiles of the rotated activation, accumulating in fp32.
//
// Workgroup: 4 waves, one 16-row tile each; the k codebooks live in LDS and the
// code tiles of the current group tile are staged in LDS so that each lane can
// pick the codes of exactly the weights its MFMA operand slot holds.  The
// group tiles are split over gridDim.y; partial results are added atomically
// into y (zero-filled first) when the split is more than one.
#include "aqd_internal.h"

namespace aqd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int SB_WAVES = 4;

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

__device__ __forceinline__ void add_codeword(float (&w)[8], const uint4& c) {
    const uint32_t u[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        w[2 * q] += h2f((uint16_t)(u[q] & 0xFFFFu));
        w[2 * q + 1] += h2f((uint16_t)(u[q] >> 16));
    }
}

template <int NT, bool XLO>
__global__ __launch_bounds__(64 * SB_WAVES) void gemm_sb_kernel(
    const uint8_t* __restrict__ packed, const uint4* __restrict__ codebooks, const uint16_t* __restrict__ scales,
    int k, const uint16_t* __restrict__ x, float* __restrict__ y, int64_t d_out, int64_t d_in, int64_t G,
    int64_t n_rt, int64_t n_gt, int64_t plane_bytes, int batch, int64_t gt_per_split, int atomic) {
    extern __shared__ uint4 lds[];
    uint4* cb_lds = lds;                                               // [k][256]
    uint8_t* tiles = reinterpret_cast<uint8_t*>(lds + k * CODEWORDS);  // [wave][k][1024]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t it = (int64_t)blockIdx.x * SB_WAVES + wave;
    const bool row_ok = it < n_rt;
    const int64_t gt0 = (int64_t)blockIdx.y * gt_per_split;
    const int64_t gt1 = gt0 + gt_per_split < n_gt ? gt0 + gt_per_split : n_gt;

    for (int i = tid; i < k * CODEWORDS; i += 64 * SB_WAVES) cb_lds[i] = codebooks[i];

    floatx4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    uint8_t* my_tiles = tiles + (size_t)wave * k * TILE_BYTES;
    const uint16_t* x_lo = x + (int64_t)batch * d_in;
    const int r = lane & 15;     // weight row inside the tile (MFMA A row)
    const int kq = lane >> 4;    // which 8-wide k slot of the 32-wide MFMA step

    for (int64_t jt = gt0; jt < gt1; ++jt) {
        __syncthreads();  // previous tiles consumed (and codebooks stored on the first pass)
        if (row_ok) {
            for (int m = 0; m < k; ++m) {
                const uint4 v = *reinterpret_cast<const uint4*>(packed + m * plane_bytes +
                                                                (jt * n_rt + it) * TILE_BYTES + lane * TILE_ROWS);
                *reinterpret_cast<uint4*>(my_tiles + m * TILE_BYTES + lane * TILE_ROWS) = v;
            }
        }
        __syncthreads();
        if (!row_ok) continue;
#pragma unroll 2
        for (int s = 0; s < TILE_GROUPS / 4; ++s) {
            const int gl = 4 * s + kq;
            const int64_t j = jt * TILE_GROUPS + gl;
            float w[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (j < G) {
                for (int m = 0; m < k; ++m) {
                    const uint32_t c = my_tiles[m * TILE_BYTES + gl * TILE_ROWS + r];
                    add_codeword(w, cb_lds[m * CODEWORDS + c]);
                }
            }
            bf16x8_t a_hi, a_lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const __bf16 h = (__bf16)w[e];
                a_hi[e] = h;
                a_lo[e] = (__bf16)(w[e] - (float)h);
            }
            const int64_t kk = j * GROUP;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int col = t * 16 + r;
                uint4 bh = {0u, 0u, 0u, 0u}, bl = {0u, 0u, 0u, 0u};
                if (col < batch && j < G) {
                    bh = *reinterpret_cast<const uint4*>(x + (int64_t)col * d_in + kk);
                    if (XLO) bl = *reinterpret_cast<const uint4*>(x_lo + (int64_t)col * d_in + kk);
                }
                const bf16x8_t b_hi = __builtin_bit_cast(bf16x8_t, bh);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, b_hi, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, b_hi, acc[t], 0, 0, 0);
                if (XLO) {
                    const bf16x8_t b_lo = __builtin_bit_cast(bf16x8_t, bl);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, b_lo, acc[t], 0, 0, 0);
                }
            }
        }
    }

    if (!row_ok) return;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int col = t * 16 + r;
        if (col >= batch) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t i = it * TILE_ROWS + 4 * kq + q;
            if (i >= d_out) continue;
            const float v = h2f(scales[i]) * acc[t][q];
            if (atomic) unsafeAtomicAdd(y + (int64_t)col * d_out + i, v);
            else y[(int64_t)col * d_out + i] = v;
        }
    }
}

size_t gemm_sb_workspace_bytes(const Geometry&, int) { return 0; }

template <int NT, bool XLO>
static hipError_t launch_t(const uint8_t* packed, const uint16_t* cb, const uint16_t* scales, int k,
                           const uint16_t* x, float* y, int batch, const Geometry& g, hipStream_t s) {
    const int64_t wg_rows = (g.n_rt + SB_WAVES - 1) / SB_WAVES;
    int64_t splits = (512 + wg_rows - 1) / wg_rows;
    if (splits > g.n_gt) splits = g.n_gt;
    if (splits > 16) splits = 16;
    if (splits < 1) splits = 1;
    const int64_t per = g.n_gt > 0 ? (g.n_gt + splits - 1) / splits : 0;
    if (per > 0) splits = (g.n_gt + per - 1) / per;
    const int atomic = splits > 1 ? 1 : 0;
    if (atomic || g.n_gt == 0) {
        const int64_t n = (int64_t)batch * g.d_out;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)),
                           dim3(256), 0, s, y, n);
        if (g.n_gt == 0) return hipGetLastError();
    }
    const size_t lds = (size_t)k * CODEWORDS * 16 + (size_t)SB_WAVES * k * TILE_BYTES;
    hipLaunchKernelGGL((gemm_sb_kernel<NT, XLO>), dim3((unsigned)wg_rows, (unsigned)splits), dim3(64 * SB_WAVES),
                       lds, s, packed, reinterpret_cast<const uint4*>(cb), scales, k, x, y, g.d_out, g.d_in, g.G,
                       g.n_rt, g.n_gt, g.plane_bytes, batch, per, atomic);
    return hipGetLastError();
}

template <bool XLO>
static hipError_t launch_x(const uint8_t* packed, const uint16_t* cb, const uint16_t* scales, int k,
                           const uint16_t* x, float* y, int batch, const Geometry& g, hipStream_t s) {
    const int nt = (batch + 15) / 16;
    switch (nt) {
        case 1: return launch_t<1, XLO>(packed, cb, scales, k, x, y, batch, g, s);
        case 2: return launch_t<2, XLO>(packed, cb, scales, k, x, y, batch, g, s);
        case 3: return launch_t<3, XLO>(packed, cb, scales, k, x, y, batch, g, s);
        default: return launch_t<4, XLO>(packed, cb, scales, k, x, y, batch, g, s);
    }
}

hipError_t launch_gemm_sb(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                          const void* x, int x_dt, float* y, int batch, const Geometry& g, void*, hipStream_t s) {
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    if (x_dt == AQD_BF16X2) return launch_x<true>(packed, codebooks, scales, k, xb, y, batch, g, s);
    return launch_x<false>(packed, codebooks, scales, k, xb, y, batch, g, s);
}

}  // namespace aqd
