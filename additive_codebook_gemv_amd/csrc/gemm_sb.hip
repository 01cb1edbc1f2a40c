// Small-batch product (batch 1..64) on the matrix cores.
//
// Same operation as the GEMV (Drop-by-Drop, section 3.2: a weight group is the
// sum of the codewords its codes pick; section 5: only the first k codebooks),
// but with enough activation columns that the work is a dense contraction:
//     Y[n][i] = s_i * sum_c W_k[i][c] * X[n][c].
//
// Workgroup: 8 waves (7 where that spreads the row tiles more evenly over the
// CUs, see sb_plan; 16 where the LDS holds only one workgroup per CU), one
// 16-row tile each, all batch columns, a range of 128-input chunks (the input
// dimension is split over gridDim.y).
// Per chunk:
//   - the rotated activation chunk (batch x 128) is staged once in LDS, double
//     buffered, and shared by the waves (MFMA B operands, padded rows so the
//     16-byte reads do not collide);
//   - each lane rebuilds exactly the 8 weights its MFMA A-operand slot holds:
//     it gathers the k codewords of its (row, group) from the LDS-resident
//     codebooks and adds them with packed fp16 adds;
//   - v_mfma_f32_16x16x32 multiplies the 16x32 weight slice by every 16-column
//     tile of the activation, accumulating in fp32.
// Precision modes: AQD_F16 activations use one fp16 MFMA pass (weights are the
// fp16 codeword sums); AQD_BF16 splits the weights into bf16 hi + lo (two
// passes); AQD_BF16X2 also adds the activation's lo plane (three passes).
// Split inputs: each split writes its partial rows to the workspace and a
// second kernel adds the splits in a fixed order, scales and stores Y, so the
// result is bit-reproducible.
#include "aqd_internal.h"

namespace aqd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int SB_WAVES = 8;                        // waves per workgroup at most
constexpr int SB_MIN_WAVES = 7;                    // and at least
constexpr int SB_WIDE_WAVES = 16;                  // when the LDS allows one workgroup per CU
constexpr int SB_CHUNK = 128;                      // inputs per chunk (16 groups)
constexpr int SB_CHUNK_GROUPS = SB_CHUNK / GROUP;
constexpr int SB_XROW = SB_CHUNK * 2 + 16;         // bytes per activation row in LDS (padded)
constexpr int SB_MAX_SPLITS = 16;

// Internal operand mode of the tiered batch: fp16 activation, each column n
// uses its own number of codebooks k_n, one MFMA per codebook plane with the
// columns that do not use that plane zeroed in the B operand.
constexpr int SB_MIXED = 100;

// Columns that use codebook m: bit n of cols[m] (n < 64).
struct SbPlaneCols {
    unsigned long long cols[MAX_M];
};

template <int MODE>
struct XPlanes {
    static constexpr int n = MODE == AQD_BF16X2 ? 2 : 1;
};

__device__ __forceinline__ half2_t h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp16 pair -> bf16 hi pair and bf16 lo pair (hi + lo equals the pair to 2^-16).
// Each pair conversion is one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ void split_bf16(uint32_t h, uint32_t& hi, uint32_t& lo) {
    const half2_t v = h2(h);
    const float a = (float)v[0], b = (float)v[1];
    const bf16x2_t hv = bf16x2_t{(__bf16)a, (__bf16)b};
    const bf16x2_t lv = bf16x2_t{(__bf16)(a - (float)hv[0]), (__bf16)(b - (float)hv[1])};
    hi = __builtin_bit_cast(uint32_t, hv);
    lo = __builtin_bit_cast(uint32_t, lv);
}

// store_partial with a nontemporal (streaming) store: the partials are read once, by the reduce.
// Measured 4-7 % faster at k <= 3 (batch 16 and 64, both MLP shapes) and neutral to 7 % slower at k = 4,
// so the kernel takes it for k <= 3; the prefill, whose partials it also slowed, keeps plain stores.
__device__ __forceinline__ void store_partial_nt(float* part, int64_t d_out, int batch, unsigned split, int col,
                                                 int64_t row0, float4 v) {
    const int64_t nq = (d_out + 3) / 4;
    __builtin_nontemporal_store(floatx4_t{v.x, v.y, v.z, v.w},
                                reinterpret_cast<floatx4_t*>(part) + ((int64_t)split * batch + col) * nq + row0 / 4);
}

template <int NT, int MODE, int K, int W>
__global__ __launch_bounds__(64 * W) void gemm_sb_kernel(
    const uint8_t* __restrict__ packed, const uint4* __restrict__ codebooks, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ x, float* __restrict__ out, int64_t d_out, int64_t d_in, int64_t G,
    int64_t n_rt, int64_t plane_bytes, int batch, int chunks_per_split, int64_t n_chunks, int direct,
    SbPlaneCols pc, int out_f16) {
    constexpr int XP = XPlanes<MODE>::n;
    extern __shared__ __align__(16) uint8_t lds[];
    uint4* cb_lds = reinterpret_cast<uint4*>(lds);                        // [k][256] codewords
    uint8_t* xbuf = lds + K * CODEWORDS * 16;                             // [2][XP][NT*16][SB_XROW]
    constexpr int XBUF = XP * NT * 16 * SB_XROW;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    constexpr int nthreads = 64 * W;
    const int64_t it = (int64_t)blockIdx.x * W + wave;            // this wave's row tile
    const bool row_ok = it < n_rt;
    const int64_t c0 = (int64_t)blockIdx.y * chunks_per_split;
    const int64_t c1 = c0 + chunks_per_split < n_chunks ? c0 + chunks_per_split : n_chunks;
    const int r = lane & 15;      // MFMA A row (weight row in the tile) / B column in the tile
    const int kq = lane >> 4;     // 8-wide k slot inside the 32-wide MFMA step

    for (int i = tid; i < K * CODEWORDS; i += nthreads) cb_lds[i] = codebooks[i];
    // tiered batch: the codebooks each of this lane's B columns uses (bit m)
    uint32_t col_planes[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        col_planes[t] = 0u;
#pragma unroll
        for (int m = 0; m < K; ++m) col_planes[t] |= (uint32_t)((pc.cols[m] >> ((t * 16 + r) & 63)) & 1ull) << m;
    }

    // activation chunk staging: thread t moves 16 bytes (8 inputs) of one row of one plane
    constexpr int X_ITEMS = XP * NT * 16 * (SB_CHUNK / 8);   // 16-byte pieces per chunk
    constexpr int X_PER_THREAD = (X_ITEMS + nthreads - 1) / nthreads;
    // every load is issued unconditionally (addresses clamped into the buffer, out-of-range pieces zeroed
    // afterwards), so the loads of the next chunk stay in flight while this chunk is multiplied
    auto x_load = [&](int64_t ch, uint4 (&v)[X_PER_THREAD]) {
#pragma unroll
        for (int q = 0; q < X_PER_THREAD; ++q) {
            const int item = (tid + q * nthreads) % X_ITEMS;
            const int piece = item % (SB_CHUNK / 8);
            const int col = (item / (SB_CHUNK / 8)) % (NT * 16);
            const int pl = item / ((SB_CHUNK / 8) * NT * 16);
            const int64_t kk = ch * SB_CHUNK + piece * 8;
            const int colc = col < batch ? col : batch - 1;
            const int64_t kkc = kk < d_in ? kk : d_in - 8;
            v[q] = *reinterpret_cast<const uint4*>(x + (int64_t)pl * batch * d_in + (int64_t)colc * d_in + kkc);
        }
    };
    auto x_fix = [&](int64_t ch, uint4 (&v)[X_PER_THREAD]) {
#pragma unroll
        for (int q = 0; q < X_PER_THREAD; ++q) {
            const int item = (tid + q * nthreads) % X_ITEMS;
            const int piece = item % (SB_CHUNK / 8);
            const int col = (item / (SB_CHUNK / 8)) % (NT * 16);
            if (col >= batch || ch * SB_CHUNK + piece * 8 >= d_in) v[q] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto x_store = [&](int buf, const uint4 (&v)[X_PER_THREAD]) {
#pragma unroll
        for (int q = 0; q < X_PER_THREAD; ++q) {
            const int item = tid + q * nthreads;
            if (item < X_ITEMS) {
                const int piece = item % (SB_CHUNK / 8);
                const int row = item / (SB_CHUNK / 8);          // pl * NT*16 + col
                *reinterpret_cast<uint4*>(xbuf + buf * XBUF + row * SB_XROW + piece * 16) = v[q];
            }
        }
    };
    // code bytes of this wave for one chunk: lane l needs, per plane and per 32-input step s,
    // the code of row r, group 4s + kq; inside a tile those 64 bytes are contiguous
    auto code_load = [&](int64_t ch, uint32_t (&cv)[K][4]) {
        const int64_t jt = (ch * SB_CHUNK_GROUPS) / TILE_GROUPS;
        const int g0 = (int)((ch * SB_CHUNK_GROUPS) % TILE_GROUPS);
        const int64_t itc = row_ok ? it : 0;
        const uint8_t* base = packed + (jt * n_rt + itc) * TILE_BYTES + g0 * TILE_ROWS + lane;
#pragma unroll
        for (int m = 0; m < K; ++m)
#pragma unroll
            for (int s = 0; s < 4; ++s) cv[m][s] = base[m * plane_bytes + 4 * s * TILE_ROWS];
    };

    floatx4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    uint4 xv[X_PER_THREAD];
    uint32_t cv[K][4];
    if (c0 < c1) {
        x_load(c0, xv);
        code_load(c0, cv);
        x_fix(c0, xv);
        x_store(0, xv);
    }
    int buf = 0;
    for (int64_t ch = c0; ch < c1; ++ch) {
        __syncthreads();                      // chunk `ch` is in xbuf[buf]; codebooks are in LDS
        uint32_t cur[K][4];
#pragma unroll
        for (int m = 0; m < K; ++m)
#pragma unroll
            for (int s = 0; s < 4; ++s) cur[m][s] = cv[m][s];
        if (ch + 1 < c1) {                    // prefetch the next chunk while this one is multiplied
            x_load(ch + 1, xv);
            code_load(ch + 1, cv);
        }
        const uint8_t* xb = xbuf + buf * XBUF;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int64_t j = ch * SB_CHUNK_GROUPS + 4 * s + kq;   // this lane's group
            if (MODE == SB_MIXED) {
                // one MFMA per codebook plane; a column that stops before plane m sees zeros there
                uint4 bx[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    bx[t] = *reinterpret_cast<const uint4*>(xb + (t * 16 + r) * SB_XROW + (32 * s + 8 * kq) * 2);
#pragma unroll
                for (int m = 0; m < K; ++m) {
                    uint4 c = cb_lds[m * CODEWORDS + cur[m][s]];
                    if (j >= G) c = make_uint4(0u, 0u, 0u, 0u);
                    const half8_t a = __builtin_bit_cast(half8_t, c);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const uint4 b = (col_planes[t] >> m) & 1u ? bx[t] : make_uint4(0u, 0u, 0u, 0u);
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8_t, b), acc[t], 0, 0, 0);
                    }
                }
                continue;
            }
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            if (j < G) {
#pragma unroll
                for (int m = 0; m < K; ++m) {
                    const uint4 c = cb_lds[m * CODEWORDS + cur[m][s]];
                    if (m == 0) {
                        w[0] = c.x; w[1] = c.y; w[2] = c.z; w[3] = c.w;
                    } else {
                        w[0] = u32(h2(w[0]) + h2(c.x));
                        w[1] = u32(h2(w[1]) + h2(c.y));
                        w[2] = u32(h2(w[2]) + h2(c.z));
                        w[3] = u32(h2(w[3]) + h2(c.w));
                    }
                }
            }
            const int kofs = (32 * s + 8 * kq) * 2;
            if (MODE == AQD_F16) {
                const half8_t a = __builtin_bit_cast(half8_t, make_uint4(w[0], w[1], w[2], w[3]));
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const uint4 bx = *reinterpret_cast<const uint4*>(xb + (t * 16 + r) * SB_XROW + kofs);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8_t, bx), acc[t], 0, 0, 0);
                }
            } else {
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) split_bf16(w[q], hi[q], lo[q]);
                const bf16x8_t ahi = __builtin_bit_cast(bf16x8_t, make_uint4(hi[0], hi[1], hi[2], hi[3]));
                const bf16x8_t alo = __builtin_bit_cast(bf16x8_t, make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const uint4 bh = *reinterpret_cast<const uint4*>(xb + (t * 16 + r) * SB_XROW + kofs);
                    const bf16x8_t bhi = __builtin_bit_cast(bf16x8_t, bh);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bhi, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bhi, acc[t], 0, 0, 0);
                    if (MODE == AQD_BF16X2) {
                        const uint4 bl = *reinterpret_cast<const uint4*>(xb + ((NT + t) * 16 + r) * SB_XROW + kofs);
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, __builtin_bit_cast(bf16x8_t, bl), acc[t], 0, 0, 0);
                    }
                }
            }
        }
        if (ch + 1 < c1) {                    // the other buffer was last read before this chunk's barrier
            x_fix(ch + 1, xv);
            x_store(buf ^ 1, xv);
        }
        buf ^= 1;
    }

    if (!row_ok) return;
    // lane l holds rows 4*kq .. 4*kq+3 of the tile, column t*16 + r
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int col = t * 16 + r;
        if (col >= batch) continue;
        const int64_t row0 = it * TILE_ROWS + 4 * kq;
        if (!direct) {            // one 16-byte partial per (column, row quad, split)
            if (row0 < d_out) {
                const float4 pv = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
                if constexpr (K <= 3) store_partial_nt(out, d_out, batch, blockIdx.y, col, row0, pv);
                else store_partial(out, d_out, batch, blockIdx.y, col, row0, pv);
            }
            continue;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t i = row0 + q;
            if (i >= d_out) continue;
            if (out_f16) reinterpret_cast<uint16_t*>(out)[(int64_t)col * d_out + i] = f2h(h2f(scales[i]) * acc[t][q]);
            else out[(int64_t)col * d_out + i] = h2f(scales[i]) * acc[t][q];
        }
    }
}

// y[n][i] = s_i * sum over splits (fixed order) of the partials, fp32 or
// (out_f16) rounded to fp16.  Thread (row quad, column n = blockIdx.y) reads one
// 16-byte word per split, all requested before any is added.
constexpr int SB_REDUCE_THREADS = 64;   // small blocks: the work is latency-bound, spread it over many CUs

__global__ __launch_bounds__(SB_REDUCE_THREADS) void sb_reduce_kernel(const float* __restrict__ part,
                                                        const uint16_t* __restrict__ scales, void* __restrict__ y,
                                                        int64_t d_out, int batch, int splits, int out_f16) {
    const int64_t q4 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int64_t nq = (d_out + 3) / 4;
    if (q4 >= nq) return;
    // the four rows' scales are requested with the partials (clamped rows), not after the sum
    float sc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int64_t i = 4 * q4 + c;
        sc[c] = h2f(scales[i < d_out ? i : d_out - 1]);
    }
    const float4* pq = reinterpret_cast<const float4*>(part) + (int64_t)blockIdx.y * nq + q4;
    const int64_t stride = (int64_t)batch * nq;                 // one split to the next
    float4 v[SB_MAX_SPLITS];
#pragma unroll
    for (int sp = 0; sp < SB_MAX_SPLITS; ++sp) v[sp] = pq[(sp < splits ? sp : 0) * stride];
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int sp = 0; sp < SB_MAX_SPLITS; ++sp)
        if (sp < splits) {
            a.x += v[sp].x;
            a.y += v[sp].y;
            a.z += v[sp].z;
            a.w += v[sp].w;
        }
    const float r[4] = {sc[0] * a.x, sc[1] * a.y, sc[2] * a.z, sc[3] * a.w};
    const int64_t e0 = (int64_t)blockIdx.y * d_out + 4 * q4;
    if ((d_out & 3) == 0) {                                      // four whole, aligned rows: one store
        if (out_f16)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + e0) =
                make_uint2((uint32_t)f2h(r[0]) | ((uint32_t)f2h(r[1]) << 16),
                           (uint32_t)f2h(r[2]) | ((uint32_t)f2h(r[3]) << 16));
        else
            *reinterpret_cast<float4*>(static_cast<float*>(y) + e0) = make_float4(r[0], r[1], r[2], r[3]);
        return;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (4 * q4 + c < d_out) {
            if (out_f16) static_cast<uint16_t*>(y)[e0 + c] = f2h(r[c]);
            else static_cast<float*>(y)[e0 + c] = r[c];
        }
    }
}

__global__ void sb_zero_kernel(float* __restrict__ y, int64_t n) {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x)
        y[e] = 0.f;
}

hipError_t launch_split_reduce(const float* part, const uint16_t* scales, float* y, int64_t d_out, int batch,
                               int splits, hipStream_t s) {
    if (splits > SB_MAX_SPLITS) return hipErrorInvalidValue;
    hipLaunchKernelGGL(sb_reduce_kernel,
                       dim3((unsigned)(((d_out + 3) / 4 + SB_REDUCE_THREADS - 1) / SB_REDUCE_THREADS), (unsigned)batch),
                       dim3(SB_REDUCE_THREADS), 0, s, part, scales, static_cast<void*>(y), d_out, batch, splits, 0);
    return hipGetLastError();
}

__global__ void sb_zero16_kernel(uint16_t* __restrict__ y, int64_t n) {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x)
        y[e] = 0;
}

hipError_t launch_zero_f16(uint16_t* y, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(sb_zero16_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)), dim3(256),
                       0, s, y, n);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float* y, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(sb_zero_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)), dim3(256),
                       0, s, y, n);
    return hipGetLastError();
}

template <int MODE>
constexpr size_t sb_lds_bytes(int k, int nt) {
    return (size_t)k * CODEWORDS * 16 + 2 * (size_t)XPlanes<MODE>::n * nt * 16 * SB_XROW;
}

struct SbPlan {
    int64_t n_chunks, wg_rows;
    int splits, chunks_per_split, waves;
};

// Waves per workgroup and splits of the input dimension.  Waves: 16 when the
// LDS holds one workgroup per CU (per_cu == 1), else 8, or 7 where that evens
// out the CUs (below).  Splits: the smallest count that minimises (rounds of
// workgroups over the chip) x (chunks per split), with `per_cu` workgroups
// resident per compute unit; at most SB_MAX_SPLITS.
static SbPlan sb_plan(const Geometry& g, int per_cu) {
    SbPlan p;
    p.n_chunks = (g.d_in + SB_CHUNK - 1) / SB_CHUNK;
    p.waves = per_cu == 1 ? SB_WIDE_WAVES : SB_WAVES;
    p.wg_rows = (g.n_rt + p.waves - 1) / p.waves;
    p.splits = 1;
    p.chunks_per_split = (int)p.n_chunks;
    if (p.wg_rows == 0 || p.n_chunks == 0) return p;
    const int64_t slots = 256 * (int64_t)per_cu;
    int64_t best = -1;
    for (int64_t sp = 1; sp <= SB_MAX_SPLITS && sp <= p.n_chunks; ++sp) {
        const int64_t cps = (p.n_chunks + sp - 1) / sp;
        const int64_t used = (p.n_chunks + cps - 1) / cps;          // splits that actually hold chunks
        const int64_t cost = ((p.wg_rows * used + slots - 1) / slots) * cps;
        if (best < 0 || cost < best) {
            best = cost;
            p.splits = (int)used;
            p.chunks_per_split = (int)cps;
        }
    }
    // With 8-wave workgroups the busiest CU may hold one more workgroup than the others.  Workgroups of
    // 7 waves (same splits, so the same sums) are taken when they fit one round and leave the busiest CU
    // fewer row tiles.
    const int64_t wgs8 = p.wg_rows * p.splits;
    const int64_t rows7 = (g.n_rt + SB_MIN_WAVES - 1) / SB_MIN_WAVES;
    const int64_t wgs7 = rows7 * p.splits;
    if (p.waves == SB_WAVES && wgs7 <= slots && ((wgs7 + 255) / 256) * SB_MIN_WAVES < ((wgs8 + 255) / 256) * SB_WAVES) {
        p.waves = SB_MIN_WAVES;
        p.wg_rows = rows7;
    }
    return p;
}

// Workgroups resident per CU: bounded by the LDS the batch tile needs (VGPR
// use, at most 128 per lane, allows two of 7 or 8 waves).  Where only one fits,
// it has 16 waves.
template <int MODE>
static int sb_per_cu(int k, int batch) {
    const size_t lds = sb_lds_bytes<MODE>(k, (batch + 15) / 16);
    const int by_lds = (int)((160 * 1024) / lds);
    return by_lds < 2 ? (by_lds < 1 ? 1 : by_lds) : 2;
}

static SbPlan sb_plan_for(const Geometry& g, int k, int batch, int x_dt) {
    const int per_cu = x_dt == AQD_BF16X2 ? sb_per_cu<AQD_BF16X2>(k, batch) : sb_per_cu<AQD_F16>(k, batch);
    return sb_plan(g, per_cu);
}

size_t gemm_sb_workspace_bytes(const Geometry& g, int batch) {
    // the largest the plan can ask for over k and the operand modes
    size_t need = 0;
    for (int k = 1; k <= g.M && k <= MAX_M; ++k)
        for (int dt : {AQD_F16, AQD_BF16X2}) {
            const SbPlan p = sb_plan_for(g, k, batch, dt);
            if (p.splits > 1) {
                const size_t b = partial_bytes(g.d_out, batch, p.splits);
                need = b > need ? b : need;
            }
        }
    return need;
}

template <int NT, int MODE, int K>
static hipError_t launch_t(const uint8_t* packed, const uint16_t* cb, const uint16_t* scales,
                           const uint16_t* x, float* y, int batch, const Geometry& g, void* ws, hipStream_t s,
                           const SbPlaneCols& pc, int out_f16) {
    const SbPlan p = sb_plan(g, sb_per_cu<MODE>(K, batch));
    const int64_t n = (int64_t)batch * g.d_out;
    if (p.n_chunks == 0) return out_f16 ? launch_zero_f16(reinterpret_cast<uint16_t*>(y), n, s)
                                        : launch_zero_f32(y, n, s);   // empty input: Y = 0
    const bool direct = p.splits == 1;
    constexpr size_t lds = sb_lds_bytes<MODE>(K, NT);
    if constexpr (2 * lds > 160 * 1024) {
        // one workgroup per CU fits the LDS: 16 waves, so the CU still holds 16
        static const hipError_t attr16 = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&gemm_sb_kernel<NT, MODE, K, SB_WIDE_WAVES>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (attr16 != hipSuccess) return attr16;
        if (p.waves != SB_WIDE_WAVES) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_sb_kernel<NT, MODE, K, SB_WIDE_WAVES>), dim3((unsigned)p.wg_rows, (unsigned)p.splits),
                           dim3(64 * p.waves), lds, s, packed, reinterpret_cast<const uint4*>(cb), scales, x,
                           direct ? y : static_cast<float*>(ws), g.d_out, g.d_in, g.G, g.n_rt, g.plane_bytes, batch,
                           p.chunks_per_split, p.n_chunks, direct ? 1 : 0, pc, out_f16);
    } else {
        static const hipError_t attr8 = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&gemm_sb_kernel<NT, MODE, K, SB_WAVES>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        static const hipError_t attr7 = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&gemm_sb_kernel<NT, MODE, K, SB_MIN_WAVES>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (attr8 != hipSuccess) return attr8;
        if (attr7 != hipSuccess) return attr7;
        auto kern = p.waves == SB_MIN_WAVES ? &gemm_sb_kernel<NT, MODE, K, SB_MIN_WAVES>
                                            : &gemm_sb_kernel<NT, MODE, K, SB_WAVES>;
        hipLaunchKernelGGL(kern, dim3((unsigned)p.wg_rows, (unsigned)p.splits),
                           dim3(64 * p.waves), lds, s, packed, reinterpret_cast<const uint4*>(cb), scales, x,
                           direct ? y : static_cast<float*>(ws), g.d_out, g.d_in, g.G, g.n_rt, g.plane_bytes, batch,
                           p.chunks_per_split, p.n_chunks, direct ? 1 : 0, pc, out_f16);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || direct) return e;
    hipLaunchKernelGGL(sb_reduce_kernel,
                       dim3((unsigned)(((g.d_out + 3) / 4 + SB_REDUCE_THREADS - 1) / SB_REDUCE_THREADS),
                            (unsigned)batch),
                       dim3(SB_REDUCE_THREADS), 0, s, static_cast<const float*>(ws), scales, static_cast<void*>(y),
                       g.d_out, batch, p.splits, out_f16);
    return hipGetLastError();
}

template <int MODE, int K>
static hipError_t launch_n(const uint8_t* packed, const uint16_t* cb, const uint16_t* scales,
                           const uint16_t* x, float* y, int batch, const Geometry& g, void* ws, hipStream_t s,
                           const SbPlaneCols& pc, int out_f16) {
    switch ((batch + 15) / 16) {
        case 1: return launch_t<1, MODE, K>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
        case 2: return launch_t<2, MODE, K>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
        case 3: return launch_t<3, MODE, K>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
        default: return launch_t<4, MODE, K>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
    }
}

template <int MODE>
static hipError_t launch_m(const uint8_t* packed, const uint16_t* cb, const uint16_t* scales, int k,
                           const uint16_t* x, float* y, int batch, const Geometry& g, void* ws, hipStream_t s,
                           const SbPlaneCols& pc, int out_f16 = 0) {
    switch (k) {
        case 1: return launch_n<MODE, 1>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
        case 2: return launch_n<MODE, 2>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
        case 3: return launch_n<MODE, 3>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
        case 4: return launch_n<MODE, 4>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
        case 5: return launch_n<MODE, 5>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
        case 6: return launch_n<MODE, 6>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
        case 7: return launch_n<MODE, 7>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
        default: return launch_n<MODE, 8>(packed, cb, scales, x, y, batch, g, ws, s, pc, out_f16);
    }
}

hipError_t launch_gemm_sb(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                          const void* x, int x_dt, float* y, int batch, const Geometry& g, void* ws,
                          hipStream_t s) {
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const SbPlaneCols none = {};
    if (x_dt == AQD_F16) return launch_m<AQD_F16>(packed, codebooks, scales, k, xb, y, batch, g, ws, s, none);
    if (x_dt == AQD_BF16X2) return launch_m<AQD_BF16X2>(packed, codebooks, scales, k, xb, y, batch, g, ws, s, none);
    return launch_m<AQD_BF16>(packed, codebooks, scales, k, xb, y, batch, g, ws, s, none);
}

hipError_t launch_gemm_sb_f16out(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                                 const uint16_t* x, uint16_t* y, int batch, const Geometry& g, void* ws,
                                 hipStream_t s) {
    const SbPlaneCols none = {};
    return launch_m<AQD_F16>(packed, codebooks, scales, k, x, reinterpret_cast<float*>(y), batch, g, ws, s, none, 1);
}

hipError_t launch_gemm_sb_tiered(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales,
                                 const int32_t* ks, const uint16_t* x, float* y, int batch, const Geometry& g,
                                 void* ws, hipStream_t s) {
    SbPlaneCols pc = {};
    int kmax = 1;
    for (int n = 0; n < batch; ++n) {
        kmax = ks[n] > kmax ? ks[n] : kmax;
        for (int m = 0; m < ks[n]; ++m) pc.cols[m] |= 1ull << n;
    }
    return launch_m<SB_MIXED>(packed, codebooks, scales, kmax, x, y, batch, g, ws, s, pc);
}

}  // namespace aqd
