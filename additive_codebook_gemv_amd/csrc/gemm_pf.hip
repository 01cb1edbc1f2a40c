// Prefill / large-batch product on the matrix cores (batch up to 32768).
//
// Same operation as the other paths (Drop-by-Drop, section 3.2: a weight group
// is the sum of the codewords its codes pick; section 5: only the first k
// codebooks are used), at batch sizes where the work is a compute-bound dense
// contraction:  Y[n][i] = s_i * sum_c W_k[i][c] * X[n][c].
//
// Workgroup: 4 waves.  Wave w owns 64 weight rows (four 16-row A fragments of
// v_mfma_f32_16x16x32_f16) and every one of the workgroup's 16*NB batch
// columns, so a weight row is rebuilt exactly once per workgroup and the
// accumulators (4 x NB fragments) stay in registers for the whole input range.
// Per 64-input chunk:
//   - the activation chunk (16*NB columns x 64 inputs, fp16) is copied into
//     LDS by direct global-to-LDS loads (no registers), double buffered, with
//     an XOR swizzle so the 16 lanes that read one B fragment row hit 16
//     different bank groups;
//   - the chunk's code bytes (16 row tiles x 8 groups x k planes, 128
//     contiguous bytes per tile and plane) are copied the same way;
//   - a lane's A-operand slot (row r of the fragment, 8 consecutive inputs) is
//     exactly one code group, and the 64 slots of a fragment are 64
//     consecutive bytes of a packed code tile: one conflict-free byte read per
//     plane.  The lane adds its k codewords (LDS-resident codebooks) with
//     packed fp16 adds;
//   - each A fragment meets all NB B fragments: 4*NB MFMAs per 32 inputs.
// When the tiles cannot fill the chip the input dimension is split; each split
// writes fp32 partials to the workspace and the small-batch reduce adds them in
// a fixed order, so results are bit-reproducible.
#include "aqd_internal.h"

namespace aqd {

typedef _Float16 pf_half8_t __attribute__((ext_vector_type(8)));
typedef float pf_floatx4_t __attribute__((ext_vector_type(4)));

constexpr int PF_WAVES = 8;                              // waves per workgroup (4: slower; 16: equal, twice the activation reads)
constexpr int PF_PER_CU = 1;                              // workgroups resident per compute unit (two spill)
constexpr int PF_FRAGS = 16 / PF_WAVES;                  // 16-row A fragments per wave
constexpr int PF_TILES = PF_WAVES * PF_FRAGS;            // 16-row code tiles per workgroup (256 rows)
constexpr int PF_CHUNK = 64;                             // inputs per staged chunk (8 groups)
constexpr int PF_CHUNK_GROUPS = PF_CHUNK / GROUP;
constexpr int PF_MAX_SPLITS = 16;

struct PfArgs {
    const uint8_t* packed;
    const uint4* codebooks;
    const uint16_t* scales;
    const uint16_t* x;
    float* out;
    int64_t d_out, d_in, G, n_rt, plane_bytes, n_chunks;
    int batch, chunks_per_split, direct;
};

__device__ __forceinline__ half2_t pf_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t pf_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

typedef __attribute__((address_space(3))) void pf_lds_t;

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes dst + 16 * l (dst is uniform over the wave).
__device__ __forceinline__ void pf_dma16(const void* src, uint8_t* dst) {
    __builtin_amdgcn_global_load_lds(src, (pf_lds_t*)dst, 16, 0, 0);
}

// Activation slot of (column, 8-input piece) inside a chunk buffer: columns of
// 128 bytes, the eight 16-byte pieces XOR-swizzled by bits 1..3 of the column,
// so the 16 columns a B fragment reads at one piece fall in 16 bank groups.
__device__ __forceinline__ int pf_xslot(int col, int piece) {
    return col * (PF_CHUNK * 2) + ((piece ^ ((col >> 1) & 7)) << 4);
}

// LDS of one workgroup.  Each buffer is its own object, so the compiler can see
// that the copies in flight into one buffer never alias the reads of the other
// (and of the codebooks) and does not wait for them.
template <int K, int NB>
struct PfLds {
    static constexpr int XB = NB * 16 * PF_CHUNK * 2;                     // activations: NB*16 columns x 128 B
    static constexpr int CB = K * PF_TILES * PF_CHUNK_GROUPS * TILE_ROWS; // codes: [K][PF_TILES][8 groups][16]
};

template <int K, int NB>
__global__ __launch_bounds__(64 * PF_WAVES, PF_WAVES / 4 * PF_PER_CU) void gemm_pf_kernel(PfArgs p) {
    using L = PfLds<K, NB>;
    __shared__ __align__(16) uint4 cb_lds[K * CODEWORDS];                 // [K][256] codewords
    __shared__ __align__(16) uint8_t x0[L::XB];
    __shared__ __align__(16) uint8_t x1[L::XB];
    __shared__ __align__(16) uint8_t k0[L::CB];
    __shared__ __align__(16) uint8_t k1[L::CB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);              // uniform: scalar addresses
    const int r = lane & 15;      // A: row in the fragment; B: column in the fragment
    const int kq = lane >> 4;     // 8-input slot inside a 32-input MFMA step
    const int64_t rtb = (int64_t)blockIdx.x * PF_TILES;                    // first row tile of the workgroup
    const int col0 = blockIdx.y * NB * 16;
    const int64_t c0 = (int64_t)blockIdx.z * p.chunks_per_split;
    const int64_t c1 = c0 + p.chunks_per_split < p.n_chunks ? c0 + p.chunks_per_split : p.n_chunks;

    for (int i = tid; i < K * CODEWORDS; i += 64 * PF_WAVES) cb_lds[i] = p.codebooks[i];

    // Staging of chunk `ch` into (xd, kd), straight from global memory to LDS.
    // Activations: one wave instruction moves 8 columns (1 KiB); lane l takes
    // column l/8 and slot l%8 of them.  Pieces past the batch, past d_in or in
    // the padding chunk after this split are written as zeros instead
    // (ordinary LDS stores, only in ragged chunks).
    // Codes: one wave instruction moves 8 row tiles x 8 groups of one plane.
    auto stage = [&](int64_t ch, uint8_t* xd, uint8_t* kd) {
#pragma unroll
        for (int q = 0; q < 2 * NB / PF_WAVES; ++q) {
            const int blk = q * PF_WAVES + wave;                           // 8-column block
            const int col = blk * 8 + (lane >> 3);
            const int piece = (lane & 7) ^ ((col >> 1) & 7);
            const int64_t kk = ch * PF_CHUNK + piece * GROUP;
            uint8_t* dst = xd + blk * 1024;
            if (col0 + col < p.batch && kk < p.d_in && ch < c1)
                pf_dma16(p.x + (int64_t)(col0 + col) * p.d_in + kk, dst);
            else
                *reinterpret_cast<uint4*>(dst + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
        }
        const int64_t chc = ch < p.n_chunks ? ch : p.n_chunks - 1;        // the trailing padding chunk
        const int64_t jt = chc / (TILE_GROUPS / PF_CHUNK_GROUPS);
        const int g0 = (int)(chc % (TILE_GROUPS / PF_CHUNK_GROUPS)) * PF_CHUNK_GROUPS;
#pragma unroll
        for (int q = 0; q < (2 * K + PF_WAVES - 1) / PF_WAVES; ++q) {
            const int idx = q * PF_WAVES + wave;                           // (plane, half of the tiles)
            if (idx >= 2 * K) break;                                       // uniform over the wave
            const int m = idx >> 1;
            const int f = (idx & 1) * 8 + (lane >> 3);
            const int64_t rt = rtb + f < p.n_rt ? rtb + f : p.n_rt - 1;    // rows past the layer: never stored
            pf_dma16(p.packed + m * p.plane_bytes + (jt * p.n_rt + rt) * TILE_BYTES + (g0 + (lane & 7)) * TILE_ROWS,
                     kd + idx * 1024);
        }
    };

    pf_floatx4_t acc[PF_FRAGS][NB];
#pragma unroll
    for (int f = 0; f < PF_FRAGS; ++f)
#pragma unroll
        for (int t = 0; t < NB; ++t) acc[f][t] = pf_floatx4_t{0.f, 0.f, 0.f, 0.f};

    // products of chunk `ch` held in (xb, kb)
    auto compute = [&](int64_t ch, const uint8_t* xb, const uint8_t* kb) {
        const uint8_t* cw = kb + wave * PF_FRAGS * PF_CHUNK_GROUPS * TILE_ROWS + lane;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            // one 32-input step at a time: keeps the compiler from hoisting the next step's operand reads
            // (and their registers) above this step's products
            __builtin_amdgcn_sched_barrier(0);
            // this lane's group exists and belongs to this split (not the trailing padding chunk)
            // (inputs past d_in and the padding chunk already hold zero activations; the weights there are
            // zeroed too, in the rare chunks that have any, so no stray codeword meets them)
            const bool whole = ch < c1 && (ch + 1) * PF_CHUNK_GROUPS <= p.G;           // uniform
            const bool valid = ch < c1 && ch * PF_CHUNK_GROUPS + 4 * s + kq < p.G;
            pf_half8_t a[PF_FRAGS];
#pragma unroll
            for (int f = 0; f < PF_FRAGS; ++f) {
                uint32_t w[4];
#pragma unroll
                for (int m = 0; m < K; ++m) {
                    // row r, group 4s + kq of fragment f: byte (4s + kq) * 16 + r = 64 s + lane of its tile
                    const uint32_t code = cw[(m * PF_TILES + f) * PF_CHUNK_GROUPS * TILE_ROWS + 64 * s];
                    const uint4 c = cb_lds[m * CODEWORDS + code];
                    if (m == 0) {
                        w[0] = c.x; w[1] = c.y; w[2] = c.z; w[3] = c.w;
                    } else {
                        w[0] = pf_u32(pf_h2(w[0]) + pf_h2(c.x));
                        w[1] = pf_u32(pf_h2(w[1]) + pf_h2(c.y));
                        w[2] = pf_u32(pf_h2(w[2]) + pf_h2(c.z));
                        w[3] = pf_u32(pf_h2(w[3]) + pf_h2(c.w));
                    }
                }
                uint4 wv = make_uint4(w[0], w[1], w[2], w[3]);
                if (!whole && !valid) wv = make_uint4(0u, 0u, 0u, 0u);
                a[f] = __builtin_bit_cast(pf_half8_t, wv);
            }
#pragma unroll
            for (int t = 0; t < NB; ++t) {
                const uint4 bx = *reinterpret_cast<const uint4*>(xb + pf_xslot(t * 16 + r, 4 * s + kq));
                const pf_half8_t b = __builtin_bit_cast(pf_half8_t, bx);
#pragma unroll
                for (int f = 0; f < PF_FRAGS; ++f)
                    acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[f], b, acc[f][t], 0, 0, 0);
            }
        }
    };

    // Two chunks per trip: even chunks (relative to c0) live in (x0, k0), odd ones in (x1, k1), so each half
    // reads one pair of buffers while the next chunk is copied into the other.  An odd count gets one
    // trailing chunk past the input (zero activations, zero weights, clamped code addresses).  Every
    // launched split holds at least one chunk (the plan never makes an empty one).
    const int64_t c1e = c0 + ((c1 - c0 + 1) & ~(int64_t)1);
    stage(c0, x0, k0);
    int64_t ch = c0;
    do {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // this thread's copies of chunk ch have landed
        __syncthreads();                                     // ... and every thread's; (x1, k1) is free
        stage(ch + 1, x1, k1);                               // the next chunk's copies overlap these products
        compute(ch, x0, k0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();                                     // (x0, k0) is free
        if (ch + 2 < c1e) stage(ch + 2, x0, k0);
        compute(ch + 1, x1, k1);
        ch += 2;
    } while (ch < c1e);

    const int64_t rt0 = rtb + wave * PF_FRAGS;                             // first row tile of this wave
    // lane l holds rows 4*kq .. 4*kq+3 of each fragment, column t*16 + r
#pragma unroll
    for (int f = 0; f < PF_FRAGS; ++f) {
        const int64_t row0 = (rt0 + f) * TILE_ROWS + 4 * kq;
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int col = col0 + t * 16 + r;
            if (col >= p.batch || row0 >= p.d_out) continue;
            if (!p.direct) {          // one 16-byte partial per (column, row quad, split)
                store_partial(p.out, p.d_out, p.batch, blockIdx.z, col, row0,
                              make_float4(acc[f][t][0], acc[f][t][1], acc[f][t][2], acc[f][t][3]));
                continue;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t i = row0 + q;
                if (i < p.d_out) p.out[(int64_t)col * p.d_out + i] = h2f(p.scales[i]) * acc[f][t][q];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Two-phase form for large batches.  The fused kernel above rebuilds every
// weight group once per column block, with k random codeword reads from LDS
// that conflict in the bank groups; at a few column blocks and more that
// rebuild is a large share of its time.  Here the weights are rebuilt once per
// call instead:
//   1. pf_dequant_kernel writes W_k as fp16 into the workspace, in the order
//      of the packed codes with each code byte widened to the 16 bytes (8
//      halves) of its group's codeword sum.  The sum is the same packed fp16
//      add, in the same plane order, as in the fused kernel, so both forms
//      multiply the same fp16 weights.  Groups past the input get zeros.
//   2. gemm_pfw_kernel stages 16 row tiles x 64 inputs of those weights per
//      chunk into LDS with direct global-to-LDS copies, beside the
//      activations, and runs the same MFMA loop.  In the packed order a
//      tile's 8 groups of one chunk are 128 consecutive code bytes whose
//      position is exactly a lane's A slot (row r, group 4s + kq), so each
//      1 KiB copy lands as one A fragment and every operand read from LDS is
//      one conflict-free 16-byte read.
// Workgroup tile: 256 rows x 256 columns, 8 waves as 4 row groups x 2 column
// groups; a wave owns 64 rows (4 A fragments) x 128 columns (8 B fragments),
// which reads fewer operand bytes from LDS per product than 32 x 256.  (4 waves
// of 128 x 128 would read fewer still, but with 256 accumulators per wave the
// compiler moves them between register ranges every step and spills.)

constexpr int PFW_COLS = 256;                          // batch columns per workgroup
constexpr int PFW_WAVES = 8;                           // waves per workgroup
constexpr int PFW_WC = 2;                              // column groups of waves (128 columns each)
constexpr int PFW_WR = PFW_WAVES / PFW_WC;             // row groups of waves
constexpr int PFW_WAVE_FRAGS = PF_TILES / PFW_WR;      // A fragments per wave
constexpr int PFW_WAVE_COLF = PFW_COLS / 16 / PFW_WC;  // B fragments per wave (128 columns)
constexpr int PFW_MIN_BATCH = 512;                     // below this the fused kernel is faster everywhere
constexpr int64_t PFW_MAX_WEIGHT_BYTES = int64_t(1) << 31;   // largest fp16 weight kept in the workspace

static_assert(PF_TILES == 16 && PFW_WAVE_FRAGS == 4 && PFW_WAVE_COLF == 8, "two-phase tile: 64 x 128 per wave");

static int64_t pfw_weight_bytes(const Geometry& g) { return g.plane_bytes * 16; }

static int pf_nb(const Geometry& g, int batch, int k);

// The fused kernel stays where it measured faster or equal: its 256-column form at k <= 2, and at
// k = 3, 4 below 1024 columns.  The staged form takes k = 3, 4 from 1024 columns and k >= 5 (the
// fused kernel's 128-column form) from 512.
static bool pfw_used(const Geometry& g, int batch, int k) {
    if (batch < PFW_MIN_BATCH || g.plane_bytes == 0 || pfw_weight_bytes(g) > PFW_MAX_WEIGHT_BYTES) return false;
    return pf_nb(g, batch, k) == 8 || (k >= 3 && batch >= 1024);
}

// One wave pass covers 256 consecutive code bytes (a quarter of a tile, so one group tile): lane l
// takes bytes 64 j + l, j = 0..3, so each 16-byte store of the wave writes 1 KiB contiguously.
template <int K>
__global__ __launch_bounds__(256) void pf_dequant_kernel(const uint8_t* packed, const uint4* codebooks,
                                                         int64_t plane_bytes, int64_t n_rt, int64_t G, uint4* w) {
    __shared__ __align__(16) uint4 cb[K * CODEWORDS];
    for (int i = threadIdx.x; i < K * CODEWORDS; i += 256) cb[i] = codebooks[i];
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int64_t n_pass = plane_bytes / 256;
    const int64_t first = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int64_t ps = first; ps < n_pass; ps += (int64_t)gridDim.x * 4) {
        const int64_t i0 = ps * 256;
        const int64_t jt = i0 / TILE_BYTES / n_rt;                        // group tile of these bytes
        uint32_t c[4][K];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int m = 0; m < K; ++m) c[j][m] = packed[m * plane_bytes + i0 + 64 * j + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t i = i0 + 64 * j + lane;
            uint4 v = cb[c[j][0]];
#pragma unroll
            for (int m = 1; m < K; ++m) {
                const uint4 e = cb[m * CODEWORDS + c[j][m]];
                v.x = pf_u32(pf_h2(v.x) + pf_h2(e.x));
                v.y = pf_u32(pf_h2(v.y) + pf_h2(e.y));
                v.z = pf_u32(pf_h2(v.z) + pf_h2(e.z));
                v.w = pf_u32(pf_h2(v.w) + pf_h2(e.w));
            }
            if (jt * TILE_GROUPS + (i % TILE_BYTES) / TILE_ROWS >= G) v = make_uint4(0u, 0u, 0u, 0u);
            w[i] = v;
        }
    }
}

struct PfwArgs {
    const uint4* w;            // fp16 weights from pf_dequant_kernel
    const uint16_t* scales;
    const uint16_t* x;
    float* out;
    int64_t d_out, d_in, n_rt, n_chunks;
    int batch, chunks_per_split, direct;
};

__global__ __launch_bounds__(64 * PFW_WAVES, PFW_WAVES / 4) void gemm_pfw_kernel(PfwArgs p) {
    constexpr int XB = PFW_COLS * PF_CHUNK * 2;                           // 256 columns x 128 B
    constexpr int AB = PF_TILES * 2 * 1024;                               // 16 tiles x 2 fragments
    __shared__ __align__(16) uint8_t x0[XB];
    __shared__ __align__(16) uint8_t x1[XB];
    __shared__ __align__(16) uint8_t a0[AB];
    __shared__ __align__(16) uint8_t a1[AB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);              // uniform: scalar addresses
    const int r = lane & 15;
    const int kq = lane >> 4;
    const int wr = wave % PFW_WR;                                          // row group of the wave
    const int wc = wave / PFW_WR;                                          // column group: 128 columns
    const int64_t rtb = (int64_t)blockIdx.x * PF_TILES;
    const int col0 = blockIdx.y * PFW_COLS;
    const int64_t c0 = (int64_t)blockIdx.z * p.chunks_per_split;
    const int64_t c1 = c0 + p.chunks_per_split < p.n_chunks ? c0 + p.chunks_per_split : p.n_chunks;

    // Chunk `ch` into (xd, ad).  Activations as in the fused kernel (4 blocks of 8 columns per wave);
    // weights: 32 copies of 1 KiB, fragment idx = (row tile f, half h) at ad + idx * 1 KiB.  The
    // padding chunk after the split gets zeros on both sides.
    auto stage = [&](int64_t ch, uint8_t* xd, uint8_t* ad) {
#pragma unroll
        for (int q = 0; q < PFW_COLS / 8 / PFW_WAVES; ++q) {
            const int blk = q * PFW_WAVES + wave;
            const int col = blk * 8 + (lane >> 3);
            const int piece = (lane & 7) ^ ((col >> 1) & 7);
            const int64_t kk = ch * PF_CHUNK + piece * GROUP;
            uint8_t* dst = xd + blk * 1024;
            if (col0 + col < p.batch && kk < p.d_in && ch < c1)
                pf_dma16(p.x + (int64_t)(col0 + col) * p.d_in + kk, dst);
            else
                *reinterpret_cast<uint4*>(dst + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
        }
        const int64_t chc = ch < p.n_chunks ? ch : p.n_chunks - 1;
        const int64_t jt = chc / (TILE_GROUPS / PF_CHUNK_GROUPS);
        const int g0 = (int)(chc % (TILE_GROUPS / PF_CHUNK_GROUPS)) * PF_CHUNK_GROUPS;
#pragma unroll
        for (int q = 0; q < 2 * PF_TILES / PFW_WAVES; ++q) {
            const int idx = q * PFW_WAVES + wave;
            const int f = idx >> 1;
            const int h = idx & 1;
            uint8_t* dst = ad + idx * 1024;
            const int64_t rt = rtb + f < p.n_rt ? rtb + f : p.n_rt - 1;    // rows past the layer: never stored
            if (ch < c1)
                pf_dma16(p.w + (jt * p.n_rt + rt) * TILE_BYTES + g0 * TILE_ROWS + h * 64 + lane, dst);
            else
                *reinterpret_cast<uint4*>(dst + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
        }
    };

    pf_floatx4_t acc[PFW_WAVE_FRAGS][PFW_WAVE_COLF];
#pragma unroll
    for (int f = 0; f < PFW_WAVE_FRAGS; ++f)
#pragma unroll
        for (int t = 0; t < PFW_WAVE_COLF; ++t) acc[f][t] = pf_floatx4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const uint8_t* xb, const uint8_t* ab) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            pf_half8_t a[PFW_WAVE_FRAGS];
#pragma unroll
            for (int f = 0; f < PFW_WAVE_FRAGS; ++f)
                a[f] = __builtin_bit_cast(pf_half8_t,
                                          *reinterpret_cast<const uint4*>(ab + ((wr * PFW_WAVE_FRAGS + f) * 2 + s) * 1024 + lane * 16));
#pragma unroll
            for (int t = 0; t < PFW_WAVE_COLF; ++t) {
                const uint4 bx = *reinterpret_cast<const uint4*>(xb + pf_xslot(wc * 128 + t * 16 + r, 4 * s + kq));
                const pf_half8_t b = __builtin_bit_cast(pf_half8_t, bx);
#pragma unroll
                for (int f = 0; f < PFW_WAVE_FRAGS; ++f)
                    acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[f], b, acc[f][t], 0, 0, 0);
            }
        }
    };

    const int64_t c1e = c0 + ((c1 - c0 + 1) & ~(int64_t)1);
    stage(c0, x0, a0);
    int64_t ch = c0;
    do {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        stage(ch + 1, x1, a1);
        compute(x0, a0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (ch + 2 < c1e) stage(ch + 2, x0, a0);
        compute(x1, a1);
        ch += 2;
    } while (ch < c1e);

#pragma unroll
    for (int f = 0; f < PFW_WAVE_FRAGS; ++f) {
        const int64_t row0 = (rtb + wr * PFW_WAVE_FRAGS + f) * TILE_ROWS + 4 * kq;
#pragma unroll
        for (int t = 0; t < PFW_WAVE_COLF; ++t) {
            const int col = col0 + wc * 128 + t * 16 + r;
            if (col >= p.batch || row0 >= p.d_out) continue;
            if (!p.direct) {
                store_partial(p.out, p.d_out, p.batch, blockIdx.z, col, row0,
                              make_float4(acc[f][t][0], acc[f][t][1], acc[f][t][2], acc[f][t][3]));
                continue;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t i = row0 + q;
                if (i < p.d_out) p.out[(int64_t)col * p.d_out + i] = h2f(p.scales[i]) * acc[f][t][q];
            }
        }
    }
}

// B fragments per wave (16 batch columns each).  128 columns by default; 256 where
// they measured faster (k <= 4: more codebooks would spill; batch >= 512, or
// >= 256 over a short input dimension, whose split reduce is small), which
// doubles the accumulators and halves the codeword gathers per product.
static int pf_nb(const Geometry& g, int batch, int k) {
    return k <= 4 && (batch >= 512 || (batch >= 256 && g.d_in < 8192)) ? 16 : 8;
}

struct PfPlan {
    int64_t n_chunks, row_blocks, col_blocks;
    int splits, chunks_per_split;
};

// Splits of the input dimension, only when the tiles do not cover the 256
// compute units: the smallest split count that minimises (rounds of workgroups
// over the chip) x (chunks per split) plus the reduce of the partials, at most
// PF_MAX_SPLITS.  The reduce reads `splits` fp32 copies of Y and writes one; it
// is charged in chunk times (a 64-input chunk of a 256-row tile takes about
// 2 us, in which HBM moves about 8 MB).
static PfPlan pf_plan(const Geometry& g, int batch, int cols) {
    PfPlan p;
    p.n_chunks = (g.d_in + PF_CHUNK - 1) / PF_CHUNK;
    p.row_blocks = (g.n_rt + PF_TILES - 1) / PF_TILES;
    p.col_blocks = (batch + cols - 1) / cols;
    p.splits = 1;
    p.chunks_per_split = (int)p.n_chunks;
    const int64_t tiles = p.row_blocks * p.col_blocks;
    if (tiles == 0 || p.n_chunks == 0) return p;
    // Tiles that cover the chip on their own are not split: the reduce of the partials (a full fp32
    // copy of Y per split, read back) costs more than the last round's idle CUs.
    if (tiles >= 256 * PF_PER_CU) return p;
    constexpr double CHUNK_BYTES = 8e6;
    const double y_bytes = 4.0 * (double)batch * (double)g.d_out;
    double best = -1;
    for (int64_t sp = 1; sp <= PF_MAX_SPLITS && sp <= p.n_chunks; ++sp) {
        const int64_t cps = (p.n_chunks + sp - 1) / sp;
        const int64_t used = (p.n_chunks + cps - 1) / cps;
        const double cost = (double)(((tiles * used + 256 * PF_PER_CU - 1) / (256 * PF_PER_CU)) * cps) +
                            (used > 1 ? (double)(used + 1) * y_bytes / CHUNK_BYTES : 0.0);
        if (best < 0 || cost < best) {
            best = cost;
            p.splits = (int)used;
            p.chunks_per_split = (int)cps;
        }
    }
    return p;
}

// Two-phase workspace: the split partials (if any), then the fp16 weights at the next 256-byte boundary.
static size_t pfw_weight_offset(const Geometry& g, int batch) {
    const PfPlan p = pf_plan(g, batch, PFW_COLS);
    const size_t b = p.splits > 1 ? partial_bytes(g.d_out, batch, p.splits) : 0;
    return (b + 255) & ~(size_t)255;
}

size_t gemm_pf_workspace_bytes(const Geometry& g, int batch) {
    size_t need = 0;                                   // the largest over k
    for (int k = 1; k <= g.M && k <= MAX_M; ++k) {
        const PfPlan p = pf_plan(g, batch, pf_nb(g, batch, k) * 16);
        const size_t b = pfw_used(g, batch, k) ? pfw_weight_offset(g, batch) + (size_t)pfw_weight_bytes(g)
                         : p.splits > 1 ? partial_bytes(g.d_out, batch, p.splits)
                                        : 0;
        need = b > need ? b : need;
    }
    return need;
}

template <int K, int NB>
static hipError_t launch_pf(const PfArgs& a, const PfPlan& pl, hipStream_t s) {
    hipLaunchKernelGGL((gemm_pf_kernel<K, NB>),
                       dim3((unsigned)pl.row_blocks, (unsigned)pl.col_blocks, (unsigned)pl.splits),
                       dim3(64 * PF_WAVES), 0, s, a);
    return hipGetLastError();
}

template <int NB>
static hipError_t launch_pf_k(int k, const PfArgs& a, const PfPlan& pl, hipStream_t s) {
    switch (k) {
        case 1: return launch_pf<1, NB>(a, pl, s);
        case 2: return launch_pf<2, NB>(a, pl, s);
        case 3: return launch_pf<3, NB>(a, pl, s);
        case 4: return launch_pf<4, NB>(a, pl, s);
        case 5: return launch_pf<5, NB>(a, pl, s);
        case 6: return launch_pf<6, NB>(a, pl, s);
        case 7: return launch_pf<7, NB>(a, pl, s);
        default: return launch_pf<8, NB>(a, pl, s);
    }
}

template <int K>
static hipError_t launch_dequant(const uint8_t* packed, const uint16_t* codebooks, const Geometry& g, uint4* w,
                                 hipStream_t s) {
    const int64_t n_pass = g.plane_bytes / 256;
    const int64_t blocks = (n_pass + 3) / 4 < 2048 ? (n_pass + 3) / 4 : 2048;
    hipLaunchKernelGGL((pf_dequant_kernel<K>), dim3((unsigned)blocks), dim3(256), 0, s, packed,
                       reinterpret_cast<const uint4*>(codebooks), g.plane_bytes, g.n_rt, g.G, w);
    return hipGetLastError();
}

static hipError_t launch_gemm_pfw(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                                  const uint16_t* x, float* y, int batch, const Geometry& g, void* ws,
                                  hipStream_t s) {
    const PfPlan pl = pf_plan(g, batch, PFW_COLS);
    uint4* w = reinterpret_cast<uint4*>(static_cast<uint8_t*>(ws) + pfw_weight_offset(g, batch));
    hipError_t e;
    switch (k) {
        case 1: e = launch_dequant<1>(packed, codebooks, g, w, s); break;
        case 2: e = launch_dequant<2>(packed, codebooks, g, w, s); break;
        case 3: e = launch_dequant<3>(packed, codebooks, g, w, s); break;
        case 4: e = launch_dequant<4>(packed, codebooks, g, w, s); break;
        case 5: e = launch_dequant<5>(packed, codebooks, g, w, s); break;
        case 6: e = launch_dequant<6>(packed, codebooks, g, w, s); break;
        case 7: e = launch_dequant<7>(packed, codebooks, g, w, s); break;
        default: e = launch_dequant<8>(packed, codebooks, g, w, s); break;
    }
    if (e != hipSuccess) return e;
    PfwArgs a;
    a.w = w;
    a.scales = scales;
    a.x = x;
    a.direct = pl.splits == 1 ? 1 : 0;
    a.out = a.direct ? y : static_cast<float*>(ws);
    a.d_out = g.d_out;
    a.d_in = g.d_in;
    a.n_rt = g.n_rt;
    a.n_chunks = pl.n_chunks;
    a.batch = batch;
    a.chunks_per_split = pl.chunks_per_split;
    hipLaunchKernelGGL(gemm_pfw_kernel, dim3((unsigned)pl.row_blocks, (unsigned)pl.col_blocks, (unsigned)pl.splits),
                       dim3(64 * PFW_WAVES), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.direct) return e;
    return launch_split_reduce(static_cast<const float*>(ws), scales, y, g.d_out, batch, pl.splits, s);
}

hipError_t launch_gemm_pf(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                          const uint16_t* x, float* y, int batch, const Geometry& g, void* ws, hipStream_t s) {
    const PfPlan pl = pf_plan(g, batch, pf_nb(g, batch, k) * 16);
    if (pl.n_chunks == 0) return launch_zero_f32(y, (int64_t)batch * g.d_out, s);   // empty input: Y = 0
    if (pfw_used(g, batch, k)) return launch_gemm_pfw(packed, codebooks, scales, k, x, y, batch, g, ws, s);
    PfArgs a;
    a.packed = packed;
    a.codebooks = reinterpret_cast<const uint4*>(codebooks);
    a.scales = scales;
    a.x = x;
    a.direct = pl.splits == 1 ? 1 : 0;
    a.out = a.direct ? y : static_cast<float*>(ws);
    a.d_out = g.d_out;
    a.d_in = g.d_in;
    a.G = g.G;
    a.n_rt = g.n_rt;
    a.plane_bytes = g.plane_bytes;
    a.n_chunks = pl.n_chunks;
    a.batch = batch;
    a.chunks_per_split = pl.chunks_per_split;
    const hipError_t e = pf_nb(g, batch, k) == 16 ? launch_pf_k<16>(k, a, pl, s) : launch_pf_k<8>(k, a, pl, s);
    if (e != hipSuccess || a.direct) return e;
    return launch_split_reduce(static_cast<const float*>(ws), scales, y, g.d_out, batch, pl.splits, s);
}

}  // namespace aqd
