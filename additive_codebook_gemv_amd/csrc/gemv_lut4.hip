// Decode GEMV for three or four activation columns through per-group lookup
// tables.
//
// Drop-by-Drop ("Multi-Bitwidth Quantization for LLMs Using Additive
// Codebooks"), section 3.2 and section 5: row i of column n is
//     sum_{j} sum_{m<k} T_{m,j,n}[code(i,j,m)],   T_{m,j,n}[c] = < C_m[c], xrot_n[8j .. 8j+8) >.
// All columns look up the same code, so the tables of one (group, codebook)
// hold four fp16 entries per codeword: entry (codeword c, lane l) is the
// quadruple (column 0..3) at byte c*512 + l*8 of a 128 KiB LDS array, one slot
// (64 groups of one codebook plane) per workgroup.  One conflict-free 8-byte
// read per code byte returns the four columns' entries; its address is the
// code byte moved into place by one v_perm_b32 and doubled.
//
// Row sums on the matrix cores, as at batch 2: the two 8-byte reads of rows
// 4q + 2p and 4q + 2p + 1 are the B operand (half h = 4 (m - 2p) + column) of a
// v_mfma_f32_16x16x32_f16 whose 0/1 A operand (lut_route2(p)) sends half h to
// output row 8p + h, i.e. (row 4q + m, column) to output row 4m + column of
// accumulator q.  Four accumulators hold the 64 (row, column) sums of a tile;
// the batch-1 butterfly over the remaining 16 lanes leaves output row i of
// accumulator a in lanes 4i .. 4i+3, and lane 4i + a adds it through the
// counted fixed-point word of its (column, row) (batch 1): one atomic
// instruction per tile serves all 64 sums.  With three columns the fourth is
// computed from a zero activation and not stored.  The reads of a product go
// out two products ahead (a software pipeline held in order by scheduling
// barriers), as in the batch-1 kernel.
#include "lut_device.h"

namespace aqd {

constexpr int LUT4_COLS = 4;
constexpr int LUT4_ENTRY = 8;                 // bytes per (codeword, lane): four fp16
// Where the route pays (measured against the matrix-core and codeword-gather
// kernels, both MLP shapes and 4096x4096, batch 3 and 4): k <= 2 and at most
// 32 slots.  Beyond that every (column, row) word takes so many contributions
// that the other kernels are faster.
constexpr int LUT4_MAX_K = 2;
constexpr int64_t LUT4_MAX_SLOTS = 32;

struct Lut4Args {
    const uint8_t* packed;
    const uint16_t* codebooks;
    const uint16_t* scales;
    const uint16_t* x;          // [batch][d_in] rotated activation, fp16
    uint16_t* y;                // [batch][d_out] fp16
    unsigned long long* acc;    // workspace: [4][d_out] counted fixed-point row sums, zero between calls
    int64_t d_out, d_in, G, n_gt, n_rt, plane_bytes;
    int k, batch, n_slots, tiles_per_block;
};

template <int K, int TPW, int W = LUT_WAVES>
__global__ __launch_bounds__(64 * W) void gemv_lut4_kernel(Lut4Args p) {
    __shared__ __align__(16) uint8_t lds[CODEWORDS * 64 * LUT4_ENTRY];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int slice = (int)blockIdx.x % p.n_slots;           // one slot per workgroup
    const int rb = (int)blockIdx.x / p.n_slots;
    const int64_t t0 = (int64_t)rb * p.tiles_per_block;
    const int64_t t1 = t0 + p.tiles_per_block < p.n_rt ? t0 + p.tiles_per_block : p.n_rt;
    const int gt = slice / K, plane = slice % K;               // group tile and codebook of the slot
    const __amdgpu_buffer_rsrc_t slot_buf =
        slot_rsrc(p.packed + (int64_t)plane * p.plane_bytes + (int64_t)gt * p.n_rt * TILE_BYTES, p.n_rt * TILE_BYTES);

    // ---- table operands.  Item i (16 of them, 16 / W per wave: item wave + u * W) builds codewords
    // 32*(i >> 1) .. +32 for groups 32*(i & 1) .. +32; its four products are the four columns.
    constexpr int IW = 16 / W;
    static_assert(IW * W == 16, "table items per wave");
    const int e0 = 4 * (lane >> 5);
    uint2 av[IW], bv[IW][LUT4_COLS];
    bool gok[IW];
#pragma unroll
    for (int u = 0; u < IW; ++u) {
        const int item = wave + u * W;
        const int cb = item >> 1, gb = item & 1;
        const int64_t g = (int64_t)gt * TILE_GROUPS + gb * 32 + (lane & 31);
        gok[u] = g < p.G;
        const int64_t gc = gok[u] ? g : p.G - 1;
        av[u] = *reinterpret_cast<const uint2*>(p.codebooks + ((int64_t)plane * CODEWORDS + cb * 32 + (lane & 31)) *
                                                                  GROUP + e0);
#pragma unroll
        for (int c = 0; c < LUT4_COLS; ++c) {
            const int cc = c < p.batch ? c : p.batch - 1;
            bv[u][c] = *reinterpret_cast<const uint2*>(p.x + cc * p.d_in + gc * GROUP + e0);
        }
    }
    // operand loads of every wave go out before any code load (see the batch-1 kernel)
    __builtin_amdgcn_s_barrier();

    uint4 codes[TPW];
    auto load_tile = [&](int u) {
        const int64_t it = t0 + wave + (int64_t)u * W;
        codes[u] = load_stream(slot_buf, it < t1 ? (uint32_t)(it * TILE_BYTES) + lane * TILE_ROWS : NO_TILE);
    };
    load_tile(0);
    // this lane's sum after the butterflies: accumulator a = lane & 3 (rows 4a .. 4a+3), output row
    // i = (lane >> 2) & 15, i.e. tile row 4a + (i >> 2), column i & 3
    const int oi = (lane >> 2) & 15;
    const int acc_q = lane & 3;
    const int col = oi & 3;
    const int trow = 4 * acc_q + (oi >> 2);
    uint16_t row_scale[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int64_t row = (t0 + wave + (int64_t)u * W) * TILE_ROWS + trow;
        row_scale[u] = p.scales[row < p.d_out ? row : p.d_out - 1];
    }
#pragma unroll
    for (int u = 0; u < IW; ++u)
#pragma unroll
        for (int c = 0; c < LUT4_COLS; ++c)
            if (!gok[u] || c >= p.batch) bv[u][c] = make_uint2(0u, 0u);   // zero activation -> zero entries

#pragma unroll
    for (int u = 0; u < IW; ++u) {
        const int item = wave + u * W;
        const int cb = item >> 1, gb = item & 1;
        floatx16_t t[LUT4_COLS];
#pragma unroll
        for (int c = 0; c < LUT4_COLS; ++c) {
#pragma unroll
            for (int r = 0; r < 16; ++r) t[c][r] = 0.f;
            t[c] = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(half4_t, av[u]),
                                                        __builtin_bit_cast(half4_t, bv[u][c]), t[c], 0, 0, 0);
        }
        const int gl = gb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = cb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const half2_t lo = half2_t{(_Float16)t[0][r], (_Float16)t[1][r]};
            const half2_t hi = half2_t{(_Float16)t[2][r], (_Float16)t[3][r]};
            *reinterpret_cast<uint2*>(lds + c * (64 * LUT4_ENTRY) + gl * LUT4_ENTRY) =
                make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 1; u < TPW; ++u) load_tile(u);

    const uint32_t base = (uint32_t)(lane * 4);              // halved: the address is doubled after the v_perm
    half8_t route[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) route[h] = lut_route2(h, lane);

    unsigned long long old_word[TPW], term[TPW];
    bool mine[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        mine[u] = false;
        old_word[u] = 0ull;
        term[u] = 0ull;
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int64_t it = t0 + wave + (int64_t)u * W;
        if (it >= t1) break;                    // uniform across the wave
        floatx4_t d[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) d[q] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        // (q, pr) pairs: the (column 0..3) entries of rows 4q + 2pr and 4q + 2pr + 1; pair n + 2's reads
        // go out before pair n's product
        auto read_pair = [&](int n, uint4& v) {
            const int q = n >> 1, pr = n & 1;
            const uint32_t w = q == 0 ? codes[u].x : q == 1 ? codes[u].y : q == 2 ? codes[u].z : codes[u].w;
            const uint2 e = *reinterpret_cast<const uint2*>(lds + 2 * lut_addr(w, base, 2 * pr));
            const uint2 f = *reinterpret_cast<const uint2*>(lds + 2 * lut_addr(w, base, 2 * pr + 1));
            v = make_uint4(e.x, e.y, f.x, f.y);
        };
        constexpr int NP = 8, LA = 2;
        uint4 ev[LA + 1];
#pragma unroll
        for (int n = 0; n < LA; ++n) read_pair(n, ev[n]);
#pragma unroll
        for (int n = 0; n < NP; ++n) {
            if (n + LA < NP) read_pair(n + LA, ev[(n + LA) % (LA + 1)]);
            __builtin_amdgcn_sched_barrier(0);
            d[n >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(route[n & 1], __builtin_bit_cast(half8_t, ev[n % (LA + 1)]),
                                                               d[n >> 1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        float sq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) sq[q] = fold_quads(d[q], lane);
        const float sum = acc_q == 0 ? sq[0] : acc_q == 1 ? sq[1] : acc_q == 2 ? sq[2] : sq[3];
        const int64_t row = it * TILE_ROWS + trow;
        if (col < p.batch && row < p.d_out) {
            mine[u] = true;
            term[u] = fix_term(sum);
            old_word[u] = atomicAdd(p.acc + col * p.d_out + row, fix_add_word(term[u]));
        }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        if (!mine[u] || !fix_is_last(old_word[u], p.n_slots)) continue;
        const int64_t row = (t0 + wave + (int64_t)u * W) * TILE_ROWS + trow;
        p.y[col * p.d_out + row] = f2h(h2f(row_scale[u]) * (float)fix_total(old_word[u], term[u], p.n_slots));
        __hip_atomic_store(p.acc + col * p.d_out + row, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---- host side ---------------------------------------------------------------

size_t gemv_lut4_workspace_bytes(const Geometry& g) { return ((size_t)g.d_out * LUT4_COLS * 8 + 255) / 256 * 256; }

bool gemv_lut4_supported(const Geometry& g, int batch, int k) {
    return (batch == 3 || batch == 4) && k <= LUT4_MAX_K && g.n_gt > 0 && g.n_rt > 0 &&
           g.n_rt <= LUT_MAX_ROW_TILES && (int64_t)k * g.n_gt <= LUT4_MAX_SLOTS;
}

template <int TPW>
static void launch_lut4_k(int k, dim3 gd, dim3 bd, hipStream_t s, const Lut4Args& a) {
    if (k == 1) hipLaunchKernelGGL((gemv_lut4_kernel<1, TPW>), gd, bd, 0, s, a);
    else hipLaunchKernelGGL((gemv_lut4_kernel<2, TPW>), gd, bd, 0, s, a);
}

hipError_t launch_gemv_lut4(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                            const uint16_t* x, uint16_t* y, int batch, const Geometry& g, void* ws, hipStream_t s) {
    if (k > LUT4_MAX_K) return hipErrorInvalidValue;
    Lut4Args a = {};
    a.packed = packed;
    a.codebooks = codebooks;
    a.scales = scales;
    a.x = x;
    a.y = y;
    a.acc = static_cast<unsigned long long*>(ws);
    a.d_out = g.d_out;
    a.d_in = g.d_in;
    a.G = g.G;
    a.n_gt = g.n_gt;
    a.n_rt = g.n_rt;
    a.plane_bytes = g.plane_bytes;
    a.k = k;
    a.batch = batch;
    a.n_slots = (int)((int64_t)k * g.n_gt);
    // two row tiles per wave, or four when two would need a second round of workgroups
    int tpw = LUT_TILES_PER_WAVE, tpb = 0, blocks = 0;
    lut_plan(&g.n_rt, 1, a.n_slots, tpw, &tpb, &blocks);
    if ((int64_t)a.n_slots * blocks > LUT_CUS) {
        tpw = LUT_TILES_PER_WAVE_BIG;
        lut_plan(&g.n_rt, 1, a.n_slots, tpw, &tpb, &blocks);
    }
    a.tiles_per_block = tpb;
    const dim3 gd((unsigned)(a.n_slots * blocks)), bd(64 * LUT_WAVES);
    // plans of at most 8 row tiles per workgroup run in 8-wave workgroups (two table items per wave): the
    // same tiles, sums and bits (4096x4096 batch 4, k = 1: 5.25 -> 4.87 us; 1024 and 2048 rows 5-9 % faster)
    if (tpw == LUT_TILES_PER_WAVE && tpb <= LUT_WAVES_SMALL) {
        const dim3 bd8(64 * LUT_WAVES_SMALL);
        if (k == 1) hipLaunchKernelGGL((gemv_lut4_kernel<1, LUT_TILES_PER_WAVE, LUT_WAVES_SMALL>), gd, bd8, 0, s, a);
        else hipLaunchKernelGGL((gemv_lut4_kernel<2, LUT_TILES_PER_WAVE, LUT_WAVES_SMALL>), gd, bd8, 0, s, a);
        return hipGetLastError();
    }
    if (tpw == LUT_TILES_PER_WAVE_BIG) launch_lut4_k<LUT_TILES_PER_WAVE_BIG>(k, gd, bd, s, a);
    else launch_lut4_k<LUT_TILES_PER_WAVE>(k, gd, bd, s, a);
    return hipGetLastError();
}

}  // namespace aqd
