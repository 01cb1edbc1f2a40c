// Decode GEMV for two activation columns through per-group lookup tables.
//
// Drop-by-Drop ("Multi-Bitwidth Quantization for LLMs Using Additive
// Codebooks"), section 3.2 and section 5: row i of column n is
//     sum_{j} sum_{m<k} T_{m,j,n}[code(i,j,m)],   T_{m,j,n}[c] = < C_m[c], xrot_n[8j .. 8j+8) >.
// At batch 2 each (group, codebook) has one 256-entry table per column, and
// both columns look up the same code.
//
// This is the batch-1 lookup-table kernel with the second column in place of
// the second slot of a pair.  Entry (slot s, codeword c, lane l) is the fp16
// pair (column 0, column 1) at byte
//     s*64K + c*256 + l*4,
// so one conflict-free dword read per code byte returns both columns' entries,
// and the address is the same single v_perm_b32 of the code dword.  A
// workgroup holds 2 slots (128 KiB of tables) instead of 4, so a launch has
// twice as many slices as at batch 1.  The tables are built with the same
// matrix-core product (32 codewords x 8 elements times 8 elements x 32
// groups), one product per column.
//
// Per code byte a lane spends one address and one LDS read.  The four dwords
// read for rows 4q .. 4q+3 of one slot (both columns each) are the B operand
// of one v_mfma_f32_16x16x32_f16 whose 0/1 A operand routes half h of quad q
// to output row 8(q mod 2) + h (lut_route2): two accumulators, for quads 0-1
// and 2-3, collect the sums over slots and over four lanes at a time in fp32,
// and the batch-1 butterfly over the remaining 16 lanes (fold_quads) leaves
// output row (l >> 2) of each accumulator in lane l.  Row sums of both columns
// leave through the counted fixed-point words of batch 1 (one word per column
// and row): lane 4i adds output row i of the first accumulator and lane 4i+1
// that of the second, so one atomic instruction serves all 32 (row, column)
// sums of a tile.
#include "lut_device.h"

namespace aqd {

constexpr int LUT2_SLOTS = 2;  // slots per workgroup; each 64 KiB region holds both columns

struct Lut2Args {
    const uint8_t* packed;
    const uint16_t* codebooks;
    const uint16_t* scales;
    const uint16_t* x;          // [2][d_in] rotated activation, fp16
    uint16_t* y;                // [2][d_out] fp16
    unsigned long long* acc;    // workspace: [2][d_out] counted fixed-point row sums, zero between calls
    int64_t d_out, d_in, G, n_gt, n_rt, plane_bytes;
    int k, n_slots, slices, tiles_per_block;
};

template <int K, int TPW, int W = LUT_WAVES>
__global__ __launch_bounds__(64 * W) void gemv_lut2_kernel(Lut2Args p) {
    __shared__ __align__(16) uint8_t lds[LUT_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int slice = (int)blockIdx.x % p.slices;
    const int rb = (int)blockIdx.x / p.slices;
    const int64_t t0 = (int64_t)rb * p.tiles_per_block;
    const int64_t t1 = t0 + p.tiles_per_block < p.n_rt ? t0 + p.tiles_per_block : p.n_rt;

    // slot s of this slice: q = slice*2 + s -> group tile q / K, codebook q % K.
    // As at batch 1, every load is unconditional; inactive slots, padding
    // groups and missing tiles read a valid address and their value is zeroed.
    __amdgpu_buffer_rsrc_t slot_buf[LUT2_SLOTS];
    bool slot_on[LUT2_SLOTS];
#pragma unroll
    for (int s = 0; s < LUT2_SLOTS; ++s) {
        const int q = slice * LUT2_SLOTS + s;
        slot_on[s] = q < p.n_slots;
        const int qq = slot_on[s] ? q : 0;
        slot_buf[s] = slot_rsrc(p.packed + (int64_t)(qq % K) * p.plane_bytes + (int64_t)(qq / K) * p.n_rt * TILE_BYTES,
                                p.n_rt * TILE_BYTES);
    }

    // ---- table operands.  Item = (slot, block of 32 codewords, block of 32
    // groups); its two products are the two columns.
    constexpr int ITEMS = 32 / W;
    uint2 av[ITEMS], bv[ITEMS][2];
    bool bok[ITEMS];
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
        const int item = wave + u * W;
        const int s = item >> 4, cb = (item >> 1) & 7, gb = item & 1;
        const int q = slice * LUT2_SLOTS + s;
        const int qq = q < p.n_slots ? q : 0;
        const int e0 = 4 * (lane >> 5);
        const int c = cb * 32 + (lane & 31);
        const int64_t g = (int64_t)(qq / K) * TILE_GROUPS + gb * 32 + (lane & 31);
        bok[u] = q < p.n_slots && g < p.G;
        const int64_t gc = g < p.G ? g : p.G - 1;
        av[u] = *reinterpret_cast<const uint2*>(p.codebooks + ((int64_t)(qq % K) * CODEWORDS + c) * GROUP + e0);
#pragma unroll
        for (int h = 0; h < 2; ++h) bv[u][h] = *reinterpret_cast<const uint2*>(p.x + h * p.d_in + gc * GROUP + e0);
    }
    // operand loads of every wave go out before any code load (see the batch-1 kernel)
    __builtin_amdgcn_s_barrier();

    uint4 codes[TPW][LUT2_SLOTS];
    auto load_tile = [&](int u) {
        const int64_t it = t0 + wave + (int64_t)u * W;
        const uint32_t off = it < t1 ? (uint32_t)(it * TILE_BYTES) + lane * TILE_ROWS : NO_TILE;
#pragma unroll
        for (int s = 0; s < LUT2_SLOTS; ++s) codes[u][s] = load_stream(slot_buf[s], slot_on[s] ? off : NO_TILE);
    };
    load_tile(0);
    uint16_t row_scale[TPW];
    {
        const int oi_ = (lane >> 2) & 15;
        const int trow_ = ((lane & 3) == 1 ? 8 : 0) + 4 * (oi_ >> 3) + ((oi_ >> 1) & 3);
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int64_t row = (t0 + wave + (int64_t)u * W) * TILE_ROWS + trow_;
            row_scale[u] = p.scales[row < p.d_out ? row : p.d_out - 1];
        }
    }
#pragma unroll
    for (int u = 0; u < ITEMS; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            if (!bok[u]) bv[u][h] = make_uint2(0u, 0u);      // zero activation -> zero table entries

#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
        const int item = wave + u * W;
        const int s = item >> 4, cb = (item >> 1) & 7, gb = item & 1;
        floatx16_t t[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int r = 0; r < 16; ++r) t[h][r] = 0.f;
            t[h] = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(half4_t, av[u]),
                                                        __builtin_bit_cast(half4_t, bv[u][h]), t[h], 0, 0, 0);
        }
        const int gl = gb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = cb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const half2_t v = half2_t{(_Float16)t[0][r], (_Float16)t[1][r]};
            *reinterpret_cast<half2_t*>(lds + s * LUT_PAIR_BYTES + c * 256 + gl * 4) = v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 1; u < TPW; ++u) load_tile(u);

    uint32_t base[LUT2_SLOTS];
#pragma unroll
    for (int s = 0; s < LUT2_SLOTS; ++s) base[s] = (uint32_t)(lane * 4) | ((uint32_t)s << 16);
    half8_t route[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) route[h] = lut_route2(h, lane);
    // after the butterflies lane l holds output row i = (l >> 2) & 15 of both accumulators; lane 4i
    // adds the first one's (quads 0-1), lane 4i + 1 the second one's (quads 2-3)
    const int oi = (lane >> 2) & 15;
    const int part = lane & 3;
    const int col = oi & 1;                                                // column of output row i
    const int trow = (part == 1 ? 8 : 0) + 4 * (oi >> 3) + ((oi >> 1) & 3); // tile row of this lane's sum

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
        floatx4_t d[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int s = 0; s < LUT2_SLOTS; ++s) {
                const uint4& c = codes[u][s];
                const uint32_t w = q == 0 ? c.x : q == 1 ? c.y : q == 2 ? c.z : c.w;
                uint32_t e[4];                  // (column 0, column 1) entries of rows 4q .. 4q+3
#pragma unroll
                for (int m = 0; m < 4; ++m) e[m] = *reinterpret_cast<const uint32_t*>(lds + lut_addr(w, base[s], m));
                d[q >> 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    route[q & 1], __builtin_bit_cast(half8_t, make_uint4(e[0], e[1], e[2], e[3])), d[q >> 1], 0, 0, 0);
            }
        }
        const float s0 = fold_quads(d[0], lane);
        const float s1 = fold_quads(d[1], lane);
        const int64_t row = it * TILE_ROWS + trow;
        if (part < 2 && row < p.d_out) {
            mine[u] = true;
            term[u] = fix_term(part == 0 ? s0 : s1);
            old_word[u] = atomicAdd(p.acc + col * p.d_out + row, fix_add_word(term[u]));
        }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        if (!mine[u] || !fix_is_last(old_word[u], p.slices)) continue;
        const int64_t row = (t0 + wave + (int64_t)u * W) * TILE_ROWS + trow;
        p.y[col * p.d_out + row] = f2h(h2f(row_scale[u]) * (float)fix_total(old_word[u], term[u], p.slices));
        __hip_atomic_store(p.acc + col * p.d_out + row, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---- host side ---------------------------------------------------------------

size_t gemv_lut2_workspace_bytes(const Geometry& g) { return ((size_t)g.d_out * 2 * 8 + 255) / 256 * 256; }

bool gemv_lut2_supported(const Geometry& g, int batch, int k) {
    return batch == 2 && g.n_gt > 0 && g.n_rt > 0 && g.n_rt <= LUT_MAX_ROW_TILES &&
           lut_slices(g.n_gt, k, LUT2_SLOTS) <= LUT_MAX_SLICES;
}

template <int TPW>
static void launch_lut2_k(int k, dim3 gd, dim3 bd, hipStream_t s, const Lut2Args& a) {
    switch (k) {
        case 1: hipLaunchKernelGGL((gemv_lut2_kernel<1, TPW>), gd, bd, 0, s, a); break;
        case 2: hipLaunchKernelGGL((gemv_lut2_kernel<2, TPW>), gd, bd, 0, s, a); break;
        case 3: hipLaunchKernelGGL((gemv_lut2_kernel<3, TPW>), gd, bd, 0, s, a); break;
        case 4: hipLaunchKernelGGL((gemv_lut2_kernel<4, TPW>), gd, bd, 0, s, a); break;
        case 5: hipLaunchKernelGGL((gemv_lut2_kernel<5, TPW>), gd, bd, 0, s, a); break;
        case 6: hipLaunchKernelGGL((gemv_lut2_kernel<6, TPW>), gd, bd, 0, s, a); break;
        case 7: hipLaunchKernelGGL((gemv_lut2_kernel<7, TPW>), gd, bd, 0, s, a); break;
        default: hipLaunchKernelGGL((gemv_lut2_kernel<8, TPW>), gd, bd, 0, s, a); break;
    }
}

hipError_t launch_gemv_lut2(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                            const uint16_t* x, uint16_t* y, const Geometry& g, void* ws, hipStream_t s) {
    Lut2Args a = {};
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
    a.n_slots = (int)((int64_t)k * g.n_gt);
    a.slices = lut_slices(g.n_gt, k, LUT2_SLOTS);
    // two row tiles per wave, or four when two would need a second round of workgroups
    int tpw = LUT_TILES_PER_WAVE, tpb = 0, blocks = 0;
    lut_plan(&g.n_rt, 1, a.slices, tpw, &tpb, &blocks);
    if ((int64_t)a.slices * blocks > LUT_CUS) {
        tpw = LUT_TILES_PER_WAVE_BIG;
        lut_plan(&g.n_rt, 1, a.slices, tpw, &tpb, &blocks);
    }
    a.tiles_per_block = tpb;
    const dim3 gd((unsigned)(a.slices * blocks)), bd(64 * LUT_WAVES);
    // plans of at most 8 row tiles per workgroup run in 8-wave workgroups: the same tiles, sums and bits
    // (4096x4096 k = 1: 4.56 -> 4.25 us; 1024 and 2048 rows 5-9 % faster at k = 1..4)
    if (tpw == LUT_TILES_PER_WAVE && k <= 4 && tpb <= LUT_WAVES_SMALL) {
        const dim3 bd8(64 * LUT_WAVES_SMALL);
        constexpr int T = LUT_TILES_PER_WAVE, W8 = LUT_WAVES_SMALL;
        if (k == 1) hipLaunchKernelGGL((gemv_lut2_kernel<1, T, W8>), gd, bd8, 0, s, a);
        else if (k == 2) hipLaunchKernelGGL((gemv_lut2_kernel<2, T, W8>), gd, bd8, 0, s, a);
        else if (k == 3) hipLaunchKernelGGL((gemv_lut2_kernel<3, T, W8>), gd, bd8, 0, s, a);
        else hipLaunchKernelGGL((gemv_lut2_kernel<4, T, W8>), gd, bd8, 0, s, a);
        return hipGetLastError();
    }
    if (tpw == LUT_TILES_PER_WAVE_BIG) launch_lut2_k<LUT_TILES_PER_WAVE_BIG>(k, gd, bd, s, a);
    else launch_lut2_k<LUT_TILES_PER_WAVE>(k, gd, bd, s, a);
    return hipGetLastError();
}

}  // namespace aqd
