// Device helpers shared by the lookup-table GEMV kernels (batch 1 and the
// two-column variant): the LDS table geometry, streaming loads of code tiles
// through buffer descriptors, the table address of a code byte, the 0/1
// routing operands that sum table entries on the matrix cores, and the
// transposing butterfly over the remaining 16 lanes.
#pragma once
#include "fixed_sum.h"

namespace aqd {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int LUT_SLOTS = 4;
constexpr int LUT_PAIR_BYTES = CODEWORDS * 64 * 4;           // 64 KiB
constexpr int LUT_BYTES = (LUT_SLOTS / 2) * LUT_PAIR_BYTES;  // 128 KiB
constexpr int LUT_CUS = 256;                                  // one 128 KiB workgroup per CU
constexpr int LUT_WAVES = 16;
constexpr int LUT_WAVES_SMALL = 8;                            // waves of a workgroup with at most 8 row tiles
constexpr int LUT_TILES_PER_WAVE = 2;                         // row tiles per wave, default
constexpr int LUT_TILES_PER_WAVE_BIG = 4;                     // ... when 2 would need more workgroups than CUs

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Buffer descriptor over the row tiles of one slot (the dword-3 format word of
// the gfx9 family for raw byte-addressed buffers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const uint8_t* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes, 0x00020000);
}

// Streaming 16-byte load of codes that are read exactly once (nontemporal).
// An offset past the end of the descriptor returns zeros without touching
// memory, which is how a wave without a tile keeps its load count fixed.
constexpr uint32_t NO_TILE = 0x80000000u;
__device__ __forceinline__ uint4 load_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t lut_addr(uint32_t code_dword, uint32_t base, int byte) {
    // byte 0 <- base byte 0 (lane offset), byte 1 <- code byte `byte`, byte 2 <- base byte 2 (slot pair)
    return __builtin_amdgcn_perm(code_dword, base, 0x0C020000u | ((uint32_t)(4 + byte) << 8));
}

// Row sums travel between workgroups as counted fixed-point words (fixed_sum.h).
constexpr int LUT_MAX_SLICES = FIX_MAX_TERMS;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, false));
}

// Row sums of a code tile on the matrix cores.
//
// Lane l (group l of the tile) holds table entries e[r][s] for the 16 rows r
// and the slots s of its slice.  v_mfma_f32_16x16x32_f16 takes, per lane, 8
// fp16 B values B[8*(l>>4) + h][l & 15] and 8 A values A[l & 15][8*(l>>4) + h].
// With B = (row 4q + m, slot s) at h = 2m and zero at h = 2m + 1 (the dword a
// 2-byte LDS read returns), and A_q the 0/1 matrix A_q[i][8g + 2m + hs] =
// [i == 4q + m], one product adds, into D[4q + m][j], the entries of row
// 4q + m, slot s, of the four lanes j + 16g.  Over the row quads q and the
// slots s, D[i][j] = sum over g and s of the entries of row i in lane j + 16g:
// the sums over slots and over the lane groups cost no vector-ALU instruction,
// only the 16 lanes j remain.  (A second slot in the odd halves would halve the
// products but cost a pack per pair of entries; measured slower.)
//
// lut_route(): lane l's operand A_q, nonzero only for q = (l & 15) >> 2, in the
// dword (l & 3): two fp16 ones.
__device__ __forceinline__ half8_t lut_route(int q, int lane) {
    const int i = lane & 15;
    uint32_t d[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) d[m] = i == 4 * q + m ? 0x3C003C00u : 0u;
    return __builtin_bit_cast(half8_t, make_uint4(d[0], d[1], d[2], d[3]));
}

// Two activation columns: B dword m holds the (column 0, column 1) entries of
// row 4q + m, so half h = 2m + c is (row 4q + m, column c).  lut_route2(p)
// is the A operand with A[i][8g + h] = [i == 8p + h]: with p = q mod 2, one
// product adds half h of quad q into D[8(q mod 2) + h][j], so two accumulators
// (quads 0-1 and 2-3) hold the 32 (row, column) sums.
__device__ __forceinline__ half8_t lut_route2(int p, int lane) {
    const int i = lane & 15;
    const uint32_t one = 0x3C00u << (16 * (i & 1));          // the fp16 one, in half (i & 1)
    uint32_t d[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) d[m] = (i >> 1) == 4 * p + m ? one : 0u;
    return __builtin_bit_cast(half8_t, make_uint4(d[0], d[1], d[2], d[3]));
}

// D as left by the products above: lane l holds D[4*(l>>4) + r][l & 15],
// r = 0..3.  Returns, in lane l, the sum over the 16 lanes of its 16-lane row
// of D[l >> 2][.] : output row (l >> 2) summed over all 64 groups, the same
// value in the four lanes of a quad.  Each step keeps half of the rows and adds
// the partner's copy of them (partner j <-> 15 - j, then j <-> 7 - j, then the
// quad), so rows are transposed into lanes as they are summed.
__device__ __forceinline__ float fold_quads(const floatx4_t& d, int lane) {
    const bool lo8 = (lane & 8) == 0;
    float c[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = lo8 ? d[i] : d[i + 2];
        const float send = lo8 ? d[i + 2] : d[i];
        c[i] = keep + dpp<0x140>(send);
    }
    const bool lo4 = (lane & 4) == 0;
    const float keep = lo4 ? c[0] : c[1];
    const float send = lo4 ? c[1] : c[0];
    float e = keep + dpp<0x141>(send);
    e += dpp<0xB1>(e);
    e += dpp<0x4E>(e);
    return e;
}

// Row tiles per workgroup for each linear: the grid aims at one workgroup per
// CU, shared among the linears in proportion to their rows; a workgroup holds
// at most LUT_WAVES * tiles_per_wave tiles.
//
// round4: tile u of wave w is tile w + LUT_WAVES * u, and wave w runs on SIMD
// w % 4, so t tiles put at most ceil(t / 4) on one SIMD; rounding t up to a
// multiple of 4 (within the cap) never adds work to the busiest SIMD and can
// save workgroups.  Measured on the single-linear batch-1 launch (4096 rows
// at 28 slices: 8 workgroups of 32 tiles instead of 9 of 29, 3% faster); the
// two-column kernel was slower with it at 28 slices, so it is not general.
static inline void lut_plan(const int64_t* n_rt, int n, int slices, int tiles_per_wave, int* tpb, int* blocks,
                            bool round4 = false) {
    int64_t total = 0;
    for (int i = 0; i < n; ++i) total += n_rt[i];
    const int64_t cap = LUT_WAVES * tiles_per_wave;
    for (int i = 0; i < n; ++i) {
        int64_t rb = total > 0 ? (LUT_CUS / slices) * n_rt[i] / total : 1;
        if (rb < 1) rb = 1;
        if (rb > n_rt[i]) rb = n_rt[i];
        int64_t t = (n_rt[i] + rb - 1) / rb;
        if (round4) t = (t + 3) / 4 * 4;
        if (t > cap) t = cap;
        tpb[i] = (int)t;
        blocks[i] = (int)((n_rt[i] + t - 1) / t);
    }
}

// Code tiles are addressed through buffer descriptors with 32-bit offsets (and
// the tiles of one group tile of one plane are n_rt * 1 KiB long), so a layer
// may have at most this many row tiles (about 33.5 million rows).
constexpr int64_t LUT_MAX_ROW_TILES = 0x7FFFFFFF / TILE_BYTES;

// Table slices of a launch: k * n_gt slots, LUT_SLOTS per workgroup.
static inline int lut_slices(int64_t n_gt, int k, int slots_per_wg = LUT_SLOTS) {
    return (int)(((int64_t)k * n_gt + slots_per_wg - 1) / slots_per_wg);
}

}  // namespace aqd
