// Device helpers shared by the lookup-table GEMV kernels (batch 1 and the
// two-column variant): the LDS table geometry, streaming loads of code tiles
// through buffer descriptors, the table address of a code byte, and the
// transposing butterfly that sums 16 row partials over a wave.
#pragma once
#include "fixed_sum.h"

namespace aqd {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int LUT_SLOTS = 4;
constexpr int LUT_PAIR_BYTES = CODEWORDS * 64 * 4;           // 64 KiB
constexpr int LUT_BYTES = (LUT_SLOTS / 2) * LUT_PAIR_BYTES;  // 128 KiB
constexpr int LUT_CUS = 256;                                  // one 128 KiB workgroup per CU
constexpr int LUT_WAVES = 16;
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

__device__ __forceinline__ float2 swap32(float a, float b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float2 swap16(float a, float b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// v[r] = partial of row r in this lane.  Returns, in lane l, the sum over the
// 64 lanes of row (l >> 2).
__device__ __forceinline__ float fold_rows(const float (&v)[16], int lane) {
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {          // lanes 0-31 keep row i, lanes 32-63 keep row i+8
        const float2 s = swap32(v[i], v[i + 8]);
        a[i] = s.x + s.y;
    }
    float b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {          // even 16-lane rows keep i, odd rows keep i+4
        const float2 s = swap16(a[i], a[i + 4]);
        b[i] = s.x + s.y;
    }
    const bool lo8 = (lane & 8) == 0;      // partner lane j <-> 15-j inside 16 lanes
    float c[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = lo8 ? b[i] : b[i + 2];
        const float send = lo8 ? b[i + 2] : b[i];
        c[i] = keep + dpp<0x140>(send);
    }
    const bool lo4 = (lane & 4) == 0;      // partner lane j <-> 7-j inside 8 lanes
    const float keep = lo4 ? c[0] : c[1];
    const float send = lo4 ? c[1] : c[0];
    float d = keep + dpp<0x141>(send);
    d += dpp<0xB1>(d);                     // quad: lanes 4q..4q+3 hold the same row
    d += dpp<0x4E>(d);
    return d;
}

// 1.0f in a scalar register the compiler cannot see through, so that
// fma((float)h0, one, (float)h1) of two fp16 values stays one v_fma_mix_f32
// instead of two conversions and an add.
__device__ __forceinline__ float opaque_one() {
    float v;
    asm volatile("s_mov_b32 %0, 1.0" : "=s"(v));
    return v;
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
