// Block Walsh-Hadamard butterflies on one 64-wide wavefront (Drop-by-Drop,
// section 5: block-wise Walsh-Hadamard rotation of the activation, online).
//
// Lane l holds the elements l, l + 64, l + 128, ... of a block of B inputs
// (B/64 per lane).  The six stages whose partners are 1..32 lanes apart cross
// lanes, the stages 64 and 128 apart stay in registers.  Sums are fp32; the
// result is scaled by 1/sqrt(B).  The network gives the Sylvester-order matrix
// H[r][c] = (-1)^popcount(r & c).  Shared by the standalone rotation and the
// GEMV that rotates its own input, so both produce the same bits.
//
// Cross-lane partners come from the VALU's own lane networks, not through the
// LDS crossbar:
//   1, 2   quad permutation (DPP quad_perm);
//   4, 8   row shifts by 4 / 8 (DPP row_shl / row_shr), each written only into
//          the lanes whose partner lies in that direction (DPP bank mask: a
//          bank is 4 consecutive lanes of a 16-lane row);
//   16, 32 gfx950's v_permlane16_swap / v_permlane32_swap, which exchange
//          odd and even 16-lane rows, or the two 32-lane halves, between two
//          registers.
// Each stage then computes partner + v (lower lane of the pair) or
// partner - v (upper lane) as one fma with a per-lane sign of +-1, which is
// exact in its product and so rounds like the plain add or subtract.
#pragma once
#include "aqd_internal.h"

namespace aqd {

template <int B>
__device__ __forceinline__ float inv_sqrt_block() {
    return B == 64 ? 0.125f : (B == 128 ? 0.0883883476483184405f : 0.0625f);
}

namespace fwht_detail {

constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROW_SHL4 = 0x104, DPP_ROW_SHR4 = 0x114;
constexpr int DPP_ROW_SHL8 = 0x108, DPP_ROW_SHR8 = 0x118;

template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp_into(float old, float v) {
    return __uint_as_float(
        __builtin_amdgcn_update_dpp(__float_as_uint(old), __float_as_uint(v), CTRL, 0xF, BANKS, false));
}

// every lane written (no old value); with a partial bank mask the other lanes are undefined
template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp(float v) {
    return __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(v), CTRL, 0xF, BANKS, false));
}

// value of lane (l ^ H) in lane l, for H in {1, 2, 4, 8}
template <int H>
__device__ __forceinline__ float partner(float v) {
    if constexpr (H == 1) return dpp<DPP_QUAD_XOR1, 0xF>(v);
    if constexpr (H == 2) return dpp<DPP_QUAD_XOR2, 0xF>(v);
    // lanes with bit H clear read H lanes up, the others H lanes down; a bank is 4 lanes
    if constexpr (H == 4) return dpp_into<DPP_ROW_SHL4, 0x5>(dpp<DPP_ROW_SHR4, 0xA>(v), v);
    return dpp_into<DPP_ROW_SHL8, 0x3>(dpp<DPP_ROW_SHR8, 0xC>(v), v);
}

}  // namespace fwht_detail

template <int B>
__device__ __forceinline__ void fwht_block(float (&v)[B / 64], int lane) {
    using namespace fwht_detail;
    constexpr int E = B / 64;
    // sign of v in stage h: +1 in the lower lane of a pair, -1 in the upper
    const float s1 = (lane & 1) ? -1.f : 1.f, s2 = (lane & 2) ? -1.f : 1.f;
    const float s4 = (lane & 4) ? -1.f : 1.f, s8 = (lane & 8) ? -1.f : 1.f;
    const float s16 = (lane & 16) ? -1.f : 1.f, s32 = (lane & 32) ? -1.f : 1.f;
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = __builtin_fmaf(s1, v[e], partner<1>(v[e]));
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = __builtin_fmaf(s2, v[e], partner<2>(v[e]));
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = __builtin_fmaf(s4, v[e], partner<4>(v[e]));
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = __builtin_fmaf(s8, v[e], partner<8>(v[e]));
#pragma unroll
    for (int e = 0; e < E; ++e) {
        // even rows: (own row, odd row) = (lower, upper) of each pair; odd rows: (even row, own row)
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[e]), __float_as_uint(v[e]), false, false);
        v[e] = __builtin_fmaf(s16, __uint_as_float(r[1]), __uint_as_float(r[0]));
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        // lanes 0-31: (own, lane + 32); lanes 32-63: (lane - 32, own)
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[e]), __float_as_uint(v[e]), false, false);
        v[e] = __builtin_fmaf(s32, __uint_as_float(r[1]), __uint_as_float(r[0]));
    }
#pragma unroll
    for (int hb = 1; hb < E; hb <<= 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if ((e & hb) == 0) {
                const float a = v[e], c = v[e | hb];
                v[e] = a + c;
                v[e | hb] = a - c;
            }
        }
    }
    const float sc = inv_sqrt_block<B>();
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] *= sc;
}

// The same network on 256 consecutive inputs laid out as the B operand of a
// 32x32x8 matrix product over 32 groups of 8: lane l holds the four inputs
// 8 (l mod 32) + 4 (l / 32) + r, r = 0..3, so index bits 0-1 are the register
// r, bit 2 is lane bit 5 and bits 3-7 are lane bits 0-4.  A block of B inputs
// (64, 128 or 256; blocks start at multiples of B) takes the stages 1 .. B/2
// apart in the order fwht_block takes them, each element becoming the same
// lower + upper or lower - upper of the same two values, so every output has
// the bits fwht_block gives it.
template <int B>
__device__ __forceinline__ void fwht_operand(float (&v)[4], int lane) {
    using namespace fwht_detail;
    static_assert(B == 64 || B == 128 || B == 256, "block");
    // distances 1 and 2: register pairs (r, r ^ 1), then (r, r ^ 2)
#pragma unroll
    for (int hb = 1; hb <= 2; hb <<= 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if ((r & hb) == 0) {
                const float a = v[r], c = v[r | hb];
                v[r] = a + c;
                v[r | hb] = a - c;
            }
        }
    }
    // distance 4: the two 32-lane halves; lanes 0-31: (own, lane + 32), lanes 32-63: (lane - 32, own)
    const float s32 = (lane & 32) ? -1.f : 1.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[r]), __float_as_uint(v[r]), false, false);
        v[r] = __builtin_fmaf(s32, __uint_as_float(q[1]), __uint_as_float(q[0]));
    }
    // distances 8, 16, 32 (and 64, 128 for the larger blocks): lanes 1, 2, 4 (8, 16) apart
    const float s1 = (lane & 1) ? -1.f : 1.f, s2 = (lane & 2) ? -1.f : 1.f, s4 = (lane & 4) ? -1.f : 1.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = __builtin_fmaf(s1, v[r], partner<1>(v[r]));
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = __builtin_fmaf(s2, v[r], partner<2>(v[r]));
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = __builtin_fmaf(s4, v[r], partner<4>(v[r]));
    if constexpr (B >= 128) {
        const float s8 = (lane & 8) ? -1.f : 1.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = __builtin_fmaf(s8, v[r], partner<8>(v[r]));
    }
    if constexpr (B == 256) {
        // even 16-lane rows: (own, lane + 16); odd rows: (lane - 16, own)
        const float s16 = (lane & 16) ? -1.f : 1.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[r]), __float_as_uint(v[r]), false, false);
            v[r] = __builtin_fmaf(s16, __uint_as_float(q[1]), __uint_as_float(q[0]));
        }
    }
    const float sc = inv_sqrt_block<B>();
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] *= sc;
}

}  // namespace aqd
