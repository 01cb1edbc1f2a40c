// Internal declarations shared by the HIP sources of libaqd (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "aqd.h"

namespace aqd {

// Packed code tiles.  Plane-major: all tiles of codebook 0, then codebook 1, ...
// Inside a plane, tiles are ordered [group tile jt][row tile it]; a tile covers
// TILE_ROWS consecutive rows and TILE_GROUPS consecutive 8-wide groups and is
// stored lane-major: byte (l * TILE_ROWS + r) holds the code of row
// it*TILE_ROWS + r, group jt*TILE_GROUPS + l.  One tile is 1 KiB, so a wave of
// 64 lanes loading 16 bytes each reads one whole tile, and lane l receives the
// codes of one group for 16 consecutive rows.  Rows and groups past the layer
// edge are padding (code 0) and never contribute.
constexpr int TILE_ROWS = 16;
constexpr int TILE_GROUPS = 64;
constexpr int TILE_BYTES = TILE_ROWS * TILE_GROUPS;
constexpr int GROUP = 8;
constexpr int CODEWORDS = 256;
constexpr int MAX_M = 8;

struct Geometry {
    int64_t d_out, d_in, G;        // G = d_in / 8
    int64_t n_rt, n_gt;            // row tiles, group tiles
    int64_t plane_bytes;           // n_rt * n_gt * TILE_BYTES
    int32_t M;
};

inline Geometry geometry(const aqd_layer& L) {
    Geometry g;
    g.d_out = L.d_out;
    g.d_in = L.d_in;
    g.G = L.d_in / GROUP;
    g.n_rt = (L.d_out + TILE_ROWS - 1) / TILE_ROWS;
    g.n_gt = (g.G + TILE_GROUPS - 1) / TILE_GROUPS;
    g.plane_bytes = g.n_rt * g.n_gt * TILE_BYTES;
    g.M = L.M;
    return g;
}

// Per-thread error text (set by the C entry points).
void set_error(const std::string& s);
// aqd_gemv's argument checks without the workspace pointer (ws_bytes available); *need = workspace bytes
aqd_status check_gemv_args(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int32_t k,
                           const uint16_t* x_rot, const uint16_t* y, int32_t batch, const aqd_layer* layer,
                           size_t ws_bytes, size_t* need, bool* nothing);
// AQD_OK for hipSuccess, else AQD_ERR_HIP with the text in the per-thread error
aqd_status hip_fail(hipError_t e, const char* what);

// ---- launchers (return hipSuccess or the launch error) --------------------
hipError_t launch_pack(const uint8_t* codes, uint8_t* packed, const Geometry& g, hipStream_t s);
hipError_t launch_unpack(const uint8_t* packed, uint8_t* codes, const Geometry& g, hipStream_t s);
// signs: NULL, or a bit mask of d_in bits (8-byte aligned) that negates input c
// before the butterflies when bit c % 8 of byte c / 8 is set
hipError_t launch_hadamard(const void* x, void* y, int in_dt, int out_dt, int64_t batch, int64_t d_in,
                           int block, const uint8_t* signs, hipStream_t s);
size_t gemv_workspace_bytes(const Geometry& g, int batch);
// leading bytes of the GEMV workspace that must be zero when a call starts (the table routes'
// counted row sums; every call leaves them zero again)
size_t gemv_zeroed_bytes(const Geometry& g);
hipError_t launch_gemv(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                       const uint16_t* x, uint16_t* y, int batch, const Geometry& g, void* ws, hipStream_t s);
size_t gemv_lut_workspace_bytes(const Geometry& g);
bool gemv_lut_supported(const Geometry& g, int batch, int k);
hipError_t launch_gemv_lut(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                           const uint16_t* x, uint16_t* y, const Geometry& g, void* ws, hipStream_t s);
// batch 2 through the lookup tables: x [2][d_in], y [2][d_out], ws holds [2][d_out] words kept zero
size_t gemv_lut2_workspace_bytes(const Geometry& g);
bool gemv_lut2_supported(const Geometry& g, int batch, int k);
size_t gemv_lut4_workspace_bytes(const Geometry& g);
bool gemv_lut4_supported(const Geometry& g, int batch, int k);
hipError_t launch_gemv_lut4(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                            const uint16_t* x, uint16_t* y, int batch, const Geometry& g, void* ws, hipStream_t s);
hipError_t launch_gemv_lut2(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                            const uint16_t* x, uint16_t* y, const Geometry& g, void* ws, hipStream_t s);
// several batch-1 linears sharing one input and k, in one launch
struct LutLinearRef {
    const uint8_t* packed;
    const uint16_t* codebooks;
    const uint16_t* scales;
    uint16_t* y;
    int64_t d_out;
};
bool gemv_lut_grouped_supported(int64_t G, int k, const int64_t* d_out, int n);
size_t gemv_lut_grouped_workspace_bytes(const int64_t* d_out, int n);
// rotate_block 0: x is already rotated; 64/128/256: x is raw and each workgroup rotates what it needs
hipError_t launch_gemv_lut_grouped(const LutLinearRef* lins, int n, int k, const uint16_t* x, int64_t d_in,
                                   void* ws, hipStream_t s, int rotate_block, const uint8_t* signs);
size_t gemm_sb_workspace_bytes(const Geometry& g, int batch);
// tiered batch: column n uses the first ks[n] codebooks (host array)
hipError_t launch_gemm_sb_tiered(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales,
                                 const int32_t* ks, const uint16_t* x, float* y, int batch, const Geometry& g,
                                 void* ws, hipStream_t s);
hipError_t launch_gemm_sb(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                          const void* x, int x_dt, float* y, int batch, const Geometry& g, void* ws,
                          hipStream_t s);

// y[n][i] = s_i * sum over splits (fixed order) of part[split][n][i]; at most 16 splits
hipError_t launch_split_reduce(const float* part, const uint16_t* scales, float* y, int64_t d_out, int batch,
                               int splits, hipStream_t s);
hipError_t launch_zero_f32(float* y, int64_t n, hipStream_t s);
hipError_t launch_zero_f16(uint16_t* y, int64_t n, hipStream_t s);
// fp16 activations, fp16 output y = fp16(s * acc): the matrix-core route of the batch 2..8 GEMV
hipError_t launch_gemm_sb_f16out(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                                 const uint16_t* x, uint16_t* y, int batch, const Geometry& g, void* ws,
                                 hipStream_t s);
// prefill / large batch (fp16 activations, fp32 output)
size_t gemm_pf_workspace_bytes(const Geometry& g, int batch);
hipError_t launch_gemm_pf(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                          const uint16_t* x, float* y, int batch, const Geometry& g, void* ws, hipStream_t s);

// encode side: greedy residual codes [d_out][d_in/8][M] for fp32 targets [d_out][d_in]
hipError_t launch_encode_greedy(const float* target, const uint16_t* codebooks, int M, int64_t d_out,
                                int64_t d_in, uint8_t* codes, hipStream_t s);

// Split partial sums, shared by the small-batch and prefill kernels and their
// reduce: [split][column][row quad] of float4 (rows 4q .. 4q+3).  The lanes that
// hold consecutive row quads of one column write one contiguous run, and a
// reduce thread reads each split's quad as one 16-byte word.
inline size_t partial_bytes(int64_t d_out, int batch, int splits) {
    return (size_t)splits * (size_t)batch * (size_t)((d_out + 3) / 4) * 16;
}

// ---- device helpers --------------------------------------------------------
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float h2f(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint16_t f2h(float f) {  // round to nearest even
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float bf2f(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}
// float -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ void store_partial(float* part, int64_t d_out, int batch, unsigned split, int col,
                                              int64_t row0, float4 v) {
    const int64_t nq = (d_out + 3) / 4;
    reinterpret_cast<float4*>(part)[((int64_t)split * batch + col) * nq + row0 / 4] = v;
}

}  // namespace aqd
