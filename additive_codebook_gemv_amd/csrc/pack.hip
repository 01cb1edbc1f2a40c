// Code packing: logical [d_out][d_in/8][M] <-> plane-major tiles (see aqd_internal.h).
#include "aqd_internal.h"

namespace aqd {

// One thread per (plane, group tile, row tile, lane): gathers the 16 codes of
// one group for 16 consecutive rows and writes them as one 16-byte vector.
__global__ void pack_kernel(const uint8_t* __restrict__ codes, uint8_t* __restrict__ packed, int64_t d_out,
                            int64_t G, int32_t M, int64_t n_rt, int64_t n_gt) {
    const int64_t total = (int64_t)M * n_gt * n_rt * TILE_GROUPS;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int l = (int)(t % TILE_GROUPS);
        const int64_t tile = t / TILE_GROUPS;          // (m * n_gt + jt) * n_rt + it
        const int64_t it = tile % n_rt;
        const int64_t jt = (tile / n_rt) % n_gt;
        const int m = (int)(tile / (n_rt * n_gt));
        const int64_t j = jt * TILE_GROUPS + l;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (j < G) {
            for (int r = 0; r < TILE_ROWS; ++r) {
                const int64_t i = it * TILE_ROWS + r;
                if (i < d_out) w[r >> 2] |= (uint32_t)codes[(i * G + j) * M + m] << (8 * (r & 3));
            }
        }
        uint4 v;
        v.x = w[0]; v.y = w[1]; v.z = w[2]; v.w = w[3];
        *reinterpret_cast<uint4*>(packed + tile * TILE_BYTES + l * TILE_ROWS) = v;
    }
}

// One thread per (row, group): reads its M codes from the M planes.
__global__ void unpack_kernel(const uint8_t* __restrict__ packed, uint8_t* __restrict__ codes, int64_t d_out,
                              int64_t G, int32_t M, int64_t n_rt, int64_t n_gt) {
    const int64_t total = d_out * G;
    const int64_t plane = n_rt * n_gt * TILE_BYTES;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = t / G, j = t % G;
        const int64_t it = i / TILE_ROWS, jt = j / TILE_GROUPS;
        const int64_t off = (jt * n_rt + it) * TILE_BYTES + (j % TILE_GROUPS) * TILE_ROWS + (i % TILE_ROWS);
        for (int m = 0; m < M; ++m) codes[t * M + m] = packed[m * plane + off];
    }
}

static unsigned grid_for(int64_t total, int block) {
    int64_t g = (total + block - 1) / block;
    if (g > 65536) g = 65536;
    if (g < 1) g = 1;
    return (unsigned)g;
}

hipError_t launch_pack(const uint8_t* codes, uint8_t* packed, const Geometry& g, hipStream_t s) {
    const int64_t total = (int64_t)g.M * g.n_gt * g.n_rt * TILE_GROUPS;
    hipLaunchKernelGGL(pack_kernel, dim3(grid_for(total, 256)), dim3(256), 0, s, codes, packed, g.d_out, g.G, g.M,
                       g.n_rt, g.n_gt);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, uint8_t* codes, const Geometry& g, hipStream_t s) {
    hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(g.d_out * g.G, 256)), dim3(256), 0, s, packed, codes, g.d_out,
                       g.G, g.M, g.n_rt, g.n_gt);
    return hipGetLastError();
}

}  // namespace aqd
