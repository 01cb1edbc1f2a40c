// A plain streaming-read kernel: the measurement reference for what one launch
// can stream from HBM (launch, ramp, latency and drain included).  It reads
// every 16-byte word of a buffer once through a buffer descriptor with
// nontemporal loads, the load form the GEMV uses for its code stream, and
// folds the words into an XOR that is stored only on a value that does not
// occur in practice, so the loads stay live and the launch writes nothing.
#include <string>

#include "aqd_internal.h"
#include "aqd_probe.h"
#include "lut_device.h"

namespace aqd {

constexpr uint32_t PROBE_MAGIC = 0x9E3779B9u;

template <int U, bool CONTIG>
__global__ void read_probe_kernel(const uint8_t* __restrict__ src, uint32_t n16, uint32_t* __restrict__ sink) {
    const __amdgpu_buffer_rsrc_t r = slot_rsrc(src, (int64_t)n16 * 16);
    uint32_t first, step, end;
    if (CONTIG) {               // this workgroup's segment, lanes striding inside it
        const uint32_t per = (uint32_t)(((uint64_t)n16 + gridDim.x - 1) / gridDim.x);
        const uint64_t lo = (uint64_t)blockIdx.x * per;
        first = (uint32_t)(lo < n16 ? lo : n16) + threadIdx.x;
        end = (uint32_t)(lo + per < n16 ? lo + per : n16);
        step = blockDim.x;
    } else {                    // the whole grid strides over the buffer
        first = blockIdx.x * blockDim.x + threadIdx.x;
        end = n16;
        step = gridDim.x * blockDim.x;
    }
    uint32_t acc = 0;
    uint32_t i = first;
    for (; (uint64_t)i + (uint64_t)(U - 1) * step < end; i += U * step) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = load_stream(r, (i + u * step) * 16u);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += step) {
        const uint4 v = load_stream(r, i * 16u);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == PROBE_MAGIC) sink[blockIdx.x] = acc;
}

template <bool CONTIG>
static void launch_probe(int unroll, dim3 gd, dim3 bd, hipStream_t s, const uint8_t* src, uint32_t n16,
                         uint32_t* sink) {
    switch (unroll) {
        case 1: hipLaunchKernelGGL((read_probe_kernel<1, CONTIG>), gd, bd, 0, s, src, n16, sink); break;
        case 2: hipLaunchKernelGGL((read_probe_kernel<2, CONTIG>), gd, bd, 0, s, src, n16, sink); break;
        case 4: hipLaunchKernelGGL((read_probe_kernel<4, CONTIG>), gd, bd, 0, s, src, n16, sink); break;
        default: hipLaunchKernelGGL((read_probe_kernel<8, CONTIG>), gd, bd, 0, s, src, n16, sink); break;
    }
}

}  // namespace aqd

using namespace aqd;

extern "C" aqd_status aqd_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                                     int32_t waves, int32_t unroll, int32_t contiguous, void* stream) {
    if (bytes == 0) return AQD_OK;
    if (!src || !sink) {
        set_error("src or sink is NULL");
        return AQD_ERR_NULL;
    }
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u)) {
        set_error("src must be 16-byte and sink 4-byte aligned");
        return AQD_ERR_ALIGN;
    }
    if (bytes % 16 || bytes > 0xFFFFFFF0ull || workgroups < 1 || workgroups > 65536 || waves < 1 || waves > 16 ||
        (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) || (contiguous != 0 && contiguous != 1)) {
        set_error("bytes, workgroups, waves, unroll or contiguous out of range");
        return AQD_ERR_SHAPE;
    }
    const dim3 gd((unsigned)workgroups), bd((unsigned)(64 * waves));
    const uint32_t n16 = (uint32_t)(bytes / 16);
    hipStream_t s = (hipStream_t)stream;
    const uint8_t* p = static_cast<const uint8_t*>(src);
    if (contiguous) launch_probe<true>(unroll, gd, bd, s, p, n16, sink);
    else launch_probe<false>(unroll, gd, bd, s, p, n16, sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error(std::string("aqd_read_probe: ") + hipGetErrorString(e));
        return AQD_ERR_HIP;
    }
    return AQD_OK;
}
