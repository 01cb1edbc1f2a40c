// aqd_gemv_noalloc: the decode GEMV (aqd_gemv, batch 1..8) for callers that
// cannot allocate device memory: code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation.  Its workspace is the file-scope
// device array `scratch` below, AQD_NOALLOC_SCRATCH_BYTES per GPU, held by each
// GPU the library runs on until the process ends.
//
// In host code the array's name is a host-side stand-in, not a device address,
// so it is never passed to a kernel or a copy: the device address of each GPU's
// copy is looked up once per device (hipGetSymbolAddress, with that device
// current) on the entry point's first call there, and only that address is
// used.  Every call clears the leading part that must start at zero (the table
// routes' counted row sums) with a fill kernel on the caller's stream, then
// runs exactly the kernels aqd_gemv runs.  Every call on one GPU shares that
// GPU's array: calls that may overlap in time race and give undefined results.
#include <mutex>

#include "aqd_internal.h"

namespace aqd {

static __device__ __align__(256) uint8_t scratch[AQD_NOALLOC_SCRATCH_BYTES];

constexpr int NOALLOC_MAX_DEVICES = 64;
static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[NOALLOC_MAX_DEVICES];

// Device address of the current device's scratch array (looked up once per device).
static aqd_status scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "aqd_gemv_noalloc: hipGetDevice");
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) {
        set_error("aqd_gemv_noalloc: device index above the supported 64 devices");
        return AQD_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "aqd_gemv_noalloc: hipGetSymbolAddress");
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) {
            set_error("aqd_gemv_noalloc: scratch array has no usable device address");
            return AQD_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return AQD_OK;
}

}  // namespace aqd

using namespace aqd;

extern "C" aqd_status aqd_gemv_noalloc(const uint8_t* packed_codes, const uint16_t* codebooks,
                                       const uint16_t* scales, int32_t k, const uint16_t* x_rot, uint16_t* y,
                                       int32_t batch, const aqd_layer* layer, void* stream) {
    size_t need = 0;
    bool nothing = false;
    aqd_status st = check_gemv_args(packed_codes, codebooks, scales, k, x_rot, y, batch, layer,
                                    AQD_NOALLOC_SCRATCH_BYTES, &need, &nothing);
    if (st != AQD_OK || nothing) return st;
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != AQD_OK) return st;
    const Geometry g = geometry(*layer);
    hipStream_t s = (hipStream_t)stream;
    const size_t zeroed = gemv_zeroed_bytes(g);                      // a multiple of 256 bytes
    hipError_t e = launch_zero_f32(static_cast<float*>(ws), (int64_t)(zeroed / 4), s);
    if (e != hipSuccess) return hip_fail(e, "aqd_gemv_noalloc: clearing the scratch");
    return hip_fail(launch_gemv(packed_codes, codebooks, scales, k, x_rot, y, batch, g, ws, s), "aqd_gemv_noalloc");
}
