/*
 * aqd_probe.h -- a plain streaming-read kernel, exported by libaqd as a
 * measurement reference.  It is not part of the method: it reads a buffer
 * once with 16-byte loads and does nothing else, so the time one launch of it
 * takes bounds what any kernel that must stream the same bytes in one launch
 * can reach on this part (launch, ramp, memory latency and drain included).
 * The GEMV's code stream is timed against it as well as against the 8 TB/s
 * HBM peak.
 */
#ifndef AQD_PROBE_H_
#define AQD_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include "aqd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of device memory at `src` once.
 *
 * src:        device pointer, 16-byte aligned; bytes a multiple of 16, at most 2^32 - 16.
 * sink:       device uint32_t [workgroups]; written only if the XOR of everything a
 *             workgroup's lane read equals 0x9E3779B9 (which keeps the loads live and
 *             in practice writes nothing), so the launch is read-only.
 * workgroups: 1..65536 workgroups of 64 * waves lanes; waves 1..16.
 * unroll:     16-byte loads each lane keeps in flight: 1, 2, 4 or 8.
 * contiguous: 0: the grid strides over the buffer (consecutive lanes of the whole grid read
 *             consecutive 16 bytes); 1: workgroup w reads the w-th of `workgroups`
 *             contiguous segments, its lanes striding inside it.
 * Errors: AQD_ERR_NULL, AQD_ERR_ALIGN, AQD_ERR_SHAPE for arguments out of range;
 * AQD_ERR_HIP if the launch fails.  bytes = 0 launches nothing.
 */
aqd_status aqd_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups, int32_t waves,
                          int32_t unroll, int32_t contiguous, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AQD_PROBE_H_ */
