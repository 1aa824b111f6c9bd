/*
 * w4_measure.h - measurement aids of the W4A16 library (not part of the
 * quantization method): reference kernels the benchmark times beside the
 * method's kernels. Same conventions as w4a16.h.
 */
#ifndef W4_MEASURE_H
#define W4_MEASURE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "w4a16.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * w4_read_stream - read `bytes` bytes of device memory at p once, with
 * 16-byte loads (each wave reads 4 contiguous KB), and discard them: the
 * read bandwidth a plain streaming kernel reaches on this device, the
 * ceiling for a kernel that must read the same bytes.
 *
 * p       in   device pointer, 16-byte aligned, read only
 * bytes   in   16 <= bytes <= 2^40, a multiple of 16
 * sink    out  device pointer to 64 uint32 (16-byte aligned); written only
 *              if the xor of the data equals 0x9E3779B9 (keeps the loads)
 * Returns W4_ERR_NULL, W4_ERR_SHAPE or W4_ERR_ALIGN before any HIP call on
 * bad arguments, W4_ERR_HIP on a launch error.
 */
w4_status w4_read_stream(const void *p, int64_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W4_MEASURE_H */
