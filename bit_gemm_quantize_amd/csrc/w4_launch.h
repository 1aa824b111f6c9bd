// Host-side launchers of the gfx950 kernels (internal to the library).
// Arguments are already validated by the C interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4a16.h"

namespace w4 {

// Compute units of the current device, and the LDS one workgroup may use
// (at most 160 KB), cached per device.
int compute_units();
size_t max_lds_per_block();

hipError_t launch_quantize(const uint16_t *W, int64_t N, int64_t K, int G,
                           uint8_t *codes, uint16_t *scales, uint16_t *zeros,
                           hipStream_t stream);

// Several quantize jobs (same G) in one launch; jobs validated by the caller.
hipError_t launch_quantize_batch(const w4_quant_job *jobs, int njobs, int G,
                                 hipStream_t stream);

// Quantize -> dequantize round trip of launch_quantize, bf16 out.
hipError_t launch_fake_quant(const uint16_t *W, int64_t N, int64_t K, int G, uint16_t *what,
                             hipStream_t stream);

// Plain layout -> pre-shuffled layout (codes_ps [N, K/2], sz [N, K/G]).
hipError_t launch_repack(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros,
                         int64_t N, int64_t K, int G, uint8_t *codes_ps, uint32_t *sz,
                         hipStream_t stream);

// Per-token int8 activations: x8 [M, K], sx [M].
hipError_t launch_act_quant(const uint16_t *x, int64_t M, int64_t K, int8_t *x8, float *sx,
                            hipStream_t stream);

// W4A8 linear on the int8 matrix cores, any M >= 1, K % 64 == 0.
hipError_t launch_w4a8_gemm(const int8_t *x8, const float *sx, int64_t M, const uint8_t *codes,
                            const uint16_t *scales, const uint16_t *zeros,
                            const uint16_t *bias, int64_t N, int64_t K, int G, uint16_t *y,
                            hipStream_t stream);

// Its decode kernel on the vector ALUs for 1 <= M <= A8_ROWS_MAX_M and
// K <= A8_ROWS_MAX_K (32-bit buffer offsets); hipErrorInvalidValue otherwise.
constexpr int64_t A8_ROWS_MAX_M = 8;
constexpr int64_t A8_ROWS_MAX_K = int64_t(1) << 24;
hipError_t launch_w4a8_rows(const int8_t *x8, const float *sx, int64_t M, const uint8_t *codes,
                            const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                            int64_t N, int64_t K, int G, uint16_t *y, hipStream_t stream);

// Int8 weight-only: quantizer (codes int8 [N, K], scales [N, K/G]) and the
// linear for any M >= 1 (K % 64 == 0).
hipError_t launch_quantize8(const uint16_t *W, int64_t N, int64_t K, int G, int8_t *q8,
                            uint16_t *scales, hipStream_t stream);
hipError_t launch_w8a16(const uint16_t *x, int64_t M, const int8_t *q8, const uint16_t *scales,
                        const uint16_t *bias, int64_t N, int64_t K, int G, uint16_t *y,
                        hipStream_t stream);
// Its decode kernel on the vector ALUs for 1 <= M <= W8_ROWS_MAX_M and
// K <= W8_ROWS_MAX_K (32-bit buffer offsets); hipErrorInvalidValue otherwise.
constexpr int64_t W8_ROWS_MAX_M = 4;
constexpr int64_t W8_ROWS_MAX_K = int64_t(1) << 24;
hipError_t launch_w8a16_rows(const uint16_t *x, int64_t M, const int8_t *q8,
                             const uint16_t *scales, const uint16_t *bias, int64_t N, int64_t K,
                             int G, uint16_t *y, hipStream_t stream);

// Decode GEMV, 1 <= M <= 16. Plain layout (scales, zeros; sz == NULL) or
// pre-shuffled layout (codes pre-shuffled, sz != NULL; scales, zeros unused).
hipError_t launch_gemv(const uint16_t *x, int M, const uint8_t *codes,
                       const uint16_t *scales, const uint16_t *zeros, const uint32_t *sz,
                       const uint16_t *bias, int64_t N, int64_t K, int G,
                       uint16_t *y, hipStream_t stream);

// Prefill GEMM, any M >= 1; layouts as launch_gemv.
hipError_t launch_gemm(const uint16_t *x, int64_t M, const uint8_t *codes,
                       const uint16_t *scales, const uint16_t *zeros, const uint32_t *sz,
                       const uint16_t *bias, int64_t N, int64_t K, int G,
                       uint16_t *y, hipStream_t stream);

} // namespace w4
