/*
 * w4a16.h - group-wise asymmetric int4 weight-only quantization and the
 * W4A16 linear layer, for AMD Instinct MI355X (gfx950).
 *
 * The method (sources are web pages, cited by title and section):
 *   - "Optimum Quanto", "Design overview / Tensors": below 8 bits a tensor is
 *     projected group-wise and affinely, with an offset ("zero-point"), onto
 *     the target integer range, and mapped by rounding (torch.round: half to
 *     even).
 *   - "Optimum Quanto", "Modules": weights are quantized per output channel
 *     along their first dimension; the bias is not quantized.
 *   - "Optimum Quanto", "Pitfalls when quantizing activations": matmul
 *     results are accumulated much wider than the inputs (float32) and then
 *     dequantized.
 *   - torchao README ("PyTorch原生训练至推理模型优化"), quick start, and
 *     "torchao模型量化完全指南" section 3.1: int4 weight-only quantization
 *     configured by a group size (32 recommended; 32/64/128 in use) applied
 *     in place to nn.Linear weights [out_features, in_features].
 *
 * Data formats (all row-major, bf16 carried as raw uint16_t bits):
 *   W      bf16  [N, K]      weight, N = out_features, K = in_features
 *   codes  uint8 [N, K/2]    4-bit codes q in 0..15, two per byte:
 *                            codes[n][j] = q[n][2j] | q[n][2j+1] << 4
 *   scales bf16  [N, K/G]    s = bf16_rne((max - min) / 15)   (binary32 ops)
 *   zeros  bf16  [N, K/G]    z = group minimum (the offset), +0 for zeros
 *   dequantized weight       w_hat[n][k] = q[n][k] * s[n][k/G] + z[n][k/G]
 *   x      bf16  [M, K],  bias bf16 [N] (optional),  y bf16 [M, N]
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers owned by the caller; every base pointer
 *     must be 16-byte aligned. Outputs must not overlap inputs.
 *   - Arguments are validated before any HIP call. On a validation error
 *     nothing is launched and nothing is written; the status says why.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *     A launch failure returns W4_ERR_HIP; faults during execution surface
 *     at the caller's next synchronisation, as for any HIP kernel.
 *   - The library allocates no memory and keeps no per-call state (it
 *     caches a few device attributes per device, set once, and the LDS
 *     limit of one kernel); calls are reentrant. No C++ exception crosses
 *     the interface.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4_OK = 0,
    W4_ERR_NULL = 1,   /* a required pointer is NULL                         */
    W4_ERR_SHAPE = 2,  /* N < 1, K < 1, M < 0, K % G != 0, or size overflow  */
    W4_ERR_GROUP = 3,  /* G not in {32, 64, 128}                             */
    W4_ERR_ALIGN = 4,  /* a pointer is not 16-byte aligned                   */
    W4_ERR_HIP = 5,    /* the HIP runtime reported a launch error            */
    W4_ERR_ALIAS = 6,  /* an output buffer overlaps an input buffer          */
    W4_ERR_PATH = 7    /* a forced kernel path cannot serve this M           */
} w4_status;

/* Kernel selection for w4a16_linear_select. AUTO is what w4a16_linear does:
 * the decode GEMV for M <= 16, the prefill GEMM for M > 16 - except when
 * the GEMM's 128 x 128 tiles would be too few to fill the chip (ceil(M/16)
 * x tiles <= 0.6 x compute units): then the decode GEMV runs on 16-row
 * slices of x and y, one launch per slice. Results meet the same accuracy
 * bound either way. */
typedef enum {
    W4_PATH_AUTO = 0,
    W4_PATH_GEMV = 1,  /* valid for 1 <= M <= 16 */
    W4_PATH_GEMM = 2   /* valid for any M >= 1   */
} w4_path;

/* Largest M the decode GEMV serves. */
#define W4_GEMV_MAX_M 16

/* Largest K the decode GEMV serves (its kernels address one row block with
 * 32-bit offsets); W4_PATH_AUTO sends larger K to the GEMM. */
#define W4_GEMV_MAX_K (1 << 24)

/*
 * quantize_int4_grouped - quantize a bf16 weight W[N, K] with group size G
 * along K ("Optimum Quanto", "Design overview / Tensors"; torchao int4
 * weight-only config with group_size).
 *
 * For every row n and group g (elements k in [gG, gG+G)), in IEEE binary32:
 *   lo = min(W) + 0, hi = max(W) + 0          (signed zeros made +0)
 *   s  = bf16_rne((hi - lo) / 15)              (correctly rounded divide)
 *   z  = lo                                    (exact: lo is an input)
 *   q  = s == 0 ? 0 : clamp(rint((w - lo) / s), 0, 15)   (ties to even)
 * and writes codes/scales/zeros in the formats above. Results are bit-exact
 * and deterministic for finite inputs whose group range hi - lo is finite;
 * for other inputs the outputs are unspecified (no fault).
 *
 * W       in   bf16 [N, K], read only; the caller may free it once the
 *              stream has passed this call (the "freeze" step).
 * N, K    in   N >= 1, K >= 1, K % G == 0
 * G       in   32, 64 or 128
 * codes   out  uint8 [N, K/2]
 * scales  out  bf16  [N, K/G]
 * zeros   out  bf16  [N, K/G]
 */
w4_status quantize_int4_grouped(const uint16_t *W, int64_t N, int64_t K,
                                int64_t G, uint8_t *codes, uint16_t *scales,
                                uint16_t *zeros, hipStream_t stream);

/*
 * fake_quant_int4_grouped - the quantize -> dequantize round trip of
 * quantize_int4_grouped, in bf16: the weight a quantization-aware training
 * forward uses to simulate int4 weight quantization (torchao README
 * ("PyTorch原生训练至推理模型优化"), "Training / quantization-aware
 * training": prepare / convert steps over a group-wise int4 weight config;
 * "torchao模型量化完全指南" section 4.1: QAT simulates the quantization error
 * during training; torchao release notes, "BC Breaking": the int4 weight
 * fake-quantize config).
 *
 * For every element, with q, s, z exactly as quantize_int4_grouped computes
 * them (same group, same binary32 steps):
 *   W_hat[n][k] = bf16_rne( fl32( q[n][k] * s[n][g] + z[n][g] ) )
 * (q * s is exact in binary32, so this is one fused multiply-add, then the
 * round to bf16). Bit-exact and deterministic for the inputs
 * quantize_int4_grouped accepts; constant groups come back unchanged.
 *
 * W       in   bf16 [N, K], read only
 * N, K, G in   as for quantize_int4_grouped
 * W_hat   out  bf16 [N, K]; must not overlap W
 */
w4_status fake_quant_int4_grouped(const uint16_t *W, int64_t N, int64_t K, int64_t G,
                                  uint16_t *W_hat, hipStream_t stream);

/*
 * w4a16_linear - y = x . w_hat^T (+ bias), the bf16-int4 mixed-precision
 * linear ("Optimum Quanto": accelerated bf16-int4 matmul; accumulation wider
 * than the inputs, then dequantization; bias kept in float).
 *
 * Each output is accumulated in float32 as
 *   sum_g ( s[n][g] * sum_{k in g} x[m][k] * q[n][k] + z[n][g] * sum_{k in g} x[m][k] )
 * plus bias[n] (if bias != NULL), then rounded to bf16 (nearest, ties to
 * even). w_hat is never rounded to bf16. The summation order is the
 * kernel's own, so results agree with an exact evaluation to float32
 * accumulation error, not bit for bit.
 *
 * x       in   bf16 [M, K]; may be NULL when M == 0
 * M       in   M >= 0; M == 0 returns W4_OK and launches nothing
 * codes, scales, zeros   in   as produced by quantize_int4_grouped
 * bias    in   bf16 [N] or NULL
 * N, K, G in   as for quantize_int4_grouped
 * y       out  bf16 [M, N]; may be NULL when M == 0
 */
w4_status w4a16_linear(const uint16_t *x, int64_t M, const uint8_t *codes,
                       const uint16_t *scales, const uint16_t *zeros,
                       const uint16_t *bias, int64_t N, int64_t K, int64_t G,
                       uint16_t *y, hipStream_t stream);

/*
 * w4a16_linear_select - w4a16_linear with an explicit kernel choice, so both
 * kernels can be exercised at the same M. Same arguments and results as
 * w4a16_linear; returns W4_ERR_PATH if path is W4_PATH_GEMV and M > 16 or
 * K > W4_GEMV_MAX_K, or if path is not a w4_path value.
 */
w4_status w4a16_linear_select(const uint16_t *x, int64_t M,
                              const uint8_t *codes, const uint16_t *scales,
                              const uint16_t *zeros, const uint16_t *bias,
                              int64_t N, int64_t K, int64_t G, uint16_t *y,
                              int path, hipStream_t stream);

/*
 * Pre-shuffled weight layout. The pages' int4 paths ship kernel-specific
 * packings beside the plain one (torchao README ("PyTorch原生训练至推理模型优化"),
 * int4 weight quantization: the weight-only config takes a packing format,
 * tile-packed for one accelerator and plain for another; torchao release
 * notes, "New Features": a pre-shuffled int4 tensor). They give no format;
 * this one is the library's own, made for its gfx950 kernels. The plain
 * layout stays the interchange format; the pre-shuffled one holds the same
 * q, s and z and gives the same results.
 *
 *   codes_ps [N, K/2] bytes: each 4-byte word (little endian) holds the
 *            codes of k = 8j .. 8j+7 of its row with nibble i = q[8j + 2i]
 *            and nibble 4 + i = q[8j + 2i + 1], i = 0..3 (even k in the low
 *            half-word, odd k in the high one)
 *   sz       uint32 [N, K/G]: s[n][g] | z[n][g] << 16 (bf16 bits)
 *
 * repack_int4_preshuffled - plain (codes, scales, zeros) -> (codes_ps, sz).
 * A pure rearrangement: bit-exact and deterministic.
 *
 * codes, scales, zeros   in   as produced by quantize_int4_grouped
 * N, K, G  in   as for quantize_int4_grouped
 * codes_ps out  [N, K/2] bytes; sz out uint32 [N, K/G]; no overlap with the
 *               inputs or each other (W4_ERR_ALIAS)
 */
w4_status repack_int4_preshuffled(const uint8_t *codes, const uint16_t *scales,
                                  const uint16_t *zeros, int64_t N, int64_t K, int64_t G,
                                  uint8_t *codes_ps, uint32_t *sz, hipStream_t stream);

/*
 * w4a16_linear_preshuffled - w4a16_linear on the pre-shuffled layout: same
 * arguments (codes_ps and sz in place of codes, scales and zeros), same
 * validation and status codes, the same result to float32 accumulation
 * error. sz must be 16-byte aligned.
 */
w4_status w4a16_linear_preshuffled(const uint16_t *x, int64_t M, const uint8_t *codes_ps,
                                   const uint32_t *sz, const uint16_t *bias, int64_t N,
                                   int64_t K, int64_t G, uint16_t *y, hipStream_t stream);

/* w4a16_linear_preshuffled with an explicit kernel path, as w4a16_linear_select. */
w4_status w4a16_linear_preshuffled_select(const uint16_t *x, int64_t M, const uint8_t *codes_ps,
                                          const uint32_t *sz, const uint16_t *bias, int64_t N,
                                          int64_t K, int64_t G, uint16_t *y, int path,
                                          hipStream_t stream);

/*
 * W4A8: int8 activations with the int4 weights above, on the int8 matrix
 * cores (torchao README ("PyTorch原生训练至推理模型优化"): int8 dynamic
 * activations with group-wise int4 weights, the edge and QAT configuration,
 * group size 32 in its example; "Optimum Quanto", "Design overview /
 * Tensors": int8 takes a symmetric projection per tensor or per channel;
 * the per-token reading is this library's, stated in its design notes).
 *
 * quantize_act_int8 - per-token (per row) symmetric int8 of x:
 *   a = max_k |x[m][k]|;  sx[m] = fl32(a / 127);
 *   x8[m][k] = clamp(rne(fl32(x[m][k] / sx[m])), -127, 127), 0 where a == 0
 * (IEEE binary32 division, ties to even). Bit-exact and deterministic.
 *
 * x   in   bf16 [M, K]; M >= 0 (0: nothing is launched, pointers may be
 *          NULL), K a multiple of 32
 * x8  out  int8 [M, K] (natural k order); sx out float32 [M]; neither may
 *          overlap x or the other
 */
w4_status quantize_act_int8(const uint16_t *x, int64_t M, int64_t K, int8_t *x8, float *sx,
                            hipStream_t stream);

/*
 * w4a8_linear - y = sx[m] * sum_g ( s[n][g] * P + z[n][g] * X ) (+ bias[n]),
 * P = sum_{k in g} x8[m][k] q[n][k], X = sum_{k in g} x8[m][k], per output:
 * P and X are exact int32 sums; the fold over groups, the scale by sx and
 * the bias are float32, then y is rounded to bf16 (nearest, ties to even).
 * Same weights (codes, scales, zeros) as w4a16_linear. With K <= 2^24,
 * M <= 8 runs a dot-product kernel on the vector ALUs (v_dot4_i32_i8), and
 * so do 8-row slices of larger M while the tiled int8-MFMA kernel's
 * 128 x 128 tiles would be too few to fill the chip (the rule of
 * w4a16_linear); otherwise the tiled kernel. K must be a multiple of 64.
 *
 * x8, sx  in   from quantize_act_int8 (may be NULL when M == 0)
 * codes, scales, zeros, bias, N, K, G, y   as for w4a16_linear
 */
w4_status w4a8_linear(const int8_t *x8, const float *sx, int64_t M, const uint8_t *codes,
                      const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                      int64_t N, int64_t K, int64_t G, uint16_t *y, hipStream_t stream);

/*
 * Int8 weight-only (torchao README and its diffusers example: an int8
 * weight-only config with per-group granularity, group size 128; the
 * release notes' 0.9.0 API change names the same config with group_size=128;
 * "Optimum Quanto", "Design overview / Tensors": int8 takes a symmetric
 * projection).
 *
 * quantize_int8_grouped - per group g of G consecutive k of row n:
 *   a = max |v|;  s = bf16_rne(fl32(a / 127));
 *   q = clamp(rne(fl32(v / s)), -127, 127), 0 when s == 0
 * (IEEE binary32 division by the stored scale, ties to even). Bit-exact.
 *
 * W       in   bf16 [N, K]; N, K, G as for quantize_int4_grouped
 * codes8  out  int8 [N, K]; scales out bf16 [N, K/G]; no overlaps
 */
w4_status quantize_int8_grouped(const uint16_t *W, int64_t N, int64_t K, int64_t G,
                                int8_t *codes8, uint16_t *scales, hipStream_t stream);

/*
 * w8a16_linear - y = x . w_hat^T (+ bias), w_hat = q * s (exact), each output
 * accumulated in float32 as sum_g s[n][g] * sum_{k in g} x[m][k] q[n][k] and
 * rounded to bf16. With K <= 2^24, M <= 4 runs a dot-product kernel on the
 * vector ALUs and 5 <= M <= 16 a split-K matrix-core kernel, and so do
 * 16-row slices of larger M while the tiled MFMA kernel's 128 x 128 tiles
 * would be too few to fill the chip (the rule of w4a16_linear); other shapes
 * the tiled MFMA kernel. K must be a multiple of 64. Arguments as w4a16_linear
 * with codes8 and scales from quantize_int8_grouped.
 */
w4_status w8a16_linear(const uint16_t *x, int64_t M, const int8_t *codes8,
                       const uint16_t *scales, const uint16_t *bias, int64_t N, int64_t K,
                       int64_t G, uint16_t *y, hipStream_t stream);

/*
 * quantize_int4_grouped_batch - quantize_int4_grouped on several weights in
 * one launch (e.g. the layers of a transformer block), all with the same G.
 * Results are bit-identical to one quantize_int4_grouped call per job.
 *
 * jobs   in  HOST array of njobs descriptors (read during the call only);
 *            each job's pointers and shapes follow quantize_int4_grouped
 * njobs  in  1 <= njobs <= W4_QUANT_BATCH_MAX
 * Errors: as quantize_int4_grouped for any job (nothing is launched then),
 * W4_ERR_SHAPE for njobs out of range, W4_ERR_ALIAS when an output overlaps
 * any input or output of any job.
 */
#define W4_QUANT_BATCH_MAX 8
typedef struct {
    const uint16_t *W;   /* bf16 [N, K] */
    int64_t N, K;
    uint8_t *codes;      /* [N, K/2] */
    uint16_t *scales;    /* bf16 [N, K/G] */
    uint16_t *zeros;     /* bf16 [N, K/G] */
} w4_quant_job;

w4_status quantize_int4_grouped_batch(const w4_quant_job *jobs, int64_t njobs, int64_t G,
                                      hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char *w4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
