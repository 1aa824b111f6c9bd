// C interface of the W4A16 library: argument validation and kernel dispatch.
// Every check runs before any HIP call; a failed check launches and writes
// nothing. Declarations and the meaning of every argument: include/w4a16.h.
#include "w4a16.h"
#include "w4_launch.h"

#include <stdint.h>

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 30;      // N and K
constexpr int64_t kMaxM = int64_t(1) << 23;        // M (grid rows of the GEMM)
constexpr int64_t kMaxElems = int64_t(1) << 40;    // N*K, M*K, M*N

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_group(int64_t G) { return G == 32 || G == 64 || G == 128; }

// [p, p + bytes) overlaps [q, q + qbytes)?
bool overlap(const void *p, int64_t bytes, const void *q, int64_t qbytes) {
    if (!p || !q || bytes <= 0 || qbytes <= 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uintptr_t b = reinterpret_cast<uintptr_t>(q);
    return a < b + static_cast<uintptr_t>(qbytes) && b < a + static_cast<uintptr_t>(bytes);
}

w4_status check_nkg(int64_t N, int64_t K, int64_t G) {
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return W4_ERR_SHAPE;
    if (!valid_group(G)) return W4_ERR_GROUP;
    if (K % G != 0) return W4_ERR_SHAPE;
    if (N * K > kMaxElems) return W4_ERR_SHAPE;
    return W4_OK;
}

// M > 16 whose GEMM grid would leave most compute units idle: the decode
// GEMV on ceil(M / 16) row slices reads the weight once per slice, but each
// slice streams at close to the decode rate, while a GEMM of T 128 x 128 tiles
// on C compute units runs at about T / C of its full rate. Measured on the
// Llama-3-8B decode shapes (M = 17..128) the slices win while their count
// stays below about 0.8 C / T; the rule keeps a margin (0.6 C / T).
bool slices_pay(int64_t M, int64_t N, int64_t slice_rows) {
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    const int64_t slices = (M + slice_rows - 1) / slice_rows;
    return 10 * slices * tiles <= 6 * static_cast<int64_t>(w4::compute_units());
}
bool gemv_slices_pay(int64_t M, int64_t N, int64_t K) {
    if (M <= W4_GEMV_MAX_M || K > W4_GEMV_MAX_K) return false;
    return slices_pay(M, N, W4_GEMV_MAX_M);
}

// One implementation for both weight layouts: the plain one (scales and
// zeros, sz == NULL) and the pre-shuffled one (sz, scales == zeros == NULL).
w4_status linear_impl(const uint16_t *x, int64_t M, const uint8_t *codes,
                      const uint16_t *scales, const uint16_t *zeros, const uint32_t *sz,
                      const uint16_t *bias, int64_t N, int64_t K, int64_t G,
                      uint16_t *y, int path, hipStream_t stream) {
    const bool pk = sz != nullptr;
    if (!codes || (!pk && (!scales || !zeros))) return W4_ERR_NULL;
    if (M > 0 && (!x || !y)) return W4_ERR_NULL;
    if (M < 0 || M > kMaxM) return W4_ERR_SHAPE;
    const w4_status st = check_nkg(N, K, G);
    if (st != W4_OK) return st;
    if (M * K > kMaxElems || M * N > kMaxElems) return W4_ERR_SHAPE;
    if (path != W4_PATH_AUTO && path != W4_PATH_GEMV && path != W4_PATH_GEMM)
        return W4_ERR_PATH;
    if (path == W4_PATH_GEMV && (M > W4_GEMV_MAX_M || K > W4_GEMV_MAX_K)) return W4_ERR_PATH;
    if (!aligned16(codes) || (bias && !aligned16(bias))) return W4_ERR_ALIGN;
    if (pk ? !aligned16(sz) : (!aligned16(scales) || !aligned16(zeros))) return W4_ERR_ALIGN;
    if (M > 0 && (!aligned16(x) || !aligned16(y))) return W4_ERR_ALIGN;
    if (M == 0) return W4_OK;
    const int64_t ybytes = 2 * M * N, gbytes = 2 * N * (K / G);
    if (overlap(y, ybytes, x, 2 * M * K) || overlap(y, ybytes, codes, N * K / 2) ||
        overlap(y, ybytes, scales, gbytes) || overlap(y, ybytes, zeros, gbytes) ||
        overlap(y, ybytes, sz, 2 * gbytes) || overlap(y, ybytes, bias, 2 * N))
        return W4_ERR_ALIAS;

    const bool gemv = path == W4_PATH_GEMV ||
                      (path == W4_PATH_AUTO && M <= W4_GEMV_MAX_M && K <= W4_GEMV_MAX_K);
    if (!gemv && path == W4_PATH_AUTO && gemv_slices_pay(M, N, K)) {
        // a few 16-row slices through the decode GEMV (each reads the weight
        // once) instead of a GEMM grid too small to fill the chip
        for (int64_t m0 = 0; m0 < M; m0 += W4_GEMV_MAX_M) {
            const int64_t mc = M - m0 < W4_GEMV_MAX_M ? M - m0 : W4_GEMV_MAX_M;
            const hipError_t e = w4::launch_gemv(x + m0 * K, static_cast<int>(mc), codes, scales,
                                                 zeros, sz, bias, N, K, static_cast<int>(G),
                                                 y + m0 * N, stream);
            if (e != hipSuccess) return W4_ERR_HIP;
        }
        return W4_OK;
    }
    const hipError_t e =
        gemv ? w4::launch_gemv(x, static_cast<int>(M), codes, scales, zeros, sz, bias, N, K,
                               static_cast<int>(G), y, stream)
             : w4::launch_gemm(x, M, codes, scales, zeros, sz, bias, N, K, static_cast<int>(G),
                               y, stream);
    return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

} // namespace

extern "C" {

w4_status quantize_int4_grouped(const uint16_t *W, int64_t N, int64_t K, int64_t G,
                                uint8_t *codes, uint16_t *scales, uint16_t *zeros,
                                hipStream_t stream) {
    if (!W || !codes || !scales || !zeros) return W4_ERR_NULL;
    const w4_status st = check_nkg(N, K, G);
    if (st != W4_OK) return st;
    if (!aligned16(W) || !aligned16(codes) || !aligned16(scales) || !aligned16(zeros))
        return W4_ERR_ALIGN;
    const int64_t wbytes = 2 * N * K, cbytes = N * K / 2, sbytes = 2 * N * (K / G);
    if (overlap(codes, cbytes, W, wbytes) || overlap(scales, sbytes, W, wbytes) ||
        overlap(zeros, sbytes, W, wbytes) || overlap(codes, cbytes, scales, sbytes) ||
        overlap(codes, cbytes, zeros, sbytes) || overlap(scales, sbytes, zeros, sbytes))
        return W4_ERR_ALIAS;
    const hipError_t e = w4::launch_quantize(W, N, K, static_cast<int>(G), codes, scales,
                                             zeros, stream);
    return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

w4_status fake_quant_int4_grouped(const uint16_t *W, int64_t N, int64_t K, int64_t G,
                                  uint16_t *W_hat, hipStream_t stream) {
    if (!W || !W_hat) return W4_ERR_NULL;
    const w4_status st = check_nkg(N, K, G);
    if (st != W4_OK) return st;
    if (!aligned16(W) || !aligned16(W_hat)) return W4_ERR_ALIGN;
    if (overlap(W_hat, 2 * N * K, W, 2 * N * K)) return W4_ERR_ALIAS;
    const hipError_t e = w4::launch_fake_quant(W, N, K, static_cast<int>(G), W_hat, stream);
    return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

w4_status w4a16_linear(const uint16_t *x, int64_t M, const uint8_t *codes,
                       const uint16_t *scales, const uint16_t *zeros,
                       const uint16_t *bias, int64_t N, int64_t K, int64_t G,
                       uint16_t *y, hipStream_t stream) {
    return linear_impl(x, M, codes, scales, zeros, nullptr, bias, N, K, G, y, W4_PATH_AUTO,
                       stream);
}

w4_status w4a16_linear_select(const uint16_t *x, int64_t M, const uint8_t *codes,
                              const uint16_t *scales, const uint16_t *zeros,
                              const uint16_t *bias, int64_t N, int64_t K, int64_t G,
                              uint16_t *y, int path, hipStream_t stream) {
    return linear_impl(x, M, codes, scales, zeros, nullptr, bias, N, K, G, y, path, stream);
}

w4_status repack_int4_preshuffled(const uint8_t *codes, const uint16_t *scales,
                                  const uint16_t *zeros, int64_t N, int64_t K, int64_t G,
                                  uint8_t *codes_ps, uint32_t *sz, hipStream_t stream) {
    if (!codes || !scales || !zeros || !codes_ps || !sz) return W4_ERR_NULL;
    const w4_status st = check_nkg(N, K, G);
    if (st != W4_OK) return st;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(zeros) || !aligned16(codes_ps) ||
        !aligned16(sz))
        return W4_ERR_ALIGN;
    const int64_t cbytes = N * K / 2, gbytes = 2 * N * (K / G);
    const void *in[3] = {codes, scales, zeros};
    const int64_t inb[3] = {cbytes, gbytes, gbytes};
    for (int i = 0; i < 3; ++i)
        if (overlap(codes_ps, cbytes, in[i], inb[i]) || overlap(sz, 2 * gbytes, in[i], inb[i]))
            return W4_ERR_ALIAS;
    if (overlap(codes_ps, cbytes, sz, 2 * gbytes)) return W4_ERR_ALIAS;
    const hipError_t e = w4::launch_repack(codes, scales, zeros, N, K, static_cast<int>(G),
                                           codes_ps, sz, stream);
    return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

w4_status w4a16_linear_preshuffled(const uint16_t *x, int64_t M, const uint8_t *codes_ps,
                                   const uint32_t *sz, const uint16_t *bias, int64_t N,
                                   int64_t K, int64_t G, uint16_t *y, hipStream_t stream) {
    if (!sz) return W4_ERR_NULL;
    return linear_impl(x, M, codes_ps, nullptr, nullptr, sz, bias, N, K, G, y, W4_PATH_AUTO,
                       stream);
}

w4_status w4a16_linear_preshuffled_select(const uint16_t *x, int64_t M, const uint8_t *codes_ps,
                                          const uint32_t *sz, const uint16_t *bias, int64_t N,
                                          int64_t K, int64_t G, uint16_t *y, int path,
                                          hipStream_t stream) {
    if (!sz) return W4_ERR_NULL;
    return linear_impl(x, M, codes_ps, nullptr, nullptr, sz, bias, N, K, G, y, path, stream);
}

w4_status quantize_act_int8(const uint16_t *x, int64_t M, int64_t K, int8_t *x8, float *sx,
                            hipStream_t stream) {
    if (M < 0 || M > kMaxM || K < 32 || K > kMaxDim || K % 32 != 0 || M * K > kMaxElems)
        return W4_ERR_SHAPE;
    if (M == 0) return W4_OK;
    if (!x || !x8 || !sx) return W4_ERR_NULL;
    if (!aligned16(x) || !aligned16(x8) || !aligned16(sx)) return W4_ERR_ALIGN;
    if (overlap(x8, M * K, x, 2 * M * K) || overlap(sx, 4 * M, x, 2 * M * K) ||
        overlap(sx, 4 * M, x8, M * K))
        return W4_ERR_ALIAS;
    const hipError_t e = w4::launch_act_quant(x, M, K, x8, sx, stream);
    return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

w4_status w4a8_linear(const int8_t *x8, const float *sx, int64_t M, const uint8_t *codes,
                      const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                      int64_t N, int64_t K, int64_t G, uint16_t *y, hipStream_t stream) {
    if (!codes || !scales || !zeros) return W4_ERR_NULL;
    if (M > 0 && (!x8 || !sx || !y)) return W4_ERR_NULL;
    if (M < 0 || M > kMaxM) return W4_ERR_SHAPE;
    const w4_status st = check_nkg(N, K, G);
    if (st != W4_OK) return st;
    if (K % 64 != 0 || M * K > kMaxElems || M * N > kMaxElems) return W4_ERR_SHAPE;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(zeros) ||
        (bias && !aligned16(bias)))
        return W4_ERR_ALIGN;
    if (M > 0 && (!aligned16(x8) || !aligned16(sx) || !aligned16(y))) return W4_ERR_ALIGN;
    if (M == 0) return W4_OK;
    const int64_t ybytes = 2 * M * N, gbytes = 2 * N * (K / G);
    if (overlap(y, ybytes, x8, M * K) || overlap(y, ybytes, sx, 4 * M) ||
        overlap(y, ybytes, codes, N * K / 2) || overlap(y, ybytes, scales, gbytes) ||
        overlap(y, ybytes, zeros, gbytes) || overlap(y, ybytes, bias, 2 * N))
        return W4_ERR_ALIAS;
    if (K <= w4::A8_ROWS_MAX_K &&
        (M <= w4::A8_ROWS_MAX_M || slices_pay(M, N, w4::A8_ROWS_MAX_M))) {
        // the decode kernel, on slices of up to A8_ROWS_MAX_M rows when the
        // GEMM's tiles would be too few to fill the chip (as for w4a16_linear)
        for (int64_t m0 = 0; m0 < M; m0 += w4::A8_ROWS_MAX_M) {
            const int64_t mc = M - m0 < w4::A8_ROWS_MAX_M ? M - m0 : w4::A8_ROWS_MAX_M;
            const hipError_t e = w4::launch_w4a8_rows(x8 + m0 * K, sx + m0, mc, codes, scales,
                                                      zeros, bias, N, K, static_cast<int>(G),
                                                      y + m0 * N, stream);
            if (e != hipSuccess) return W4_ERR_HIP;
        }
        return W4_OK;
    }
    const hipError_t e = w4::launch_w4a8_gemm(x8, sx, M, codes, scales, zeros, bias, N, K,
                                              static_cast<int>(G), y, stream);
    return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

w4_status quantize_int4_grouped_batch(const w4_quant_job *jobs, int64_t njobs, int64_t G,
                                      hipStream_t stream) {
    if (!jobs) return W4_ERR_NULL;
    if (njobs < 1 || njobs > W4_QUANT_BATCH_MAX) return W4_ERR_SHAPE;
    if (!valid_group(G)) return W4_ERR_GROUP;
    for (int64_t j = 0; j < njobs; ++j) {
        const w4_quant_job &q = jobs[j];
        if (!q.W || !q.codes || !q.scales || !q.zeros) return W4_ERR_NULL;
        const w4_status st = check_nkg(q.N, q.K, G);
        if (st != W4_OK) return st;
        if (!aligned16(q.W) || !aligned16(q.codes) || !aligned16(q.scales) || !aligned16(q.zeros))
            return W4_ERR_ALIGN;
    }
    // no output may overlap any input or output of any job
    for (int64_t j = 0; j < njobs; ++j) {
        const w4_quant_job &a = jobs[j];
        const int64_t cb = a.N * a.K / 2, gb = 2 * a.N * (a.K / G);
        const void *outs[3] = {a.codes, a.scales, a.zeros};
        const int64_t osz[3] = {cb, gb, gb};
        for (int64_t i = 0; i < njobs; ++i) {
            const w4_quant_job &b = jobs[i];
            const int64_t cbi = b.N * b.K / 2, gbi = 2 * b.N * (b.K / G);
            for (int o = 0; o < 3; ++o) {
                if (overlap(outs[o], osz[o], b.W, 2 * b.N * b.K)) return W4_ERR_ALIAS;
                if (i == j) continue;
                if (overlap(outs[o], osz[o], b.codes, cbi) ||
                    overlap(outs[o], osz[o], b.scales, gbi) ||
                    overlap(outs[o], osz[o], b.zeros, gbi))
                    return W4_ERR_ALIAS;
            }
        }
        if (overlap(a.codes, cb, a.scales, gb) || overlap(a.codes, cb, a.zeros, gb) ||
            overlap(a.scales, gb, a.zeros, gb))
            return W4_ERR_ALIAS;
    }
    const hipError_t e = w4::launch_quantize_batch(jobs, static_cast<int>(njobs),
                                                   static_cast<int>(G), stream);
    return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

w4_status quantize_int8_grouped(const uint16_t *W, int64_t N, int64_t K, int64_t G,
                                int8_t *codes8, uint16_t *scales, hipStream_t stream) {
    if (!W || !codes8 || !scales) return W4_ERR_NULL;
    const w4_status st = check_nkg(N, K, G);
    if (st != W4_OK) return st;
    if (!aligned16(W) || !aligned16(codes8) || !aligned16(scales)) return W4_ERR_ALIGN;
    const int64_t wbytes = 2 * N * K, gbytes = 2 * N * (K / G);
    if (overlap(codes8, N * K, W, wbytes) || overlap(scales, gbytes, W, wbytes) ||
        overlap(codes8, N * K, scales, gbytes))
        return W4_ERR_ALIAS;
    const hipError_t e = w4::launch_quantize8(W, N, K, static_cast<int>(G), codes8, scales,
                                              stream);
    return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

w4_status w8a16_linear(const uint16_t *x, int64_t M, const int8_t *codes8,
                       const uint16_t *scales, const uint16_t *bias, int64_t N, int64_t K,
                       int64_t G, uint16_t *y, hipStream_t stream) {
    if (!codes8 || !scales) return W4_ERR_NULL;
    if (M > 0 && (!x || !y)) return W4_ERR_NULL;
    if (M < 0 || M > kMaxM) return W4_ERR_SHAPE;
    const w4_status st = check_nkg(N, K, G);
    if (st != W4_OK) return st;
    if (K % 64 != 0 || M * K > kMaxElems || M * N > kMaxElems) return W4_ERR_SHAPE;
    if (!aligned16(codes8) || !aligned16(scales) || (bias && !aligned16(bias)))
        return W4_ERR_ALIGN;
    if (M > 0 && (!aligned16(x) || !aligned16(y))) return W4_ERR_ALIGN;
    if (M == 0) return W4_OK;
    const int64_t ybytes = 2 * M * N;
    if (overlap(y, ybytes, x, 2 * M * K) || overlap(y, ybytes, codes8, N * K) ||
        overlap(y, ybytes, scales, 2 * N * (K / G)) || overlap(y, ybytes, bias, 2 * N))
        return W4_ERR_ALIAS;
    // decode kernels: the vector-ALU rows for M <= W8_ROWS_MAX_M, the split-K
    // matrix-core GEMV up to 16 rows (inside launch_w8a16)
    auto decode = [&](const uint16_t *xs, int64_t mc, uint16_t *ys) {
        return mc <= w4::W8_ROWS_MAX_M && K <= w4::W8_ROWS_MAX_K
                   ? w4::launch_w8a16_rows(xs, mc, codes8, scales, bias, N, K,
                                           static_cast<int>(G), ys, stream)
                   : w4::launch_w8a16(xs, mc, codes8, scales, bias, N, K, static_cast<int>(G),
                                      ys, stream);
    };
    if (M > W4_GEMV_MAX_M && K <= W4_GEMV_MAX_K && slices_pay(M, N, W4_GEMV_MAX_M)) {
        // 16-row slices instead of a GEMM grid too small to fill the chip
        // (the rule of w4a16_linear)
        for (int64_t m0 = 0; m0 < M; m0 += W4_GEMV_MAX_M) {
            const int64_t mc = M - m0 < W4_GEMV_MAX_M ? M - m0 : W4_GEMV_MAX_M;
            if (decode(x + m0 * K, mc, y + m0 * N) != hipSuccess) return W4_ERR_HIP;
        }
        return W4_OK;
    }
    return decode(x, M, y) == hipSuccess ? W4_OK : W4_ERR_HIP;
}

const char *w4_status_string(int status) {
    switch (status) {
    case W4_OK: return "W4_OK: success";
    case W4_ERR_NULL: return "W4_ERR_NULL: a required pointer is NULL";
    case W4_ERR_SHAPE: return "W4_ERR_SHAPE: invalid or oversized N, K, M, or K % G != 0";
    case W4_ERR_GROUP: return "W4_ERR_GROUP: group size must be 32, 64 or 128";
    case W4_ERR_ALIGN: return "W4_ERR_ALIGN: pointers must be 16-byte aligned";
    case W4_ERR_HIP: return "W4_ERR_HIP: the HIP runtime reported a launch error";
    case W4_ERR_ALIAS: return "W4_ERR_ALIAS: an output overlaps an input";
    case W4_ERR_PATH: return "W4_ERR_PATH: the requested kernel path cannot serve this call";
    default: return "unknown w4_status";
    }
}

} // extern "C"
