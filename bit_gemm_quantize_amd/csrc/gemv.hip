// Decode-path W4A16 GEMV (1 <= M <= 16) for gfx950.
//
// y[m][n] = sum_g ( s[n][g] * sum_{k in g} x[m][k] q[n][k]
//                 + z[n][g] * sum_{k in g} x[m][k] ) (+ bias[n])
// ("Optimum Quanto": bf16-int4 matmul, accumulated in float32 and
// dequantized afterwards; bias kept in float.)
//
// The kernel streams the packed codes once from HBM. Work split:
//   * a block owns 16*T output features (rows of the code matrix) and all
//     of K; its NW waves split K into contiguous runs of 128-wide chunks and
//     combine their partial sums through LDS at the end;
//   * per chunk, lane l (feature l%16, quarter kb = l/16) loads 16 bytes =
//     32 codes (k = 128c + 32kb ... +32) with one 128-bit load per tile, so a
//     wave load covers 64 contiguous bytes of each of 16 rows;
//   * codes are expanded in registers to the exact bf16 integers 128 + q and
//     fed with bf16 x to the 16x16x32 matrix-core op; M <= 16 rows of x fill
//     the A operand (rows >= M are zero);
//   * each MFMA must contract a single group, so for G = 64 / 32 the four
//     dwords a lane holds are first exchanged across the lane quarters
//     (permlane swaps) so that slot j of every quarter lies in one group;
//   * a second MFMA against an all-ones B gives sum_{k in g} x[m][k] in the
//     same lane layout; at the end of a group, in float32:
//         acc += s * acc_g + (z - 128 s) * xsum_g.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

// k offset (inside a 128-wide chunk) of the 8 codes lane quarter kb feeds to
// slot j, after the group-alignment exchange.
template <int G>
__device__ __forceinline__ int slot_koff(int j, int kb) {
    if constexpr (G == 128) {
        return kb * 32 + 8 * j;
    } else if constexpr (G == 64) {
        return 64 * (j >> 1) + 32 * (kb & 1) + 8 * (j & 1) + 16 * (kb >> 1);
    } else {
        return 32 * j + 8 * kb;
    }
}

// Exchange the four code dwords of a lane across the four 16-lane quarters
// so that slot j of every quarter belongs to one group.
//  G = 128: a chunk is one group, nothing to do.
//  G = 64 : quarters {0,1} hold group 0 and {2,3} group 1; swapping the
//           upper half of d0/d1 with the lower half of d2/d3 leaves slots
//           0,1 in group 0 and slots 2,3 in group 1.
//  G = 32 : a 4x4 transpose (quarter x dword): slot j <- quarter j.
template <int G>
__device__ __forceinline__ void align_groups(u32x4 &d) {
    if constexpr (G <= 64) {
        auto p02 = __builtin_amdgcn_permlane32_swap(d.x, d.z, false, false);
        auto p13 = __builtin_amdgcn_permlane32_swap(d.y, d.w, false, false);
        d.x = p02[0]; d.z = p02[1];
        d.y = p13[0]; d.w = p13[1];
    }
    if constexpr (G == 32) {
        auto p01 = __builtin_amdgcn_permlane16_swap(d.x, d.y, false, false);
        auto p23 = __builtin_amdgcn_permlane16_swap(d.z, d.w, false, false);
        d.x = p01[0]; d.y = p01[1];
        d.z = p23[0]; d.w = p23[1];
    }
}

template <int G, int T, int NW>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int N, int K, uint16_t *__restrict__ y) {
    constexpr int SLOTS_PER_GROUP = G / 32;    // 4, 2 or 1 slots per group
    __shared__ float red[NW][T][16][16];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nl = lane & 15;
    const int kb = lane >> 4;
    const int n_base = blockIdx.x * 16 * T;
    const int nchunk = (K + 127) >> 7;
    const int ngroups = K / G;
    const int c_begin = wave * nchunk / NW;
    const int c_end = (wave + 1) * nchunk / NW;

    const bool m_ok = nl < M;                  // A-operand row of this lane
    const uint16_t *xrow = x + static_cast<int64_t>(m_ok ? nl : 0) * K;

    const uint8_t *crow[T];
    int nrow[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        int n = n_base + 16 * t + nl;
        nrow[t] = n < N ? n : N - 1;           // clamp; results masked on store
        crow[t] = codes + static_cast<int64_t>(nrow[t]) * (K >> 1);
    }

    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 ones = bf16x8_ones();

    constexpr int U = 4;                       // chunks in flight per wave
    for (int c0 = c_begin; c0 < c_end; c0 += U) {
        u32x4 q[U][T];
        u32x4 a[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u;
            const int kq = c * 128 + kb * 32;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                q[u][t] = u32x4{0u, 0u, 0u, 0u};
                if (c < c_end && kq < K)
                    q[u][t] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4 *>(crow[t] + (kq >> 1)));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ka = c * 128 + slot_koff<G>(j, kb);
                a[u][j] = u32x4{0u, 0u, 0u, 0u};
                if (c < c_end && m_ok && ka < K)
                    a[u][j] = *reinterpret_cast<const u32x4 *>(xrow + ka);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u;
            if (c >= c_end) break;
#pragma unroll
            for (int t = 0; t < T; ++t) align_groups<G>(q[u][t]);
            f32x4 accg[T];
            f32x4 xsg = zero4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool first = (j % SLOTS_PER_GROUP) == 0;
                const bf16x8 av = as_bf16x8(a[u][j]);
                xsg = mfma16x16x32(av, ones, first ? zero4 : xsg);
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    uint32_t b[4];
                    unpack8_bias128(q[u][t][j], b);
                    accg[t] = mfma16x16x32(av, as_bf16x8(b[0], b[1], b[2], b[3]),
                                           first ? zero4 : accg[t]);
                }
                if ((j % SLOTS_PER_GROUP) == SLOTS_PER_GROUP - 1) {
                    const int g = (c * 128 + 32 * (j - (SLOTS_PER_GROUP - 1))) / G;
                    if (g < ngroups) {
#pragma unroll
                        for (int t = 0; t < T; ++t) {
                            const int64_t si = static_cast<int64_t>(nrow[t]) * ngroups + g;
                            const float s = bf16_to_f32(scales[si]);
                            const float z = bf16_to_f32(zeros[si]);
                            const float zz = fmaf(-128.0f, s, z);
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                acc[t][i] = fmaf(s, accg[t][i], fmaf(zz, xsg[i], acc[t][i]));
                        }
                    }
                }
            }
        }
    }

    // Combine the waves' partial sums; lane holds rows 4*kb + i, column nl.
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][t][4 * kb + i][nl] = acc[t][i];
    __syncthreads();
    for (int e = threadIdx.x; e < T * M * 16; e += NW * 64) {
        const int t = e / (M * 16);
        const int r = e - t * (M * 16);
        const int m = r >> 4;
        const int nn = r & 15;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red[w][t][m][nn];
        const int n = n_base + 16 * t + nn;
        if (n < N) {
            if (bias) sum += bf16_to_f32(bias[n]);
            y[static_cast<int64_t>(m) * N + n] = static_cast<uint16_t>(f32_to_bf16_rne(sum));
        }
    }
}

template <int G>
hipError_t launch_gemv_g(const uint16_t *x, int M, const uint8_t *codes,
                         const uint16_t *scales, const uint16_t *zeros,
                         const uint16_t *bias, int N, int K, uint16_t *y,
                         hipStream_t stream) {
    constexpr int T = 1, NW = 4;
    const dim3 grid((N + 16 * T - 1) / (16 * T)), block(NW * 64);
    gemv_kernel<G, T, NW><<<grid, block, 0, stream>>>(x, M, codes, scales, zeros,
                                                      bias, N, K, y);
    return hipGetLastError();
}

} // namespace

hipError_t launch_gemv(const uint16_t *x, int M, const uint8_t *codes,
                       const uint16_t *scales, const uint16_t *zeros,
                       const uint16_t *bias, int64_t N, int64_t K, int G,
                       uint16_t *y, hipStream_t stream) {
    const int n = static_cast<int>(N), k = static_cast<int>(K);
    switch (G) {
    case 32: return launch_gemv_g<32>(x, M, codes, scales, zeros, bias, n, k, y, stream);
    case 64: return launch_gemv_g<64>(x, M, codes, scales, zeros, bias, n, k, y, stream);
    case 128: return launch_gemv_g<128>(x, M, codes, scales, zeros, bias, n, k, y, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace w4
