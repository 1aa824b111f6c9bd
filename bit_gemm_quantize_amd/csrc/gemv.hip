// Decode-path W4A16 GEMV (1 <= M <= 16) for gfx950.
//
// y[m][n] = sum_g ( s[n][g] * sum_{k in g} x[m][k] q[n][k]
//                 + z[n][g] * sum_{k in g} x[m][k] ) (+ bias[n])
// ("Optimum Quanto": bf16-int4 matmul, accumulated in float32 and
// dequantized afterwards; bias kept in float.)
//
// The kernel streams the packed codes once from HBM. Work split:
//   * a block owns 16 output features (rows of the code matrix) and all of
//     K; its 8 waves split K into contiguous runs of 128-wide chunks and
//     combine their partial sums through LDS at the end;
//   * x[0:M, :] is staged once per block in LDS (in phases of columns when
//     M*K does not fit) and read from there as the MFMA A operand;
//   * per chunk, lane l (feature l%16, quarter kb = l/16) loads 16 bytes =
//     32 codes (k = 128c + 32kb ... +32) with one 128-bit load, so a wave
//     load covers 64 contiguous bytes of each of 16 rows; the codes, scales
//     and zero-points of the next batch of chunks are in flight while the
//     current batch is computed;
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

constexpr int GV_WAVES = 8;              // waves per block (split of K)
constexpr int GV_X_ELEMS = 32768;        // bf16 elements of x staged in LDS

// Codes, scales and zero-points of U consecutive chunks of one lane.
template <int G, int U>
struct Batch {
    u32x4 q[U];
    uint16_t s[U][128 / G];
    uint16_t z[U][128 / G];
};

template <int G, int NW>
__global__ __launch_bounds__(NW * 64, 2) void gemv_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int N, int K, uint16_t *__restrict__ y) {
    constexpr int SPG = G / 32;                 // slots per group: 4, 2 or 1
    constexpr int GPC = 128 / G;                // groups per chunk: 1, 2 or 4
    constexpr int U = G == 32 ? 2 : 4;          // chunks per batch
    __shared__ __attribute__((aligned(16))) uint16_t xl[GV_X_ELEMS];
    __shared__ float red[NW][16][17];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nl = lane & 15;
    const int kb = lane >> 4;
    const int n_base = blockIdx.x * 16;
    const int nchunk = (K + 127) >> 7;
    const int ngroups = K / G;
    const int n = n_base + nl < N ? n_base + nl : N - 1;   // clamped; masked on store
    const uint8_t *crow = codes + static_cast<int64_t>(n) * (K >> 1);
    const uint16_t *srow = scales + static_cast<int64_t>(n) * ngroups;
    const uint16_t *zrow = zeros + static_cast<int64_t>(n) * ngroups;
    // A-operand row of this lane. Rows >= M of the MFMA only feed outputs
    // that are never stored, so they repeat row M-1 instead of being zeroed.
    const int mrow = nl < M ? nl : M - 1;
    const Unpack128 uc = unpack128_consts();

    // x is staged in LDS in phases of kp columns (all of K when it fits),
    // zero-padded to a whole chunk: codes past K (clamped reads below) then
    // meet x = 0 and contribute nothing.
    const int kp = min(nchunk * 128, (GV_X_ELEMS / M) & ~127);
    const int cpp = kp >> 7;                    // chunks per phase

    // Loads are unconditional (clamped addresses), so the compiler can count
    // the loads in flight and wait only for the batch being computed.
    auto load = [&](Batch<G, U> &b, int c, int c_last) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = min(c + u, c_last);
            const int kq = min(cc * 128 + kb * 32, K - 32);
            b.q[u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(crow + (kq >> 1)));
#pragma unroll
            for (int h = 0; h < GPC; ++h) {
                const int g = min(cc * GPC + h, ngroups - 1);
                b.s[u][h] = srow[g];
                b.z[u][h] = zrow[g];
            }
        }
    };

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const bf16x8 ones = bf16x8_ones();

    auto compute = [&](Batch<G, U> &b, int c, int c_end, int k_phase) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = c + u;
            if (cc >= c_end) break;             // uniform across the wave
            align_groups<G>(b.q[u]);
            f32x4 accg = zero4, xsg = zero4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool first = (j % SPG) == 0;
                const int ka = cc * 128 + slot_koff<G>(j, kb) - k_phase;
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(&xl[mrow * kp + ka]));
                uint32_t w[4];
                unpack8_bias128(b.q[u][j], w, uc);
                xsg = mfma16x16x32(a, ones, first ? zero4 : xsg);
                accg = mfma16x16x32(a, as_bf16x8(w[0], w[1], w[2], w[3]),
                                    first ? zero4 : accg);
                if ((j % SPG) == SPG - 1) {
                    const int h = j / SPG;
                    const float sv = bf16_to_f32(b.s[u][h]);
                    const float zv = bf16_to_f32(b.z[u][h]);
                    const float zz = fmaf(-128.0f, sv, zv);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[i] = fmaf(sv, accg[i], fmaf(zz, xsg[i], acc[i]));
                }
            }
        }
    };

    for (int k_phase = 0; k_phase < K; k_phase += kp) {
        const int pc0 = k_phase >> 7;
        const int pc1 = min(nchunk, pc0 + cpp);
        const int c_begin = pc0 + wave * (pc1 - pc0) / NW;
        const int c_end = pc0 + (wave + 1) * (pc1 - pc0) / NW;
        const int c_last = max(c_begin, c_end - 1);

        // issue this wave's first code loads before staging x
        Batch<G, U> b0, b1;
        load(b0, c_begin, c_last);

        // stage x[0:M, k_phase : k_phase + kp) (zero beyond K)
        if (k_phase > 0) __syncthreads();        // previous phase fully consumed
        const int kw = min(kp, ((K - k_phase + 127) >> 7) << 7);
        const int per_row = kw >> 3;            // 16-byte pieces per row
        for (int e = threadIdx.x; e < M * per_row; e += NW * 64) {
            const int m = e / per_row;
            const int kk = (e - m * per_row) * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (k_phase + kk < K)
                v = *reinterpret_cast<const u32x4 *>(x + static_cast<int64_t>(m) * K + k_phase + kk);
            *reinterpret_cast<u32x4 *>(&xl[m * kp + kk]) = v;
        }
        __syncthreads();

        int c = c_begin;
        while (c < c_end) {
            if (c + U < c_end) load(b1, c + U, c_last);
            compute(b0, c, c_end, k_phase);
            c += U;
            if (c >= c_end) break;
            if (c + U < c_end) load(b0, c + U, c_last);
            compute(b1, c, c_end, k_phase);
            c += U;
        }
    }

    // Combine the waves' partial sums; lane holds rows 4*kb + i, column nl.
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * kb + i][nl] = acc[i];
    __syncthreads();
    for (int e = threadIdx.x; e < M * 16; e += NW * 64) {
        const int m = e >> 4;
        const int nn = e & 15;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red[w][m][nn];
        const int col = n_base + nn;
        if (col < N) {
            if (bias) sum += bf16_to_f32(bias[col]);
            y[static_cast<int64_t>(m) * N + col] = static_cast<uint16_t>(f32_to_bf16_rne(sum));
        }
    }
}

template <int G>
hipError_t launch_gemv_g(const uint16_t *x, int M, const uint8_t *codes,
                         const uint16_t *scales, const uint16_t *zeros,
                         const uint16_t *bias, int N, int K, uint16_t *y,
                         hipStream_t stream) {
    const dim3 grid((N + 15) / 16), block(GV_WAVES * 64);
    gemv_kernel<G, GV_WAVES><<<grid, block, 0, stream>>>(x, M, codes, scales, zeros,
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
