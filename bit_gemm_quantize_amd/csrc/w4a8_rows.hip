// W4A8 decode GEMV for one to eight activation rows, on the vector ALUs
// (gfx950).
//
// Same result as the W4A8 GEMM: per output, with the weights' q, s, z and
// the per-token int8 activations x8, sx,
//   y[m][n] = sx[m] * sum_g ( s[n][g] * P_g + z[n][g] * X_g ) (+ bias[n])
//   P_g = sum_{k in g} x8[m][k] q[n][k],  X_g = sum_{k in g} x8[m][k]
// with P and X exact int32 sums, the fold and the scale by sx in float32.
//
// At M <= 8 a 128-row matrix-core tile is almost all padding. Here a wave
// takes R = 4 consecutive output rows and one 2048-wide K segment; lane l
// covers k = 2048 s + 32 l .. + 32 (16 code bytes of each row, one 16-byte
// load), so every code load of a row is 1 KB contiguous. A lane's 32 codes
// lie in one group (G >= 32). A code word (8 nibbles, even k low) splits
// into the even-k and odd-k bytes with one and and one shift-and; the x8
// bytes are split the same way once per wave segment (two byte permutes per
// 8 values) and the products run as v_dot4_i32_i8 (q in 0..15 is a
// non-negative int8). X_g comes from the same instruction against ones.
// Scales and zero-points: the segment's R x 2048/G values for the R rows
// come in P loads per lane and array and reach the lanes of each group by
// lane permutes. Partial sums meet across the wave with lane swaps and DPP,
// then across the segment waves of a row group in LDS.
#include "w4_device.h"
#include "w4_launch.h"
#include "w4_rows.h"

namespace w4 {

namespace {

constexpr int A8R_SEG = 2048;              // k per wave segment
constexpr int A8R_MAX_WAVES = 8;           // segment waves per row group
constexpr int A8R_R = 4;                   // output rows per wave

template <int G, int MR>
__global__ __launch_bounds__(A8R_MAX_WAVES * 64) void w4a8_gemv_rows_kernel(
    const int8_t *__restrict__ x8, const float *__restrict__ sx,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ zeros, const uint16_t *__restrict__ bias, int N, int K,
    uint16_t *__restrict__ y, int nseg, int nsb, int rg) {
    static_assert(MR >= 1 && MR <= A8_ROWS_MAX_M, "activation rows");
    constexpr int R = A8R_R;
    constexpr int GPS = A8R_SEG / G;              // groups per segment: 64, 32, 16
    constexpr int P = (R * GPS + 63) / 64;        // values per lane and array: 4, 2, 1
    constexpr int LPG = G / 32;                   // lanes per group
    __shared__ float red[A8R_MAX_WAVES * R * MR];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sw = wave % nsb, rgi = wave / nsb;
    const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * rg + rgi) * R;
    const uint32_t rows = static_cast<uint32_t>(max<int64_t>(0, min<int64_t>(R, N - row0)));
    const uint32_t ngroups = static_cast<uint32_t>(K / G);
    const uint32_t kh = static_cast<uint32_t>(K) >> 1;
    constexpr uint32_t OOB = 0x80000000u;         // past every resource: reads 0
    const __amdgpu_buffer_rsrc_t crs = buf_rsrc(codes + row0 * kh, rows * kh);
    const __amdgpu_buffer_rsrc_t srs = buf_rsrc(scales + row0 * ngroups, rows * ngroups * 2);
    const __amdgpu_buffer_rsrc_t zrs = buf_rsrc(zeros + row0 * ngroups, rows * ngroups * 2);
    __amdgpu_buffer_rsrc_t xrs[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m)
        xrs[m] = buf_rsrc(x8 + static_cast<int64_t>(m) * K, static_cast<uint32_t>(K));
    constexpr int ONES = 0x01010101;

    float v[R][MR];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) v[r][m] = 0.f;

    for (int seg = sw; seg < nseg; seg += nsb) {
        const uint32_t k0 = static_cast<uint32_t>(seg) * A8R_SEG + 32u * lane;
        const bool ok = k0 < static_cast<uint32_t>(K);
        // x8 first (needed first), then scales / zero-points, then the codes
        u32x4 xv[MR][2];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                xv[m][i] = __builtin_amdgcn_raw_buffer_load_b128(xrs[m], ok ? k0 + 16 * i : OOB, 0, 0);
        // value e = lane + 64 p: row e / GPS, group e % GPS of the segment
        uint32_t sreg[P], zreg[P];
#pragma unroll
        for (int pp = 0; pp < P; ++pp) {
            const uint32_t e = static_cast<uint32_t>(lane) + 64u * pp;
            const uint32_t gs = static_cast<uint32_t>(seg) * GPS + e % GPS;
            const bool live = e / GPS < static_cast<uint32_t>(R) && gs < ngroups;
            const uint32_t so = live ? ((e / GPS) * ngroups + gs) * 2 : OOB;
            sreg[pp] = __builtin_amdgcn_raw_buffer_load_b16(srs, so, 0, 0);
            zreg[pp] = __builtin_amdgcn_raw_buffer_load_b16(zrs, so, 0, 0);
        }
        u32x4 q[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            q[r] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? (k0 >> 1) + r * kh : OOB, 0,
                                                         W4_CPOL_STREAM);
        // x8 split into even-k and odd-k bytes per 8 values (code word j
        // covers x8 values 8 j .. 8 j + 7: dwords 2 j and 2 j + 1 of the lane)
        int xe[MR][4], xo[MR][4], xsum[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const uint32_t d[8] = {xv[m][0].x, xv[m][0].y, xv[m][0].z, xv[m][0].w,
                                   xv[m][1].x, xv[m][1].y, xv[m][1].z, xv[m][1].w};
            xsum[m] = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xe[m][j] = static_cast<int>(__builtin_amdgcn_perm(d[2 * j + 1], d[2 * j], 0x06040200u));
                xo[m][j] = static_cast<int>(__builtin_amdgcn_perm(d[2 * j + 1], d[2 * j], 0x07050301u));
                xsum[m] = __builtin_amdgcn_sdot4(static_cast<int>(d[2 * j]), ONES, xsum[m], false);
                xsum[m] = __builtin_amdgcn_sdot4(static_cast<int>(d[2 * j + 1]), ONES, xsum[m], false);
            }
        }
        const int g = lane / LPG;                 // this lane's group in the segment
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int pr[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) pr[m] = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = q[r][j];
                const int lo = static_cast<int>(w & 0x0F0F0F0Fu);          // q0 q2 q4 q6
                const int hi = static_cast<int>((w >> 4) & 0x0F0F0F0Fu);   // q1 q3 q5 q7
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    pr[m] = __builtin_amdgcn_sdot4(lo, xe[m][j], pr[m], false);
                    pr[m] = __builtin_amdgcn_sdot4(hi, xo[m][j], pr[m], false);
                }
            }
            // row r's values for group g: register (r GPS) / 64 of lane (r GPS) % 64 + g
            const int src = ((r * GPS) % 64 + g) * 4;
            const float s = bf16_to_f32(static_cast<uint16_t>(
                __builtin_amdgcn_ds_bpermute(src, static_cast<int>(sreg[(r * GPS) / 64]))));
            const float z = bf16_to_f32(static_cast<uint16_t>(
                __builtin_amdgcn_ds_bpermute(src, static_cast<int>(zreg[(r * GPS) / 64]))));
#pragma unroll
            for (int m = 0; m < MR; ++m)
                v[r][m] = fmaf(s, static_cast<float>(pr[m]), fmaf(z, static_cast<float>(xsum[m]), v[r][m]));
        }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const float t = sum_rows4(v[0][m], v[1][m], v[2][m], v[3][m]);
        if ((lane & 15) == 0) red[(wave * R + (lane >> 4)) * MR + m] = t;
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < rg * R * MR) {
        const int m = t % MR, rr = t / (R * MR), r = (t / MR) % R;
        const int64_t row = (static_cast<int64_t>(blockIdx.x) * rg + rr) * R + r;
        if (row < N) {
            float sum = 0.f;
            for (int w = 0; w < nsb; ++w) sum += red[((rr * nsb + w) * R + r) * MR + m];
            const float bv = bias ? bf16_to_f32(bias[row]) : 0.0f;
            y[static_cast<int64_t>(m) * N + row] =
                static_cast<uint16_t>(f32_to_bf16_rne(fmaf(sx[m], sum, bv)));
        }
    }
}

template <int MR>
hipError_t launch_rows(const int8_t *x8, const float *sx, const uint8_t *codes,
                       const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                       int N, int K, int G, uint16_t *y, hipStream_t stream) {
    const int nseg = (K + A8R_SEG - 1) / A8R_SEG;
    const int nsb = nseg < A8R_MAX_WAVES ? nseg : A8R_MAX_WAVES;
    const int rg = nsb >= 4 ? 1 : 4 / nsb;          // about four waves per block
    const int64_t rows_per_block = static_cast<int64_t>(rg) * A8R_R;
    const dim3 grid(static_cast<unsigned>((N + rows_per_block - 1) / rows_per_block));
    const dim3 block(static_cast<unsigned>(rg * nsb * 64));
#define W4_A8R_LAUNCH(GG)                                                                      \
    w4a8_gemv_rows_kernel<GG, MR><<<grid, block, 0, stream>>>(x8, sx, codes, scales, zeros, \
                                                               bias, N, K, y, nseg, nsb, rg)
    switch (G) {
    case 32: W4_A8R_LAUNCH(32); break;
    case 64: W4_A8R_LAUNCH(64); break;
    case 128: W4_A8R_LAUNCH(128); break;
    default: return hipErrorInvalidValue;
    }
#undef W4_A8R_LAUNCH
    return hipGetLastError();
}

} // namespace

hipError_t launch_w4a8_rows(const int8_t *x8, const float *sx, int64_t M, const uint8_t *codes,
                            const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                            int64_t N, int64_t K, int G, uint16_t *y, hipStream_t stream) {
    if (M < 1 || M > A8_ROWS_MAX_M || K > A8_ROWS_MAX_K) return hipErrorInvalidValue;
    const int n = static_cast<int>(N), k = static_cast<int>(K);
    switch (M) {
    case 1: return launch_rows<1>(x8, sx, codes, scales, zeros, bias, n, k, G, y, stream);
    case 2: return launch_rows<2>(x8, sx, codes, scales, zeros, bias, n, k, G, y, stream);
    case 3: return launch_rows<3>(x8, sx, codes, scales, zeros, bias, n, k, G, y, stream);
    case 4: return launch_rows<4>(x8, sx, codes, scales, zeros, bias, n, k, G, y, stream);
    case 5: return launch_rows<5>(x8, sx, codes, scales, zeros, bias, n, k, G, y, stream);
    case 6: return launch_rows<6>(x8, sx, codes, scales, zeros, bias, n, k, G, y, stream);
    case 7: return launch_rows<7>(x8, sx, codes, scales, zeros, bias, n, k, G, y, stream);
    default: return launch_rows<8>(x8, sx, codes, scales, zeros, bias, n, k, G, y, stream);
    }
}

} // namespace w4
