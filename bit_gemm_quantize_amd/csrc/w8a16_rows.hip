// Int8 weight-only decode GEMV for one to four activation rows, on the
// vector ALUs (gfx950).
//
// Same result as the other int8 weight-only kernels: per output, in float32,
//   y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] q[n][k]  (+ bias[n])
// with u = q + 128 (0..255, exact in bf16) against x and the group sums of x
// for the offset:  v += s * sum x u - 128 s * sum x.
//
// At M <= 4 a 16-row matrix-core tile carries 12 to 15 padding rows and ties
// each load to 16 rows x 64 bytes. Here a wave takes R = 4 consecutive output
// rows and one 1024-wide K segment; lane l covers k = 1024 s + 16 l .. + 16
// (16 code bytes of each row, one 16-byte load), so every code load of a row
// is 1 KB contiguous and the blocks of a launch sweep the weight in order.
// A lane's 16 codes lie in one group (G >= 32). Each 4 code bytes become two
// bf16 pairs of u through exact float conversions (the upper half of the
// float is the bf16 value) and meet the lane's x pairs of every activation
// row in v_dot2_f32_bf16; x (2 x 16 bytes per lane and activation row,
// natural order) stays in registers for all R rows. (Against the split-K
// matrix-core kernel, per Llama-3-8B decode layer: 15-40 % faster at M = 1
// to 3, equal to 25 % faster at M = 4.) Scales: the segment's R x 1024/G
// values for the R rows come in one or two loads per lane and reach the
// lanes of each group by lane permutes.
// The R partial sums are reduced across the wave with lane swaps and DPP,
// then across the segment waves of a row group in LDS.
#include "w4_device.h"
#include "w4_launch.h"
#include "w4_rows.h"

namespace w4 {

namespace {

constexpr int GV8R_SEG = 1024;             // k per wave segment
// segment waves per block: a row spanning more segments gives each wave
// every 8th (on the 14-segment Llama-3-8B down layer 13 against 15.4 us with
// one wave per segment; caps of 4 and 7 measured the same as 8)
constexpr int GV8R_MAX_WAVES = 8;
constexpr int GV8R_R = 4;                  // output rows per wave

// 4 code bytes -> two bf16 pairs of u = q + 128 (k = 0, 1 and 2, 3)
__device__ __forceinline__ void bytes4_to_bf16(uint32_t d, uint32_t &p01, uint32_t &p23) {
    const uint32_t u = d ^ 0x80808080u;
    const float f0 = static_cast<float>(u & 0xFFu), f1 = static_cast<float>((u >> 8) & 0xFFu);
    const float f2 = static_cast<float>((u >> 16) & 0xFFu), f3 = static_cast<float>(u >> 24);
    p01 = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    p23 = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

// A block holds rg row groups x nsb segment waves; a wave whose row needs
// more than nsb segments takes every nsb-th.
template <int G, int MR>
__global__ __launch_bounds__(GV8R_MAX_WAVES * 64) void w8a16_gemv_rows_kernel(
    const uint16_t *__restrict__ x, const int8_t *__restrict__ q8,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ bias, int N, int K,
    uint16_t *__restrict__ y, int nseg, int nsb, int rg) {
    static_assert(MR >= 1 && MR <= 4, "activation rows");
    constexpr int R = GV8R_R;
    constexpr int GPS = GV8R_SEG / G;              // groups per segment: 32, 16, 8
    constexpr int P = (R * GPS + 63) / 64;         // scale values per lane: 2, 1, 1
    constexpr int LPG = G / 16;                    // lanes per group
    __shared__ float red[GV8R_MAX_WAVES * R * MR];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sw = wave % nsb, rgi = wave / nsb;
    const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * rg + rgi) * R;
    const uint32_t rows = static_cast<uint32_t>(max<int64_t>(0, min<int64_t>(R, N - row0)));
    const uint32_t ngroups = static_cast<uint32_t>(K / G);
    constexpr uint32_t OOB = 0x80000000u;          // past every resource: reads 0
    const __amdgpu_buffer_rsrc_t crs = buf_rsrc(q8 + row0 * K, rows * static_cast<uint32_t>(K));
    const __amdgpu_buffer_rsrc_t srs = buf_rsrc(scales + row0 * ngroups, rows * ngroups * 2);
    __amdgpu_buffer_rsrc_t xrs[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m)
        xrs[m] = buf_rsrc(x + static_cast<int64_t>(m) * K, static_cast<uint32_t>(K) * 2);
    const uint32_t ones = 0x3F803F80u;             // bf16 pair (1, 1)

    float v[R][MR];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) v[r][m] = 0.f;

    for (int seg = sw; seg < nseg; seg += nsb) {
        const uint32_t k0 = static_cast<uint32_t>(seg) * GV8R_SEG + 16u * lane;
        const bool ok = k0 < static_cast<uint32_t>(K);
        // x first (needed first), then the scales, then the codes: loads
        // complete in order, so each row can be finished as soon as its own
        // codes arrive
        u32x4 xv[MR][2];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                xv[m][i] = __builtin_amdgcn_raw_buffer_load_b128(xrs[m], ok ? (k0 + 8 * i) * 2 : OOB, 0, 0);
        // value e = lane + 64 p: row e / GPS, group e % GPS of the segment
        uint32_t sreg[P];
#pragma unroll
        for (int pp = 0; pp < P; ++pp) {
            const uint32_t e = static_cast<uint32_t>(lane) + 64u * pp;
            const uint32_t gs = static_cast<uint32_t>(seg) * GPS + e % GPS;
            const bool live = e / GPS < static_cast<uint32_t>(R) && gs < ngroups;
            sreg[pp] = __builtin_amdgcn_raw_buffer_load_b16(
                srs, live ? ((e / GPS) * ngroups + gs) * 2 : OOB, 0, 0);
        }
        u32x4 q[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            q[r] = __builtin_amdgcn_raw_buffer_load_b128(
                crs, ok ? static_cast<uint32_t>(r) * static_cast<uint32_t>(K) + k0 : OOB, 0,
                W4_CPOL_STREAM);
        float xs[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            xs[m] = 0.f;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                xs[m] = dot2_bf16(xv[m][i].x, ones, xs[m]);
                xs[m] = dot2_bf16(xv[m][i].y, ones, xs[m]);
                xs[m] = dot2_bf16(xv[m][i].z, ones, xs[m]);
                xs[m] = dot2_bf16(xv[m][i].w, ones, xs[m]);
            }
        }
        const int g = lane / LPG;                  // this lane's group in the segment
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float p0[MR], p1[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) p0[m] = p1[m] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {          // code bytes 4 i .. 4 i + 3
                uint32_t a, b;
                bytes4_to_bf16(q[r][i], a, b);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    const u32x4 &xx = xv[m][i >> 1];
                    p0[m] = dot2_bf16((i & 1) ? xx.z : xx.x, a, p0[m]);
                    p1[m] = dot2_bf16((i & 1) ? xx.w : xx.y, b, p1[m]);
                }
            }
            // row r's scale for group g: register (r GPS) / 64 of lane (r GPS) % 64 + g
            const int src = ((r * GPS) % 64 + g) * 4;
            const float s = bf16_to_f32(static_cast<uint16_t>(
                __builtin_amdgcn_ds_bpermute(src, static_cast<int>(sreg[(r * GPS) / 64]))));
            const float so = -128.0f * s;
#pragma unroll
            for (int m = 0; m < MR; ++m) v[r][m] = fmaf(s, p0[m] + p1[m], fmaf(so, xs[m], v[r][m]));
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
            if (bias) sum += bf16_to_f32(bias[row]);
            y[static_cast<int64_t>(m) * N + row] = static_cast<uint16_t>(f32_to_bf16_rne(sum));
        }
    }
}

template <int MR>
hipError_t launch_rows(const uint16_t *x, const int8_t *q8, const uint16_t *scales,
                       const uint16_t *bias, int N, int K, int G, uint16_t *y,
                       hipStream_t stream) {
    const int nseg = (K + GV8R_SEG - 1) / GV8R_SEG;
    const int nsb = nseg < GV8R_MAX_WAVES ? nseg : GV8R_MAX_WAVES;
    const int rg = nsb >= 4 ? 1 : 4 / nsb;          // about four waves per block
    const int64_t rows_per_block = static_cast<int64_t>(rg) * GV8R_R;
    const dim3 grid(static_cast<unsigned>((N + rows_per_block - 1) / rows_per_block));
    const dim3 block(static_cast<unsigned>(rg * nsb * 64));
    switch (G) {
    case 32: w8a16_gemv_rows_kernel<32, MR><<<grid, block, 0, stream>>>(x, q8, scales, bias, N, K, y, nseg, nsb, rg); break;
    case 64: w8a16_gemv_rows_kernel<64, MR><<<grid, block, 0, stream>>>(x, q8, scales, bias, N, K, y, nseg, nsb, rg); break;
    case 128: w8a16_gemv_rows_kernel<128, MR><<<grid, block, 0, stream>>>(x, q8, scales, bias, N, K, y, nseg, nsb, rg); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_w8a16_rows(const uint16_t *x, int64_t M, const int8_t *q8,
                             const uint16_t *scales, const uint16_t *bias, int64_t N, int64_t K,
                             int G, uint16_t *y, hipStream_t stream) {
    if (M < 1 || M > W8_ROWS_MAX_M || K > W8_ROWS_MAX_K) return hipErrorInvalidValue;
    const int n = static_cast<int>(N), k = static_cast<int>(K);
    switch (M) {
    case 1: return launch_rows<1>(x, q8, scales, bias, n, k, G, y, stream);
    case 2: return launch_rows<2>(x, q8, scales, bias, n, k, G, y, stream);
    case 3: return launch_rows<3>(x, q8, scales, bias, n, k, G, y, stream);
    default: return launch_rows<4>(x, q8, scales, bias, n, k, G, y, stream);
    }
}

} // namespace w4
