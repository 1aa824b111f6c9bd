// W4A8 for gfx950: per-token int8 activations and the int4-weight linear on
// the int8 matrix cores.
//
// Activations ("Optimum Quanto", "Design overview / Tensors": int8 takes a
// symmetric projection per tensor or per channel; torchao README: int8
// dynamic activations with group-wise int4 weights), per row m of x:
//   a = max_k |x[m][k]|,  sx[m] = fl32(a / 127),
//   x8[m][k] = clamp(rne(fl32(x[m][k] / sx[m])), -127, 127)   (0 when a == 0)
// with IEEE binary32 division and ties to even, like the weight quantizer.
//
// Linear, with the weights' q, s, z of quantize_int4_grouped:
//   y[m][n] = sx[m] * sum_g ( s[n][g] * P_g + z[n][g] * X_g ) (+ bias[n])
//   P_g = sum_{k in g} x8[m][k] q[n][k],  X_g = sum_{k in g} x8[m][k]
// P_g and X_g are exact int32 sums from the int8 matrix cores (X_g against
// an all-ones operand); the group fold, the scale by sx and the bias are
// float32, y is rounded to bf16.
//
// GEMM structure as the W4A16 prefill GEMM: block tile 128 (m) x 128 (n),
// four waves of 64 x 64, K stages of 64 through three LDS buffers filled by
// global -> LDS copies (x8 tile 64 bytes per row, 16-byte pieces swizzled by
// (row / 4) % 4; code tile 32 bytes per row, halves swizzled by (row / 8) % 2;
// scales / zero-points of the group ends). G = 64 / 128: one
// 16x16x64 int8 MFMA per fragment pair and stage; G = 32: two 16x16x32 int8
// MFMAs (one per group). A code word (8 nibbles) becomes 8 bytes q in
// natural k order with one and, one shift-and and two byte permutes.
#include <type_traits>

#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- activations
constexpr int AQ_THREADS = 256;

// one block per row: absmax, then the codes; a row is read twice (the second
// time from L2)
__global__ __launch_bounds__(AQ_THREADS) void act_quant_kernel(const uint16_t *__restrict__ x,
                                                                int K, int8_t *__restrict__ x8,
                                                                float *__restrict__ sx) {
    __shared__ float wmax[AQ_THREADS / 64];
    const int64_t row = blockIdx.x;
    const uint16_t *xr = x + row * K;
    int8_t *qr = x8 + row * K;
    const int tid = threadIdx.x;
    const int n8 = K >> 3;                       // 16-byte pieces (K % 32 == 0)
    float a = 0.0f;
    for (int p = tid; p < n8; p += AQ_THREADS) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(xr + p * 8);
        a = fmaxf(a, fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))),
                           fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y)))));
        a = fmaxf(a, fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))),
                           fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w)))));
    }
    // maximum over each 16-lane row with DPP moves, then over the four rows
    // (lanes 0, 16, 32, 48), then across the waves through LDS
    a = fmaxf(a, dpp_f32<DPP_QUAD_XOR1>(a));
    a = fmaxf(a, dpp_f32<DPP_QUAD_XOR2>(a));
    a = fmaxf(a, dpp_f32<DPP_ROW_HALF_MIRROR>(a));
    a = fmaxf(a, dpp_f32<DPP_ROW_MIRROR>(a));
    a = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 0)),
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 16))),
              fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 32)),
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 48))));
    if ((tid & 63) == 0) wmax[tid >> 6] = a;
    __syncthreads();
    float amax = wmax[0];
#pragma unroll
    for (int w = 1; w < AQ_THREADS / 64; ++w) amax = fmaxf(amax, wmax[w]);
    const float s = amax / 127.0f;               // correctly rounded (build flag)
    if (tid == 0) sx[row] = s;
    for (int p = tid; p < n8; p += AQ_THREADS) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(xr + p * 8);
        const float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                            bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float q = 0.0f;
            if (s != 0.0f) q = fminf(fmaxf(__builtin_rintf(f[e] / s), -127.0f), 127.0f);
            o[e >> 2] |= (static_cast<uint32_t>(static_cast<int>(q)) & 0xFFu) << (8 * (e & 3));
        }
        *reinterpret_cast<u32x2 *>(qr + p * 8) = u32x2{o[0], o[1]};
    }
}

// Rows of up to 256 PPT 16-byte pieces (K <= 2048 PPT): each thread keeps
// its pieces in registers between the max pass and the codes (one read of
// the row), and divides by a reciprocal multiply checked against the exact
// quotient's rounding. With s in [2^-100, 2^100] the hardware reciprocal is
// within 1 ulp, so t = x * rcp(s) is within |t| 1.5 2^-23 <= 2^-15 of x / s,
// and the binary32 quotient within half an ulp of it (< 2^-17 at |t| <=
// 127); when every t of a piece is farther than 2^-14 from a half-integer,
// rint(t) equals rint of the binary32 quotient, otherwise (or for extreme
// scales) the piece is redone with the true divide.
template <int PPT>
__global__ __launch_bounds__(AQ_THREADS) void act_quant_reg_kernel(const uint16_t *__restrict__ x,
                                                                    int K, int8_t *__restrict__ x8,
                                                                    float *__restrict__ sx) {
    __shared__ float wmax[AQ_THREADS / 64];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int n8 = K >> 3;                       // 16-byte pieces (K % 32 == 0)
    const __amdgpu_buffer_rsrc_t xr = buf_rsrc(x + row * K, static_cast<uint32_t>(K) * 2);
    const __amdgpu_buffer_rsrc_t qr = buf_rsrc(x8 + row * K, static_cast<uint32_t>(K));
    u32x4 v[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i)                // pieces past the row read 0
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, (tid + AQ_THREADS * i) * 16, 0,
                                                     W4_CPOL_STREAM);
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        a = fmaxf(a, fmaxf(fmaxf(fabsf(bf16_lo(v[i].x)), fabsf(bf16_hi(v[i].x))),
                           fmaxf(fabsf(bf16_lo(v[i].y)), fabsf(bf16_hi(v[i].y)))));
        a = fmaxf(a, fmaxf(fmaxf(fabsf(bf16_lo(v[i].z)), fabsf(bf16_hi(v[i].z))),
                           fmaxf(fabsf(bf16_lo(v[i].w)), fabsf(bf16_hi(v[i].w)))));
    }
    a = fmaxf(a, dpp_f32<DPP_QUAD_XOR1>(a));
    a = fmaxf(a, dpp_f32<DPP_QUAD_XOR2>(a));
    a = fmaxf(a, dpp_f32<DPP_ROW_HALF_MIRROR>(a));
    a = fmaxf(a, dpp_f32<DPP_ROW_MIRROR>(a));
    a = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 0)),
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 16))),
              fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 32)),
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(a), 48))));
    if ((tid & 63) == 0) wmax[tid >> 6] = a;
    __syncthreads();
    float amax = wmax[0];
#pragma unroll
    for (int w = 1; w < AQ_THREADS / 64; ++w) amax = fmaxf(amax, wmax[w]);
    const float s = amax / 127.0f;               // correctly rounded (build flag)
    if (tid == 0) sx[row] = s;
    const bool fast = s >= 0x1p-100f && s <= 0x1p100f;
    const float r = __builtin_amdgcn_rcpf(s);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int p = tid + AQ_THREADS * i;
        if (p >= n8) break;                      // only the last piece can lie past the row
        const float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                            bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
        float q[8];
        float dmax = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float t = f[e] * r;
            q[e] = __builtin_rintf(t);
            dmax = fmaxf(dmax, fabsf(t - q[e]));
        }
        if (s == 0.0f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = 0.0f;
        } else if (!fast || !(dmax < 0.5f - 0x1p-14f)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = __builtin_rintf(f[e] / s);
        }
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float c = fminf(fmaxf(q[e], -127.0f), 127.0f);
            o[e >> 2] |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xFFu) << (8 * (e & 3));
        }
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{o[0], o[1]}, qr, p * 8, 0, W4_CPOL_STREAM);
    }
}

// ---------------------------------------------------------------- GEMM
constexpr int BM = 128, BN = 128, KS = 64;
constexpr int THREADS = 256;
constexpr int NBUF = 3;
constexpr int A_BYTES = BM * KS;                 // x8 tile
constexpr int B_BYTES = BN * KS / 2;             // code tile
constexpr int SZ_BYTES = 2 * 2 * BN * 4;         // [group end][s | z][row], 4 B each
constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SZ_BYTES;

template <int V>
using IC = std::integral_constant<int, V>;

__device__ __forceinline__ void copy16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 : : "v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void copy2(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off"
                 : : "v"(g), "s"(lds) : "memory", "m0");
}

// 8 codes (one word, natural layout) -> 8 bytes q in natural k order
__device__ __forceinline__ u32x2 codes_to_bytes(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu;         // q0, q2, q4, q6
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // q1, q3, q5, q7
    // perm(a, b, sel): byte i of the result = byte sel_i of (a:b), b = bytes 0-3
    return u32x2{__builtin_amdgcn_perm(hi, lo, 0x05010400u),    // q0 q1 q2 q3
                 __builtin_amdgcn_perm(hi, lo, 0x07030602u)};   // q4 q5 q6 q7
}

// KSP = 2: two groups of four waves split K in halves inside one block (own
// stage buffers), the second group's sums added through LDS at the end; for
// grids of at most one tile per compute unit, which then still run two waves
// per SIMD.
template <int G, int KSP = 1>
__global__ __launch_bounds__(THREADS * KSP, 2) void w4a8_gemm_kernel(
    const int8_t *__restrict__ x8, const float *__restrict__ sx, int M,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ zeros, const uint16_t *__restrict__ bias, int N, int K,
    uint16_t *__restrict__ y, int64_t tile0, int64_t ntiles) {
    static_assert(KSP == 1 || KSP == 2, "K groups");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[KSP][NBUF][STAGE_BYTES];
    constexpr int NSZ = G == 32 ? 2 : 1;         // 2-byte copies per wave and stage
    constexpr int Q = 2 + 1 + NSZ;               // copies per wave and stage

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave: index inside its K group wg, which covers [kbase, kbase + K / KSP)
    const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
    const int wg = KSP == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 8);
    const int wm = wave >> 1, wn = wave & 1;
    const int nl = lane & 15, kb = lane >> 4;
    const int ngroups = K / G;
    const int Kg = K / KSP;
    const int kbase = wg * Kg;
    const int nstages = Kg / KS;                 // K % (64 KSP) == 0 (checked by the host)

    int m0, n0;
    {
        const int64_t T = ntiles, b = blockIdx.x;
        const int64_t xcd = b & 7, j = b >> 3;
        const int64_t t = tile0 + xcd * (T >> 3) + min(xcd, T & 7) + j;
        const int64_t mtiles = (M + BM - 1) / BM, ntl = (N + BN - 1) / BN;
        const int64_t gm = min<int64_t>(4, mtiles);
        const int64_t grp = t / (gm * ntl), r = t - grp * gm * ntl;
        const int64_t gsz = min(gm, mtiles - grp * gm);
        m0 = static_cast<int>((grp * gm + r % gsz) * BM);
        n0 = static_cast<int>((r / gsz) * BN);
    }

    const uint32_t lds0 = lds_address(&smem[wg][0][0]);
    // x8: copy i of wave w fills rows 16 (2w + i) .. +16; lane l: row
    // 16 (2w + i) + l / 4, slot l % 4 holding piece (l % 4) ^ ((row / 4) % 4)
    const int8_t *a_src[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 16 * (2 * wave + i) + (lane >> 2);
        const int piece = (lane & 3) ^ ((row >> 2) & 3);
        a_src[i] = x8 + static_cast<int64_t>(min(m0 + row, M - 1)) * K + piece * 16;
    }
    // codes: lane l of wave w fills row 32 w + l / 2, 16-byte half l % 2,
    // holding k-half (l % 2) ^ ((row / 8) % 2)
    const int b_r = wave * 32 + (lane >> 1);
    const int b_half = (lane & 1) ^ ((b_r >> 3) & 1);
    const uint8_t *b_src = codes + static_cast<int64_t>(min(n0 + b_r, N - 1)) * (K >> 1) + b_half * 16;

    auto issue = [&](int kt, int buf) {
        const uint32_t base = lds0 + static_cast<uint32_t>(buf) * STAGE_BYTES;
        const int k0 = kbase + kt * KS;
#pragma unroll
        for (int i = 0; i < 2; ++i) copy16(a_src[i] + k0, base + (2 * wave + i) * 1024);
        copy16(b_src + k0 / 2, base + A_BYTES + wave * 1024);
        // scales / zero-points of the group ends in this stage: value
        // v = 64 (NSZ w + d) + lane -> row v % 128, s|z (v / 128) % 2, end v / 256;
        // at G = 128 a group ends in the odd stage of each pair, the only one
        // whose scale slots are read
        if (G == 128 && !(kt & 1)) return;
#pragma unroll
        for (int d = 0; d < NSZ; ++d) {
            const int v = 64 * (NSZ * wave + d) + lane;
            const int row = v & 127, isz = (v >> 7) & 1, h = v >> 8;
            const int k_end = k0 + (G == 32 ? (h + 1) * 32 : KS);
            const int g = max(0, min(k_end / G - 1, ngroups - 1));
            const uint16_t *src = (isz ? zeros : scales) +
                                  static_cast<int64_t>(min(n0 + row, N - 1)) * ngroups + g;
            copy2(src, base + A_BYTES + B_BYTES + 64 * 4 * (NSZ * wave + d));
        }
    };

    f32x4 acc[4][4];
    i32x4 accg[4][4], xsg[4];
    const i32x4 zi4 = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xsg[i] = zi4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            accg[i][j] = zi4;
        }
    }
    float sv[4] = {0.f, 0.f, 0.f, 0.f}, zv[4] = {0.f, 0.f, 0.f, 0.f};
    // acc += s * P_g + z * X_g for the group that just ended (row block mt)
    auto fold = [&](int mt) {
        float xf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xf[i] = static_cast<float>(xsg[mt][i]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[mt][nt][i] = fmaf(sv[nt], static_cast<float>(accg[mt][nt][i]),
                                      fmaf(zv[nt], xf[i], acc[mt][nt][i]));
    };
    auto load_sz = [&](const uint8_t *sb, int h) {
        const uint32_t *szp = reinterpret_cast<const uint32_t *>(sb + A_BYTES + B_BYTES);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int c = wn * 64 + nt * 16 + nl;
            sv[nt] = bf16_to_f32(static_cast<uint16_t>(szp[h * 256 + c]));
            zv[nt] = bf16_to_f32(static_cast<uint16_t>(szp[h * 256 + 128 + c]));
        }
    };

    // G = 64 / 128: one 64-wide slice per stage (par: stage parity for G = 128)
    auto stage64 = [&](int buf, auto par_c) {
        constexpr int par = decltype(par_c)::value;
        constexpr bool first = G == 128 ? par == 0 : true;
        constexpr bool last = G == 128 ? par == 1 : true;
        const uint8_t *sb = &smem[wg][buf][0];
        i32x4 a[4], b[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int r = wm * 64 + mt * 16 + nl;        // (r / 4) % 4 == (nl / 4) % 4
            a[mt] = __builtin_bit_cast(i32x4, *reinterpret_cast<const u32x4 *>(
                                                  sb + r * 64 + ((kb ^ ((nl >> 2) & 3)) * 16)));
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int r = wn * 64 + nt * 16 + nl;        // (r / 8) % 2 == (nl / 8) % 2
            const u32x2 w = *reinterpret_cast<const u32x2 *>(
                sb + A_BYTES + r * 32 + (((kb >> 1) ^ ((nl >> 3) & 1)) * 16) + (kb & 1) * 8);
            const u32x2 q0 = codes_to_bytes(w.x), q1 = codes_to_bytes(w.y);
            b[nt] = i32x4{static_cast<int>(q0.x), static_cast<int>(q0.y),
                          static_cast<int>(q1.x), static_cast<int>(q1.y)};
        }
        const i32x4 ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if constexpr (first) {
                fold(mt);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) asm volatile("" : "+v"(acc[mt][nt]));
                asm volatile("" : "+v"(a[mt]));
            }
            xsg[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt], ones, first ? zi4 : xsg[mt], 0, 0, 0);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                accg[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt], b[nt],
                                                                     first ? zi4 : accg[mt][nt], 0, 0, 0);
        }
        if constexpr (last) load_sz(sb, 0);
    };

    // G = 32: two 32-wide slices per stage, one group each
    auto stage32 = [&](int buf) {
        const uint8_t *sb = &smem[wg][buf][0];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            long a[4], b[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int r = wm * 64 + mt * 16 + nl;
                const int piece = 2 * sl + (kb >> 1);
                a[mt] = __builtin_bit_cast(long, *reinterpret_cast<const u32x2 *>(
                                                     sb + r * 64 + ((piece ^ ((nl >> 2) & 3)) * 16) +
                                                     (kb & 1) * 8));
            }
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int r = wn * 64 + nt * 16 + nl;
                const uint32_t w = *reinterpret_cast<const uint32_t *>(
                    sb + A_BYTES + r * 32 + ((sl ^ ((nl >> 3) & 1)) * 16) + kb * 4);
                b[nt] = __builtin_bit_cast(long, codes_to_bytes(w));
            }
            const long ones = 0x0101010101010101L;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                fold(mt);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) asm volatile("" : "+v"(acc[mt][nt]));
                asm volatile("" : "+v"(a[mt]));
                xsg[mt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[mt], ones, zi4, 0, 0, 0);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt)
                    accg[mt][nt] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[mt], b[nt], zi4, 0, 0, 0);
            }
            load_sz(sb, sl);
        }
    };

    // prologue: stages 0 and 1 in flight, wait for stage 0
    issue(0, 0);
    issue(min(1, nstages - 1), 1);
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(Q) : "memory");
    __syncthreads();

    auto step = [&](auto par_c, int kt) {
        // opaque buffer index: a scalar offset per fragment read instead of a
        // per-lane induction variable
        int buf = kt % NBUF;
        asm volatile("" : "+s"(buf));
        // stage kt + 2 goes into the buffer read in stage kt - 1; past the
        // end it repeats the last stage into a buffer that is not read again
        issue(min(kt + 2, nstages - 1), (kt + 2) % NBUF);
        if constexpr (G == 32)
            stage32(buf);
        else
            stage64(buf, par_c);
        // stage kt + 2 (same parity as kt; past the end the repeated last
        // stage is odd and issues at least as many copies) may be in flight
        constexpr int QW = (G == 128 && decltype(par_c)::value == 0) ? Q - NSZ : Q;
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"(QW) : "memory");
        __syncthreads();
    };
    if constexpr (G == 128) {
        for (int kt = 0; kt < nstages; kt += 2) {
            step(IC<0>{}, kt);
            step(IC<1>{}, kt + 1);
        }
    } else {
        for (int kt = 0; kt < nstages; ++kt) step(IC<0>{}, kt);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy outlives the block

#pragma unroll
    for (int mt = 0; mt < 4; ++mt) fold(mt);

    if constexpr (KSP == 2) {
        // the second K half's sums through the (now idle) stage buffers:
        // 4 waves x 16 tiles x 64 lanes x 16 bytes = 64 KB, lanes contiguous
        static_assert(KSP * NBUF * STAGE_BYTES >= 64 * 1024, "reduction space");
        __syncthreads();                        // every copy of the block has landed
        f32x4 *red = reinterpret_cast<f32x4 *>(&smem[0][0][0]);
        if (wg == 1) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) red[((wave * 4 + mt) * 4 + nt) * 64 + lane] = acc[mt][nt];
        }
        __syncthreads();
        if (wg == 1) return;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[mt][nt] += red[((wave * 4 + mt) * 4 + nt) * 64 + lane];
    }

#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + wm * 64 + mt * 16 + 4 * kb + i;
            if (m >= M) continue;
            const float sm = sx[m];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int n = n0 + wn * 64 + nt * 16 + nl;
                if (n >= N) continue;
                const float bv = bias ? bf16_to_f32(bias[n]) : 0.0f;
                y[static_cast<int64_t>(m) * N + n] =
                    static_cast<uint16_t>(f32_to_bf16_rne(fmaf(sm, acc[mt][nt][i], bv)));
            }
        }
}

} // namespace

hipError_t launch_act_quant(const uint16_t *x, int64_t M, int64_t K, int8_t *x8, float *sx,
                            hipStream_t stream) {
    constexpr int64_t kMaxRows = int64_t(1) << 30;
    // pieces of 8 per thread when the row fits in registers (K <= 16384)
    const int64_t ppt = (K / 8 + AQ_THREADS - 1) / AQ_THREADS;
    for (int64_t r0 = 0; r0 < M; r0 += kMaxRows) {
        const int64_t rows = M - r0 < kMaxRows ? M - r0 : kMaxRows;
        const dim3 grid(static_cast<unsigned>(rows)), block(AQ_THREADS);
        const int k = static_cast<int>(K);
        switch (ppt) {
        case 1: act_quant_reg_kernel<1><<<grid, block, 0, stream>>>(x + r0 * K, k, x8 + r0 * K, sx + r0); break;
        case 2: act_quant_reg_kernel<2><<<grid, block, 0, stream>>>(x + r0 * K, k, x8 + r0 * K, sx + r0); break;
        case 3: act_quant_reg_kernel<3><<<grid, block, 0, stream>>>(x + r0 * K, k, x8 + r0 * K, sx + r0); break;
        case 4: act_quant_reg_kernel<4><<<grid, block, 0, stream>>>(x + r0 * K, k, x8 + r0 * K, sx + r0); break;
        case 5: case 6:
            act_quant_reg_kernel<6><<<grid, block, 0, stream>>>(x + r0 * K, k, x8 + r0 * K, sx + r0); break;
        case 7: case 8:
            act_quant_reg_kernel<8><<<grid, block, 0, stream>>>(x + r0 * K, k, x8 + r0 * K, sx + r0); break;
        default:
            act_quant_kernel<<<grid, block, 0, stream>>>(x + r0 * K, k, x8 + r0 * K, sx + r0);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_w4a8_gemm(const int8_t *x8, const float *sx, int64_t M, const uint8_t *codes,
                            const uint16_t *scales, const uint16_t *zeros,
                            const uint16_t *bias, int64_t N, int64_t K, int G, uint16_t *y,
                            hipStream_t stream) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    // at most one tile per compute unit: split K inside eight-wave blocks
    // (each half a multiple of the stage pair and the group)
    const bool ksplit = tiles <= compute_units() && K % (2 * (G > KS ? G : KS)) == 0;
    constexpr int64_t kMaxTiles = int64_t(1) << 22;
    for (int64_t t0 = 0; t0 < tiles; t0 += kMaxTiles) {
        const int64_t nt = tiles - t0 < kMaxTiles ? tiles - t0 : kMaxTiles;
        const dim3 grid(static_cast<unsigned>(nt));
        const dim3 block(THREADS * (ksplit ? 2 : 1));
        if (ksplit) {
            switch (G) {
            case 32: w4a8_gemm_kernel<32, 2><<<grid, block, 0, stream>>>(x8, sx, m, codes, scales, zeros, bias, n, k, y, t0, nt); break;
            case 64: w4a8_gemm_kernel<64, 2><<<grid, block, 0, stream>>>(x8, sx, m, codes, scales, zeros, bias, n, k, y, t0, nt); break;
            case 128: w4a8_gemm_kernel<128, 2><<<grid, block, 0, stream>>>(x8, sx, m, codes, scales, zeros, bias, n, k, y, t0, nt); break;
            default: return hipErrorInvalidValue;
            }
        } else {
            switch (G) {
            case 32: w4a8_gemm_kernel<32><<<grid, block, 0, stream>>>(x8, sx, m, codes, scales, zeros, bias, n, k, y, t0, nt); break;
            case 64: w4a8_gemm_kernel<64><<<grid, block, 0, stream>>>(x8, sx, m, codes, scales, zeros, bias, n, k, y, t0, nt); break;
            case 128: w4a8_gemm_kernel<128><<<grid, block, 0, stream>>>(x8, sx, m, codes, scales, zeros, bias, n, k, y, t0, nt); break;
            default: return hipErrorInvalidValue;
            }
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

} // namespace w4
