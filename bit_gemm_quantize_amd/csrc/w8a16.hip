// Int8 weight-only for gfx950: group-wise symmetric int8 weights and the
// bf16-activation linear.
//
// Quantizer (torchao README: an int8 weight-only config with per-group
// granularity 128; "Optimum Quanto", "Design overview / Tensors": int8 takes
// a symmetric projection), per group g of G consecutive k in row n:
//   a = max |v|,  s = bf16_rne(fl32(a / 127)),
//   q = clamp(rne(fl32(v / s)), -127, 127)   (0 when s == 0)
// with IEEE binary32 division by the stored scale and ties to even.
// codes int8 [N, K], scales bf16 [N, K/G].
//
// Linear: y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] q[n][k] (+ bias[n]).
// The bf16 matrix cores take u = q + 128 (0..255, exact in bf16; the code
// byte with its top bit flipped) against x, and an all-ones operand gives
// sum_{k in g} x; per group, in float32:
//   acc += s * acc_g - 128 s * xsum_g
// A byte becomes bf16 through an exact float conversion whose upper half is
// the bf16 value (integers below 256 need at most 8 significant bits).
//
// M > 16: tiles of 128 x 128 as the W4A16 prefill GEMM (four 64 x 64 waves,
// 64-wide K stages in three LDS buffers filled by global -> LDS copies; the
// code tile 64 bytes per row, 16-byte pieces swizzled by (row / 4) % 4).
// M <= 16: blocks of 16 output columns; the 8 waves of a block split K,
// read x and the codes straight from memory (loads for the next four
// 32-wide slices in flight) and reduce their partial sums in LDS.
#include <type_traits>
#include <utility>

#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

// ---------------------------------------------------------------- quantizer
constexpr int Q8_THREADS = 256;

// 16 elements (32 bytes) per lane and step; a group is G / 16 consecutive
// lanes inside one DPP row (chunks never straddle groups: K % G == 0)
template <int G>
__global__ __launch_bounds__(Q8_THREADS) void quantize8_kernel(const uint16_t *__restrict__ W,
                                                              int64_t nchunk,
                                                              int8_t *__restrict__ q8,
                                                              uint16_t *__restrict__ scales) {
    constexpr int LPG = G / 16;
    for (int64_t c = static_cast<int64_t>(blockIdx.x) * Q8_THREADS + threadIdx.x; c < nchunk;
         c += static_cast<int64_t>(gridDim.x) * Q8_THREADS) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(W) + 2 * c;
        const u32x4 v0 = __builtin_nontemporal_load(src);
        const u32x4 v1 = __builtin_nontemporal_load(src + 1);
        float f[16] = {bf16_lo(v0.x), bf16_hi(v0.x), bf16_lo(v0.y), bf16_hi(v0.y),
                       bf16_lo(v0.z), bf16_hi(v0.z), bf16_lo(v0.w), bf16_hi(v0.w),
                       bf16_lo(v1.x), bf16_hi(v1.x), bf16_lo(v1.y), bf16_hi(v1.y),
                       bf16_lo(v1.z), bf16_hi(v1.z), bf16_lo(v1.w), bf16_hi(v1.w)};
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) a = fmaxf(a, fabsf(f[e]));
        a = fmaxf(a, dpp_f32<DPP_QUAD_XOR1>(a));
        if constexpr (LPG >= 4) a = fmaxf(a, dpp_f32<DPP_QUAD_XOR2>(a));
        if constexpr (LPG >= 8) a = fmaxf(a, dpp_f32<DPP_ROW_HALF_MIRROR>(a));
        const uint32_t sb = f32_to_bf16_rne(a / 127.0f);       // correctly rounded divide
        const float s = bf16_to_f32(static_cast<uint16_t>(sb));
        uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float q = 0.0f;
            if (s != 0.0f) q = fminf(fmaxf(__builtin_rintf(f[e] / s), -127.0f), 127.0f);
            o[e >> 2] |= (static_cast<uint32_t>(static_cast<int>(q)) & 0xFFu) << (8 * (e & 3));
        }
        __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]},
                                    reinterpret_cast<u32x4 *>(q8) + c);
        if ((threadIdx.x & (LPG - 1)) == 0) scales[(c * 16) / G] = static_cast<uint16_t>(sb);
    }
}

// 4 code bytes -> two bf16 pairs of u = q + 128 (exact)
__device__ __forceinline__ void bytes_to_bf16(uint32_t d, uint32_t &p01, uint32_t &p23) {
    const uint32_t u = d ^ 0x80808080u;
    // each a single v_cvt_f32_ubyteN
    const float f0 = static_cast<float>(u & 0xFFu), f1 = static_cast<float>((u >> 8) & 0xFFu);
    const float f2 = static_cast<float>((u >> 16) & 0xFFu), f3 = static_cast<float>(u >> 24);
    // upper halves of the floats: (f0, f1) and (f2, f3)
    p01 = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    p23 = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
}

__device__ __forceinline__ bf16x8 bytes8_to_bf16x8(u32x2 w) {
    uint32_t a, b, c, d;
    bytes_to_bf16(w.x, a, b);
    bytes_to_bf16(w.y, c, d);
    return as_bf16x8(a, b, c, d);
}

// ---------------------------------------------------------------- GEMM, M > 16
constexpr int BM = 128, BN = 128, KS = 64;
constexpr int THREADS = 256;
constexpr int NBUF = 3;
constexpr int A_BYTES = BM * KS * 2;             // x tile, bf16, swizzled rows
constexpr int B_BYTES = BN * KS;                 // code tile, int8
constexpr int SZ_BYTES = 2 * BN * 4;             // [group end][row] scales, 4 B each
constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SZ_BYTES;

template <int V>
using IC = std::integral_constant<int, V>;

// f(IC<0>{}), f(IC<1>{}), ...: a loop unrolled with compile-time indices
template <typename F, int... I>
__device__ __forceinline__ void unrolled(std::integer_sequence<int, I...>, F &&f) {
    (f(IC<I>{}), ...);
}

__device__ __forceinline__ void copy16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 : : "v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void copy2(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off"
                 : : "v"(g), "s"(lds) : "memory", "m0");
}

// KSP = 2: two groups of four waves split K in halves inside one block (own
// stage buffers), the second group's sums added through LDS at the end; for
// grids of at most one tile per compute unit, which then still run two waves
// per SIMD.
template <int G, int KSP = 1>
__global__ __launch_bounds__(THREADS * KSP, 2) void w8a16_gemm_kernel(
    const uint16_t *__restrict__ x, int M, const int8_t *__restrict__ q8,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ bias, int N, int K,
    uint16_t *__restrict__ y, int64_t tile0, int64_t ntiles) {
    static_assert(KSP == 1 || KSP == 2, "K groups");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[KSP][NBUF][STAGE_BYTES];
    constexpr int Q = 4 + 2 + 1;                 // copies per wave and stage

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
    // x: copy i of wave w fills rows 8 (4w + i) .. +8; lane l row + l / 8,
    // 16-byte slot l % 8 holding k-piece (l % 8) ^ ((row / 2) % 8)
    uint32_t a_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a_row[i] = static_cast<uint32_t>(min(m0 + (wave * 4 + i) * 8 + (lane >> 3), M - 1));
    // codes: copy i of wave w fills rows 16 (2w + i) .. +16; lane l: row
    // 16 (2w + i) + l / 4, slot l % 4 holding piece (l % 4) ^ ((row / 4) % 4)
    const int8_t *b_src[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 16 * (2 * wave + i) + (lane >> 2);
        const int piece = (lane & 3) ^ ((row >> 2) & 3);
        b_src[i] = q8 + static_cast<int64_t>(min(n0 + row, N - 1)) * K + piece * 16;
    }
    // scale of the group end h of the stage for row r: value v = 64 w + l,
    // row v % 128, end v / 128 (at G >= 64 both ends are the one group end)
    const int sz_row = (64 * wave + lane) & 127, sz_h = (64 * wave + lane) >> 7;
    const uint16_t *s_src = scales + static_cast<int64_t>(min(n0 + sz_row, N - 1)) * ngroups;

    auto issue = [&](int kt, int buf) {
        const uint32_t base = lds0 + static_cast<uint32_t>(buf) * STAGE_BYTES;
        const int k0 = kbase + kt * KS;
        const int kp0 = k0 + ((lane & 7) ^ (lane >> 4)) * 8;
        const int kp1 = k0 + ((lane & 7) ^ (4 | (lane >> 4))) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            copy16(x + (static_cast<uint64_t>(a_row[i]) * static_cast<uint32_t>(K) +
                        static_cast<uint32_t>((i & 1) ? kp1 : kp0)),
                   base + (wave * 4 + i) * 1024);
#pragma unroll
        for (int i = 0; i < 2; ++i) copy16(b_src[i] + k0, base + A_BYTES + (2 * wave + i) * 1024);
        // at G = 128 a group spans two stages and ends in the odd one: only
        // odd stages fetch scales (their slots in even stages are not read)
        if (G != 128 || (kt & 1)) {
            const int k_end = k0 + (G == 32 ? (sz_h + 1) * 32 : KS);
            copy2(s_src + max(0, min(k_end / G - 1, ngroups - 1)), base + A_BYTES + B_BYTES + 256 * wave);
        }
    };

    f32x4 acc[4][4], accg[4][4], xsg[4];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xsg[i] = zero4;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = accg[i][j] = zero4;
    }
    const bf16x8 ones = bf16x8_ones();
    float sv[4] = {0.f, 0.f, 0.f, 0.f}, zz[4] = {0.f, 0.f, 0.f, 0.f};
    auto fold = [&](int mt) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[mt][nt][i] = fmaf(sv[nt], accg[mt][nt][i], fmaf(zz[nt], xsg[mt][i], acc[mt][nt][i]));
    };

    auto slice = [&](int buf, auto par_c, auto sl_c) {
        constexpr int par = decltype(par_c)::value;
        constexpr int sl = decltype(sl_c)::value;
        constexpr bool first = G == 128 ? (par == 0 && sl == 0) : (G == 64 ? sl == 0 : true);
        constexpr bool last = G == 128 ? (par == 1 && sl == 1) : (G == 64 ? sl == 1 : true);
        const uint8_t *sb = &smem[wg][buf][0];
        bf16x8 a[4], b[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int r = wm * 64 + mt * 16 + nl;
            a[mt] = as_bf16x8(*reinterpret_cast<const u32x4 *>(
                sb + r * 128 + (((sl * 4 + kb) ^ ((r >> 1) & 7)) * 16)));
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int r = wn * 64 + nt * 16 + nl;    // (r / 4) % 4 == (nl / 4) % 4
            const int piece = 2 * sl + (kb >> 1);
            const u32x2 w = *reinterpret_cast<const u32x2 *>(
                sb + A_BYTES + r * 64 + ((piece ^ ((nl >> 2) & 3)) * 16) + (kb & 1) * 8);
            b[nt] = bytes8_to_bf16x8(w);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if constexpr (first) {
                fold(mt);
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) asm volatile("" : "+v"(acc[mt][nt]));
                asm volatile("" : "+v"(a[mt]));
            }
            xsg[mt] = mfma16x16x32(a[mt], ones, first ? zero4 : xsg[mt]);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                accg[mt][nt] = mfma16x16x32(a[mt], b[nt], first ? zero4 : accg[mt][nt]);
        }
        if constexpr (last) {
            constexpr int h = (G == 32) ? sl : 0;
            const uint32_t *szp = reinterpret_cast<const uint32_t *>(sb + A_BYTES + B_BYTES);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int c = wn * 64 + nt * 16 + nl;
                sv[nt] = bf16_to_f32(static_cast<uint16_t>(szp[h * 128 + c]));
                zz[nt] = -128.0f * sv[nt];
            }
        }
    };

    issue(0, 0);
    issue(min(1, nstages - 1), 1);
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(Q) : "memory");
    __syncthreads();

    auto stage = [&](auto par_c, int kt) {
        // opaque buffer index: a scalar offset per fragment read instead of a
        // per-lane induction variable
        int buf = kt % NBUF;
        asm volatile("" : "+s"(buf));
        issue(min(kt + 2, nstages - 1), (kt + 2) % NBUF);
        slice(buf, par_c, IC<0>{});
        slice(buf, par_c, IC<1>{});
        // stage kt + 2 (same parity as kt; past the end the repeated last
        // stage is odd and issues at least as many copies) may be in flight
        constexpr int QW = (G == 128 && decltype(par_c)::value == 0) ? Q - 1 : Q;
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"(QW) : "memory");
        __syncthreads();
    };
    if constexpr (G == 128) {
        for (int kt = 0; kt < nstages; kt += 2) {
            stage(IC<0>{}, kt);
            stage(IC<1>{}, kt + 1);
        }
    } else {
        for (int kt = 0; kt < nstages; ++kt) stage(IC<0>{}, kt);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy outlives the block

#pragma unroll
    for (int mt = 0; mt < 4; ++mt) fold(mt);

    if constexpr (KSP == 2) {
        // the second K half's sums through its own (now idle) stage buffers:
        // 4 waves x 16 tiles x 64 lanes x 16 bytes = 64 KB, lanes contiguous
        __syncthreads();                        // every copy of the block has landed
        f32x4 *red = reinterpret_cast<f32x4 *>(&smem[1][0][0]);
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
    for (int nt = 0; nt < 4; ++nt) {
        const int n = n0 + wn * 64 + nt * 16 + nl;
        if (n >= N) continue;
        const float bv = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wm * 64 + mt * 16 + 4 * kb + i;
                if (m < M)
                    y[static_cast<int64_t>(m) * N + n] =
                        static_cast<uint16_t>(f32_to_bf16_rne(acc[mt][nt][i] + bv));
            }
    }
}

// ---------------------------------------------------------------- GEMV, M <= 16
constexpr int GV8_WAVES = 8;
constexpr int GV8_DEPTH = 4;                     // 64-wide slices in flight per wave

// Block: 16 output columns n0 .. n0 + 15; the 8 waves split K in slices of
// 64 k. Lane (nl, kb): A row nl (x row; rows >= M repeat M - 1 and are never
// stored), B column n0 + nl, code bytes 16 kb .. + 16 of the slice: one
// 16-byte load per lane covers 64 contiguous bytes of each of 16 rows. The
// MFMA (16 x 16 x 32) takes 8 k per lane; any assignment of the slice's k to
// lanes works if the x operand follows it and one MFMA never mixes groups:
//   G >= 64: a wave takes whole groups (groups w, w + 8, ...); the slice feeds
//     two MFMAs, on bytes 0..7 and 8..15 of each lane;
//   G = 32: a slice is two groups (kb 0, 1 hold the first, kb 2, 3 the
//     second); swapping the upper 8 bytes of lanes kb 0, 1 with the lower 8
//     of lanes kb 2, 3 (permlane32 swaps) gives every lane 8 bytes of each
//     group: the first MFMA sees k = 16 (kb % 2) + 8 (kb / 2) .. + 8, the
//     second 32 more.
template <int G>
__global__ __launch_bounds__(GV8_WAVES * 64, 2) void w8a16_gemv_kernel(
    const uint16_t *__restrict__ x, int M, const int8_t *__restrict__ q8,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ bias, int N, int K,
    uint16_t *__restrict__ y) {
    constexpr bool PAIR = G == 32;               // two groups per slice
    constexpr int SPG = PAIR ? 1 : G / 64;       // slices per unit (group, or group pair)
    static_assert(GV8_DEPTH % SPG == 0, "slot d holds slices t with t % SPG == d % SPG");
    __shared__ float red[GV8_WAVES][16][17];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nl = lane & 15, kb = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int ncol = min(16, N - n0);
    const int ngroups = K / G;
    const int nunits = PAIR ? ngroups / 2 : ngroups;   // K % 64 == 0
    const int mrow = nl < M ? nl : M - 1;
    // buffer resources: rows past N and slices past K read 0
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x), 0, M * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(q8 + static_cast<int64_t>(n0) * K), 0, ncol * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(scales + static_cast<int64_t>(n0) * ngroups), 0,
        ncol * ngroups * 2, 0x00020000);
    // x pieces of the two MFMAs, byte offsets in the row
    const int xk0 = PAIR ? 16 * (kb & 1) + 8 * (kb >> 1) : 16 * kb;
    const int xk1 = PAIR ? xk0 + 32 : xk0 + 8;
    const int xo = (mrow * K) * 2;
    const int wo = nl * K + 16 * kb;
    const int so = nl * ngroups * 2;
    constexpr int OOB = 0x40000000;

    // a wave's slices, SPG at a time (one unit): j = (wave + 8 i) * SPG ...
    const int nun_w = (nunits - wave + GV8_WAVES - 1) / GV8_WAVES;   // units of this wave
    const bf16x8 ones = bf16x8_ones();
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc = zero4;
    u32x4 xa[GV8_DEPTH][2];
    u32x4 wb[GV8_DEPTH];
    uint32_t sr[GV8_DEPTH] = {};                  // the unit's scale (two at G = 32)
    // slice t of this wave's sequence -> global slice index
    auto gslice = [&](int t) { return ((wave + GV8_WAVES * (t / SPG)) * SPG) + (t % SPG); };
    const int nt_w = nun_w * SPG;
    auto load = [&](int t, int slot) {
        const int j = gslice(t);
        const bool live = t < nt_w;
        const int xs = live ? j * 128 : OOB;
        xa[slot][0] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + 2 * xk0, xs, 0);
        xa[slot][1] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + 2 * xk1, xs, 0);
        wb[slot] = __builtin_amdgcn_raw_buffer_load_b128(wrs, wo, live ? j * 64 : OOB, W4_CPOL_STREAM);
        // the scale rides with the slice that folds its group; the 16 lanes
        // of the first row load it (the fold broadcasts it to the others)
        if constexpr (PAIR) {
            if (kb == 0)
                sr[slot] = __builtin_amdgcn_raw_buffer_load_b32(srs, so, live ? j * 4 : OOB, 0);
        } else if (slot % SPG == SPG - 1) {
            if (kb == 0)
                sr[slot] = __builtin_amdgcn_raw_buffer_load_b16(srs, so, live ? (j / SPG) * 2 : OOB, 0);
        }
    };
    f32x4 accg = zero4, xsg = zero4;
    auto fold = [&](float sc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, accg[i], fmaf(-128.0f * sc, xsg[i], acc[i]));
    };
    // (issued slot by slot, in the order of the refills, so that the wait
    // counts at the loop head are the steady-state ones)
#pragma unroll
    for (int d = 0; d < GV8_DEPTH; ++d) {
        load(d, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    // whole rounds of DEPTH slices; slices past nt_w read nothing (zeros,
    // scale 0) and add 0
    const int nt_pad = (nt_w + GV8_DEPTH - 1) / GV8_DEPTH * GV8_DEPTH;
    for (int t0 = 0; t0 < nt_pad; t0 += GV8_DEPTH) {
        unrolled(std::make_integer_sequence<int, GV8_DEPTH>{}, [&](auto d_c) {
            constexpr int d = decltype(d_c)::value;
            const int t = t0 + d;
            const u32x4 a0 = xa[d][0], a1 = xa[d][1], w = wb[d];
            // the scales leave sr[d] before its refill, so that the ring keeps
            // its registers (a copy on the loop edge would wait for every load)
            constexpr bool folds = PAIR || d % SPG == SPG - 1;
            float s_lo = 0.0f, s_hi = 0.0f;
            if constexpr (folds) {
                // row 0 -> rows 0, 0, 2, 2 -> all four rows
                const auto r1 = __builtin_amdgcn_permlane16_swap(sr[d], sr[d], false, false);
                const auto r2 = __builtin_amdgcn_permlane32_swap(r1[0], r1[0], false, false);
                const uint32_t sv = r2[0];
                s_lo = bf16_to_f32(static_cast<uint16_t>(sv & 0xFFFFu));
                s_hi = bf16_to_f32(static_cast<uint16_t>(sv >> 16));
                if constexpr (PAIR) asm volatile("" : "+v"(s_lo), "+v"(s_hi));
                else asm volatile("" : "+v"(s_lo));
            }
            if constexpr (PAIR) {
                const auto p0 = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
                const auto p1 = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
                xsg = mfma16x16x32(as_bf16x8(a0), ones, zero4);
                accg = mfma16x16x32(as_bf16x8(a0), bytes8_to_bf16x8(u32x2{p0[0], p1[0]}), zero4);
                fold(s_lo);
                xsg = mfma16x16x32(as_bf16x8(a1), ones, zero4);
                accg = mfma16x16x32(as_bf16x8(a1), bytes8_to_bf16x8(u32x2{p0[1], p1[1]}), zero4);
                fold(s_hi);
                load(t + GV8_DEPTH, d);           // refills slot d (after its last read)
            } else {
                constexpr bool first = d % SPG == 0;     // t % SPG (t0 % DEPTH == 0)
                xsg = mfma16x16x32(as_bf16x8(a0), ones, first ? zero4 : xsg);
                accg = mfma16x16x32(as_bf16x8(a0), bytes8_to_bf16x8(u32x2{w.x, w.y}),
                                    first ? zero4 : accg);
                xsg = mfma16x16x32(as_bf16x8(a1), ones, xsg);
                accg = mfma16x16x32(as_bf16x8(a1), bytes8_to_bf16x8(u32x2{w.z, w.w}), accg);
                load(t + GV8_DEPTH, d);
                if constexpr (folds) fold(s_lo);
            }
            // keep the software pipeline as written: the compiler would
            // otherwise gather the round's loads at its end and wait for all
            __builtin_amdgcn_sched_barrier(0);
        });
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * kb + i][nl] = acc[i];
    __syncthreads();
    for (int e = threadIdx.x; e < M * 16; e += GV8_WAVES * 64) {
        const int m = e >> 4, nn = e & 15;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < GV8_WAVES; ++w) sum += red[w][m][nn];
        const int col = n0 + nn;
        if (col < N) {
            if (bias) sum += bf16_to_f32(bias[col]);
            y[static_cast<int64_t>(m) * N + col] = static_cast<uint16_t>(f32_to_bf16_rne(sum));
        }
    }
}

} // namespace

hipError_t launch_quantize8(const uint16_t *W, int64_t N, int64_t K, int G, int8_t *q8,
                            uint16_t *scales, hipStream_t stream) {
    const int64_t nchunk = N * K / 16;
    const int64_t want = (nchunk + Q8_THREADS - 1) / Q8_THREADS;
    const int64_t cap = static_cast<int64_t>(compute_units()) * 24;   // as the int4 quantizer
    const dim3 grid(static_cast<unsigned>(want < cap ? want : cap));
    switch (G) {
    case 32: quantize8_kernel<32><<<grid, dim3(Q8_THREADS), 0, stream>>>(W, nchunk, q8, scales); break;
    case 64: quantize8_kernel<64><<<grid, dim3(Q8_THREADS), 0, stream>>>(W, nchunk, q8, scales); break;
    case 128: quantize8_kernel<128><<<grid, dim3(Q8_THREADS), 0, stream>>>(W, nchunk, q8, scales); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_w8a16(const uint16_t *x, int64_t M, const int8_t *q8, const uint16_t *scales,
                        const uint16_t *bias, int64_t N, int64_t K, int G, uint16_t *y,
                        hipStream_t stream) {
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    // the split-K kernel's 32-bit buffer offsets need 32 K * 2 bytes < 2^30
    if (M <= 16 && K <= (int64_t(1) << 24)) {
        const dim3 grid(static_cast<unsigned>((N + 15) / 16));
        const dim3 block(GV8_WAVES * 64);
        switch (G) {
        case 32: w8a16_gemv_kernel<32><<<grid, block, 0, stream>>>(x, m, q8, scales, bias, n, k, y); break;
        case 64: w8a16_gemv_kernel<64><<<grid, block, 0, stream>>>(x, m, q8, scales, bias, n, k, y); break;
        case 128: w8a16_gemv_kernel<128><<<grid, block, 0, stream>>>(x, m, q8, scales, bias, n, k, y); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
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
            case 32: w8a16_gemm_kernel<32, 2><<<grid, block, 0, stream>>>(x, m, q8, scales, bias, n, k, y, t0, nt); break;
            case 64: w8a16_gemm_kernel<64, 2><<<grid, block, 0, stream>>>(x, m, q8, scales, bias, n, k, y, t0, nt); break;
            case 128: w8a16_gemm_kernel<128, 2><<<grid, block, 0, stream>>>(x, m, q8, scales, bias, n, k, y, t0, nt); break;
            default: return hipErrorInvalidValue;
            }
        } else {
            switch (G) {
            case 32: w8a16_gemm_kernel<32><<<grid, block, 0, stream>>>(x, m, q8, scales, bias, n, k, y, t0, nt); break;
            case 64: w8a16_gemm_kernel<64><<<grid, block, 0, stream>>>(x, m, q8, scales, bias, n, k, y, t0, nt); break;
            case 128: w8a16_gemm_kernel<128><<<grid, block, 0, stream>>>(x, m, q8, scales, bias, n, k, y, t0, nt); break;
            default: return hipErrorInvalidValue;
            }
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

} // namespace w4
