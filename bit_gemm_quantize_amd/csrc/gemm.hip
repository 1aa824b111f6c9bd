// Prefill-path W4A16 GEMM (any M, meant for M > 16) for gfx950.
//
// Same result as the GEMV: per output, in float32,
//   sum_g ( s[n][g] * sum_{k in g} x[m][k] q[n][k] + z[n][g] * sum_{k in g} x[m][k] )
// ("Optimum Quanto": wide accumulation, then dequantization; bias in float).
//
// Block tile 128 (m) x 128 (n), four waves in a 2 x 2 grid, 64 x 64 each.
// K advances in stages of 64 (two 32-wide slices) through three LDS buffers,
// two stages in flight while one is computed. Every operand reaches LDS by a
// direct global -> LDS copy issued from asm (16 bytes per lane; scales and
// zero-points 2 bytes per lane), with explicit s_waitcnt before each stage
// barrier, so the compiler sees no memory loads in the loop: the x tile as
// bf16 rows (XOR swizzled), the code tile as packed nibbles (16-byte halves
// swizzled), and the scales / zero-points of the groups that end in the
// stage. Each slice expands the wave's code fragments to the exact bf16
// integers 128 + q, runs 16x16x32 bf16 MFMAs into a per-group accumulator,
// and one MFMA against an all-ones B gives the group sums of x in the same
// layout. After a group, in float32:
//   acc += s * acc_g + (z - 128 s) * xsum_g
// (128 + q is exact in bf16 and the MFMA accumulates exactly-representable
// products in float32, so the only rounding is the float32 accumulation.)
//
// The pre-shuffled variant (PK) reads codes whose 4-byte words hold the
// even-k nibbles in the low half and the odd-k nibbles in the high half,
// so the expansion is a shift and one and-or per bf16 pair, and scale /
// zero-point pairs packed in one word (one 4-byte copy per row and group).
#include <type_traits>

#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

constexpr int BM = 128, BN = 128, KS = 64;
constexpr int THREADS = 256;
constexpr int NBUF = 3;                          // stages in LDS (two in flight)
constexpr int A_BYTES = BM * KS * 2;             // x tile, bf16, swizzled rows
constexpr int B_BYTES = BN * KS / 2;             // code tile, packed nibbles
constexpr int SZ_BYTES = 2 * 2 * BN * 4;         // [group end][s | z][row], 4 B each
constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SZ_BYTES;

template <int V>
using IC = std::integral_constant<int, V>;

// 16 / 2 bytes per lane, global -> LDS at lds (wave-uniform) + 16 * lane
// (2-byte copies: + 4 * lane, zero-extended). No output registers; waits are
// explicit s_waitcnt vmcnt.
__device__ __forceinline__ void copy16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 : : "v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void copy2(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off"
                 : : "v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void copy4(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 : : "v"(g), "s"(lds) : "memory", "m0");
}

template <int G, bool PK>
__global__ __launch_bounds__(THREADS, 2) void gemm_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint32_t *__restrict__ sz, const uint16_t *__restrict__ bias, int N, int K,
    uint16_t *__restrict__ y, int64_t tile0, int64_t ntiles) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF][STAGE_BYTES];
    // scale / zero-point copies per wave and stage (2 bytes each, or one
    // 4-byte pair each in the pre-shuffled layout)
    constexpr int NSZ = (G == 32 && !PK) ? 2 : 1;
    constexpr int Q = 4 + 1 + NSZ;               // copies per wave and stage

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int nl = lane & 15, kb = lane >> 4;
    const int ngroups = K / G;
    const int nstages = (K + KS - 1) / KS;

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

    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t *)&smem[0][0]));
    // x: copy i of wave w fills rows 8 (4w + i) .. +8; lane l row + l / 8,
    // 16-byte slot l % 8 holding k-piece (l % 8) ^ (row % 8)

    uint32_t a_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a_row[i] = static_cast<uint32_t>(min(m0 + (wave * 4 + i) * 8 + (lane >> 3), M - 1));
    // codes: lane l of wave w fills row 32 w + l / 2, 16-byte half l % 2,
    // holding k-half (l % 2) ^ ((row / 8) % 2) (swizzle against conflicts)
    const int b_r = wave * 32 + (lane >> 1);
    const int b_half = (lane & 1) ^ ((b_r >> 3) & 1);
    const uint8_t *b_src = codes + static_cast<int64_t>(min(n0 + b_r, N - 1)) * (K >> 1) + b_half * 16;

    auto issue = [&](int kt, int buf) {
        const uint32_t base = lds0 + static_cast<uint32_t>(buf) * STAGE_BYTES;
        const int k0 = kt * KS;
        const int kp0 = min(k0 + ((lane & 7) ^ (lane >> 4)) * 8, K - 8);
        const int kp1 = min(k0 + ((lane & 7) ^ (4 | (lane >> 4))) * 8, K - 8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            copy16(x + (static_cast<uint64_t>(a_row[i]) * static_cast<uint32_t>(K) +
                        static_cast<uint32_t>((i & 1) ? kp1 : kp0)),
                   base + (wave * 4 + i) * 1024);
        // k = min(k0 + 32 * half, K - 32)
        copy16(b_src + min(k0, K - 32 - b_half * 32) / 2, base + A_BYTES + wave * 1024);
        if constexpr (PK) {
            // (s | z << 16) of the group ends in this stage: value
            // v = 64 w + lane -> row v % 128, end v / 128 (at G >= 64 both
            // ends are the stage's one group end)
            const int v = 64 * wave + lane;
            const int row = v & 127, h = v >> 7;
            const int k_end = k0 + (G == 32 ? (h + 1) * 32 : KS);
            const int g = max(0, min(k_end / G - 1, ngroups - 1));
            copy4(sz + static_cast<int64_t>(min(n0 + row, N - 1)) * ngroups + g,
                  base + A_BYTES + B_BYTES + 256 * wave);
        } else {
            // scales / zero-points of the group ends in this stage: value
            // v = 64 (NSZ w + d) + lane -> row v % 128, s|z (v / 128) % 2, end v / 256
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
    const Unpack128 uc = unpack128_consts();
    float sv[4] = {0.f, 0.f, 0.f, 0.f}, zz[4] = {0.f, 0.f, 0.f, 0.f};
    auto epilogue = [&](int mt) {
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
        const uint8_t *sb = &smem[buf][0];
        bf16x8 a[4], b[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int r = wm * 64 + mt * 16 + nl;
            a[mt] = as_bf16x8(*reinterpret_cast<const u32x4 *>(
                sb + r * 128 + (((sl * 4 + kb) ^ ((r >> 1) & 7)) * 16)));
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int r = wn * 64 + nt * 16 + nl;
            const uint32_t w = *reinterpret_cast<const uint32_t *>(
                sb + A_BYTES + r * 32 + ((sl ^ ((r >> 3) & 1)) * 16) + kb * 4);
            uint32_t u[4];
            if constexpr (PK)
                unpack8_bias128_il(w, u, uc);    // pre-shuffled: natural k order
            else
                unpack8_bias128(w, u, uc);
            b[nt] = as_bf16x8(u[0], u[1], u[2], u[3]);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if constexpr (first) {
                epilogue(mt);
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
                if constexpr (PK) {
                    const uint32_t pr = szp[h * 128 + c];
                    sv[nt] = bf16_lo(pr);
                    zz[nt] = fmaf(-128.0f, sv[nt], bf16_hi(pr));
                } else {
                    sv[nt] = bf16_to_f32(static_cast<uint16_t>(szp[h * 256 + c]));
                    zz[nt] = fmaf(-128.0f, sv[nt], bf16_to_f32(static_cast<uint16_t>(szp[h * 256 + 128 + c])));
                }
            }
        }
    };

    // prologue: stages 0 and 1 in flight, wait for stage 0
    issue(0, 0);
    issue(min(1, nstages - 1), 1);
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(Q) : "memory");
    __syncthreads();

    auto stage = [&](auto par_c, int kt) {
        const int buf = kt % NBUF;
        // stage kt + 2 goes into the buffer read in stage kt - 1 (every wave
        // is past the barrier that ended it); past the end it repeats the
        // last stage into a buffer that is not read again
        issue(min(kt + 2, nstages - 1), (kt + 2) % NBUF);
        slice(buf, par_c, IC<0>{});
        if constexpr (G == 32) {
            if (kt * KS + 32 < K) slice(buf, par_c, IC<1>{});   // K % 64 == 32: half stage
        } else {
            slice(buf, par_c, IC<1>{});
        }
        // stage kt + 1 has landed (stage kt + 2 may still be in flight)
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"(Q) : "memory");
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
    for (int mt = 0; mt < 4; ++mt) epilogue(mt);

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

} // namespace

hipError_t launch_gemm(const uint16_t *x, int64_t M, const uint8_t *codes,
                       const uint16_t *scales, const uint16_t *zeros, const uint32_t *sz,
                       const uint16_t *bias, int64_t N, int64_t K, int G,
                       uint16_t *y, hipStream_t stream) {
    const bool pk = sz != nullptr;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    // one launch per 2^22 tiles keeps blocks x threads below 2^32
    constexpr int64_t kMaxTiles = int64_t(1) << 22;
    for (int64_t t0 = 0; t0 < tiles; t0 += kMaxTiles) {
        const int64_t nt = min(kMaxTiles, tiles - t0);
        const dim3 grid(static_cast<unsigned>(nt));
        const dim3 block(THREADS);
#define W4_GEMM_LAUNCH(GG, PP) \
    gemm_kernel<GG, PP><<<grid, block, 0, stream>>>(x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt)
        switch (G) {
        case 32: if (pk) W4_GEMM_LAUNCH(32, true); else W4_GEMM_LAUNCH(32, false); break;
        case 64: if (pk) W4_GEMM_LAUNCH(64, true); else W4_GEMM_LAUNCH(64, false); break;
        case 128: if (pk) W4_GEMM_LAUNCH(128, true); else W4_GEMM_LAUNCH(128, false); break;
        default: return hipErrorInvalidValue;
        }
#undef W4_GEMM_LAUNCH
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

} // namespace w4
