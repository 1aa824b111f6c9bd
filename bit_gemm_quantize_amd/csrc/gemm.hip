// Prefill-path W4A16 GEMM (any M, meant for M > 16) for gfx950.
//
// Same result as the GEMV: per output, in float32,
//   sum_g ( s[n][g] * sum_{k in g} x[m][k] q[n][k] + z[n][g] * sum_{k in g} x[m][k] )
// ("Optimum Quanto": wide accumulation, then dequantization; bias in float).
//
// Block tile 128 (m) x 128 (n), four waves in a 2 x 2 grid, 64 x 64 each.
// K advances in stages of 64 (two 32-wide slices), double buffered in LDS.
// The x tile is copied global -> LDS directly (16 bytes per lane, XOR
// swizzled rows); the code tile goes through registers and is expanded on
// its way into LDS to the exact bf16 integers 128 + q. Each slice runs
// 16x16x32 bf16 MFMAs into a per-group accumulator, plus one MFMA against an
// all-ones B for the group sums of x in the same layout. After a group, in
// float32:
//   acc += s * acc_g + (z - 128 s) * xsum_g
// (128 + q is exact in bf16 and the MFMA accumulates exactly-representable
// products in float32, so the only rounding is the float32 accumulation.)
#include <type_traits>

#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

constexpr int BM = 128, BN = 128, KS = 64;
constexpr int LD = KS + 8;                     // bf16 elements per LDS row
constexpr int THREADS = 256;

template <int V>
using IC = std::integral_constant<int, V>;

template <int G>
__global__ __launch_bounds__(THREADS, 2) void gemm_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int N, int K, uint16_t *__restrict__ y,
    int64_t tile0, int64_t ntiles) {
    // x tile (swizzled, see below) and the expanded code tile (bf16 128 + q,
    // rows padded by 16 bytes against bank conflicts); both double buffered.
    __shared__ __attribute__((aligned(1024))) uint16_t A0[BM * KS];
    __shared__ __attribute__((aligned(1024))) uint16_t A1[BM * KS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LD];
    __shared__ uint16_t S16[2][2][BN], Z16[2][2][BN];   // s, z per group end

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nl = lane & 15, kb = lane >> 4;
    const int ngroups = K / G;
    const int nstages = (K + KS - 1) / KS;
    const int64_t code_ld = K >> 1;

    // Tile order. Workgroups go to the 8 XCDs round-robin (block b to XCD
    // b % 8), each XCD with its own L2. Block b is given tile t so that each
    // XCD runs one contiguous run of the tile order, and the tile order walks
    // groups of up to 4 m-tiles, n-tile by n-tile: the blocks an XCD runs at
    // once (64 of them) then share 4 row tiles of x and 16 tiles of codes,
    // which its L2 keeps while they move along K together.
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

    // Staging. Loads are unconditional with clamped addresses: rows past M
    // or N only feed outputs that are never stored, and a stage past K
    // (K % 64 == 32) is never read.
    // x goes straight to LDS (16 bytes per lane per load): load i of wave w
    // fills rows 8 (4w + i) .. +8, lane l row + l / 8, 16-byte slot l % 8,
    // which holds k-piece (l % 8) ^ (row % 8) (XOR swizzle against bank
    // conflicts of the fragment reads).
    // codes: 128 rows x 2 pieces of 16 B (32 codes); thread tid loads piece
    // tid into registers.
    const int a_r8 = lane >> 3;
    const int a_piece = (lane & 7) ^ (a_r8 & 7);
    uint32_t a_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a_row[i] = static_cast<uint32_t>(min(m0 + (wave * 4 + i) * 8 + a_r8, M - 1));
    const int b_row = tid >> 1, b_half = tid & 1;
    const uint8_t *b_src = codes + static_cast<int64_t>(min(n0 + b_row, N - 1)) * code_ld +
                           b_half * 16;

    // LDS byte addresses of the two x buffers
    const uint32_t a_lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint16_t *)A0));
    const uint32_t a_lds1 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint16_t *)A1));
    auto load_stage = [&](int kt, int dbuf, u32x4 &rb) {
        const int k0 = kt * KS;
        const uint32_t k = static_cast<uint32_t>(min(k0 + a_piece * 8, K - 8));
        const uint32_t base = __builtin_amdgcn_readfirstlane((dbuf ? a_lds1 : a_lds0) + wave * 4 * 1024);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint16_t *g = x + (static_cast<uint64_t>(a_row[i]) * static_cast<uint32_t>(K) + k);
            const uint32_t l = base + i * 1024;
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                         :
                         : "v"(g), "s"(l)
                         : "memory", "m0");
        }
        // k = min(k0 + 32 * half, K - 32); cached: every m-tile reads it
        rb = *reinterpret_cast<const u32x4 *>(b_src + min(k0, K - 32 - b_half * 32) / 2);
    };
    // The codes are expanded once per block here, on their way into LDS, to
    // the exact bf16 integers 128 + q (natural k order, like x).
    const Unpack128 uc = unpack128_consts();
    auto store_stage = [&](int buf, const u32x4 &rb) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t u[4];
            unpack8_bias128(rb[w], u, uc);
            *reinterpret_cast<u32x4 *>(&Bs[buf][b_row][b_half * 32 + 8 * w]) =
                u32x4{u[0], u[1], u[2], u[3]};
        }
    };

    // Scales and zero-points of the groups that end inside a stage go
    // through LDS with the tiles: thread t fetches row t % 128 of the block
    // for group end h = t / 128 (for G = 32 one at the end of each slice,
    // for G = 64 / 128 at most one, at the end of slice 1). The index is
    // clamped; entries of groups that do not end are never read.
    const int sz_row = tid & (BN - 1), sz_h = tid >> 7;
    const int64_t sz_base = static_cast<int64_t>(min(n0 + sz_row, N - 1)) * ngroups;
    auto load_sz = [&](int kt) -> u32x2 {
        const int k_end = kt * KS + (G == 32 ? (sz_h + 1) * 32 : KS);
        // for G = 128 no group ends in even stages: k_end / G - 1 can be -1
        const int64_t g = sz_base + max(0, min(k_end / G - 1, ngroups - 1));
        return u32x2{scales[g], zeros[g]};
    };

    // accg / xsg / sv / zz start at zero so that the deferred epilogue at the
    // first slice of the first group adds nothing.
    f32x4 acc[4][4], accg[4][4], xsg[4];
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        xsg[i] = zero4;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = accg[i][j] = zero4;
    }
    const bf16x8 ones = bf16x8_ones();

    {
        u32x4 rb;
        load_stage(0, 0, rb);
        const u32x2 sz = load_sz(0);
        store_stage(0, rb);
        S16[0][sz_h][sz_row] = static_cast<uint16_t>(sz[0]);
        Z16[0][sz_h][sz_row] = static_cast<uint16_t>(sz[1]);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();

    // deferred group epilogue: acc += s * acc_g + (z - 128 s) * xsum_g
    float sv[4] = {0.f, 0.f, 0.f, 0.f}, zz[4] = {0.f, 0.f, 0.f, 0.f};
    auto epilogue = [&](int mt) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[mt][nt][i] = fmaf(sv[nt], accg[mt][nt][i], fmaf(zz[nt], xsg[mt][i], acc[mt][nt][i]));
    };

    // Slice sl of a stage held in LDS buffer buf; par is the stage's parity
    // for G = 128 (a group spans two stages). Where groups start and end is
    // known at compile time: G = 128 spans a pair of stages, G = 64 a stage,
    // G = 32 a slice.
    auto slice = [&](int buf, auto par_c, auto sl_c) {
        constexpr int par = decltype(par_c)::value;
        constexpr int sl = decltype(sl_c)::value;
        constexpr bool first = G == 128 ? (par == 0 && sl == 0) : (G == 64 ? sl == 0 : true);
        constexpr bool last = G == 128 ? (par == 1 && sl == 1) : (G == 64 ? sl == 1 : true);
        const uint16_t *Ab = buf ? A1 : A0;
        bf16x8 a[4], b[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int r = wm * 64 + mt * 16 + nl;
            a[mt] = as_bf16x8(*reinterpret_cast<const u32x4 *>(
                Ab + r * KS + (((sl * 4 + kb) ^ (r & 7)) * 8)));
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
            b[nt] = as_bf16x8(*reinterpret_cast<const u32x4 *>(
                &Bs[buf][wn * 64 + nt * 16 + nl][sl * 32 + kb * 8]));
        // The epilogue of the previous group runs in the first slice of the
        // next one, one m-tile at a time, while the MFMAs of the previous
        // m-tile are in flight: it reads accg / xsg of m-tile mt just before
        // this slice's first MFMAs overwrite them.
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if constexpr (first) {
                epilogue(mt);
                // Pin the order: the updated acc is materialised here, and
                // this m-tile's MFMAs (which start new accumulators) take an
                // operand that passes through the same point, so the old
                // accumulators die before the new ones are written.
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
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int c = wn * 64 + nt * 16 + nl;
                sv[nt] = bf16_to_f32(S16[buf][h][c]);
                zz[nt] = fmaf(-128.0f, sv[nt], bf16_to_f32(Z16[buf][h][c]));
            }
        }
    };

    auto stage = [&](int buf, auto par_c, int kt) {
        const bool more = kt + 1 < nstages;
        u32x4 rb;
        // (the last stage reloads itself into the other buffer: unused)
        load_stage(more ? kt + 1 : kt, buf ^ 1, rb);
        const u32x2 sz_nxt = load_sz(more ? kt + 1 : kt);
        __builtin_amdgcn_sched_barrier(0);      // issue the loads first
        slice(buf, par_c, IC<0>{});
        if constexpr (G == 32) {
            if (kt * KS + 32 < K) slice(buf, par_c, IC<1>{});   // K % 64 == 32: half stage
        } else {
            slice(buf, par_c, IC<1>{});                          // K % 64 == 0
        }
        // (unconditional: after the last stage the other buffer is not read)
        store_stage(buf ^ 1, rb);
        S16[buf ^ 1][sz_h][sz_row] = static_cast<uint16_t>(sz_nxt[0]);
        Z16[buf ^ 1][sz_h][sz_row] = static_cast<uint16_t>(sz_nxt[1]);
        // the x tile of the next stage has landed in LDS
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };

    if constexpr (G == 128) {
        // K is a multiple of 128: the stage count is even
        for (int kt = 0; kt < nstages; kt += 2) {
            stage(0, IC<0>{}, kt);
            stage(1, IC<1>{}, kt + 1);
        }
    } else {
        for (int kt = 0; kt < nstages; ++kt) stage(kt & 1, IC<0>{}, kt);
    }

    // the last group ends with the last slice
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) epilogue(mt);

    // Store: lane holds rows 4*kb + i of each 16 x 16 tile, column nl.
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
                       const uint16_t *scales, const uint16_t *zeros,
                       const uint16_t *bias, int64_t N, int64_t K, int G,
                       uint16_t *y, hipStream_t stream) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    // one launch per 2^22 tiles keeps blocks x threads below 2^32
    constexpr int64_t kMaxTiles = int64_t(1) << 22;
    for (int64_t t0 = 0; t0 < tiles; t0 += kMaxTiles) {
        const int64_t nt = min(kMaxTiles, tiles - t0);
        const dim3 grid(static_cast<unsigned>(nt));
        const dim3 block(THREADS);
        switch (G) {
        case 32: gemm_kernel<32><<<grid, block, 0, stream>>>(x, m, codes, scales, zeros, bias, n, k, y, t0, nt); break;
        case 64: gemm_kernel<64><<<grid, block, 0, stream>>>(x, m, codes, scales, zeros, bias, n, k, y, t0, nt); break;
        case 128: gemm_kernel<128><<<grid, block, 0, stream>>>(x, m, codes, scales, zeros, bias, n, k, y, t0, nt); break;
        default: return hipErrorInvalidValue;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

} // namespace w4
