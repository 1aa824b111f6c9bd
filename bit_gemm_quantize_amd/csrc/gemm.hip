// Prefill-path W4A16 GEMM (any M, meant for M > 16) for gfx950.
//
// Same result as the GEMV: per output, in float32,
//   sum_g ( s[n][g] * sum_{k in g} x[m][k] q[n][k] + z[n][g] * sum_{k in g} x[m][k] )
// ("Optimum Quanto": wide accumulation, then dequantization; bias in float).
//
// Block tile 128 (m) x BN (n), BN = 128 (four waves in a 2 x 2 grid) or 256
// (eight waves in a 2 x 4 grid), 64 x 64 per wave; with at most one 128-wide
// tile per compute unit, two such groups of four waves split K in one block.
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

constexpr int BM = 128, KS = 64;
constexpr int NBUF = 3;                          // stages in LDS (two in flight)
constexpr int A_BYTES = BM * KS * 2;             // x tile, bf16, swizzled rows

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

// Buffer-descriptor words for [p, p + bytes) (wave-uniform; lives in SGPRs).
// Loads past `bytes` return 0.
__device__ __forceinline__ u32x4 rsrc_words(const void *p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    u32x4 r;
    r.x = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    r.y = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    r.z = __builtin_amdgcn_readfirstlane(bytes);
    r.w = 0x00020000u;
    return r;
}
// 16 / 4 / 2 bytes per lane from buffer offset voff + soff into LDS at
// lds (wave-uniform) + size * lane (2-byte copies: + 4 * lane, zero-extended).
// The per-lane offset is fixed for the whole K loop and the stage advance is
// the scalar soff, so issuing a stage costs no vector instructions.
__device__ __forceinline__ void bcopy16(u32x4 rs, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 : : "v"(voff), "s"(rs), "s"(soff), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void bcopy4(u32x4 rs, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 : : "v"(voff), "s"(rs), "s"(soff), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void bcopy2(u32x4 rs, uint32_t voff, uint32_t soff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_ushort %0, %1, %2 offen lds"
                 : : "v"(voff), "s"(rs), "s"(soff), "s"(lds) : "memory", "m0");
}

// BUF: copies through buffer descriptors over the block's rows (needs
// 128 * K * 2 < 2^32, i.e. K < 2^24); otherwise 64-bit global addresses
// recomputed per stage. BNT: block tile columns, 128 or 256 (2 BNT threads;
// per stage the x tile is shared by BNT / 64 wave columns, so the wider
// block issues a third fewer copies per MFMA). KSP = 2 (128-wide tiles,
// buffer path): two groups of four waves split K in halves inside one block,
// each with its own stage buffers, and the second group's sums are added
// through LDS at the end; a grid of at most one tile per compute unit then
// still runs two waves per SIMD.
template <int G, bool PK, bool BUF, int BNT, int KSP = 1>
__global__ __launch_bounds__(BNT * 2 * KSP, 2) void gemm_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint32_t *__restrict__ sz, const uint16_t *__restrict__ bias, int N, int K,
    uint16_t *__restrict__ y, int64_t tile0, int64_t ntiles) {
    static_assert(BNT == 128 || BNT == 256, "block tile columns");
    static_assert(KSP == 1 || (KSP == 2 && BNT == 128 && BUF), "K split inside the block");
    constexpr int BNk = BNT;
    constexpr int NW = BNk / 32;                 // waves per block (per K group)
    constexpr int WN = BNk / 64;                 // waves along n
    constexpr int XC = 16 / NW;                  // x copies per wave and stage
    constexpr int B_BYTESk = BNk * KS / 2;       // code tile, packed nibbles
    constexpr int SZ_BYTESk = 2 * 2 * BNk * 4;   // [group end][s | z][row], 4 B each
    constexpr int STAGE_BYTESk = A_BYTES + B_BYTESk + SZ_BYTESk;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[KSP][NBUF][STAGE_BYTESk];
    // scale / zero-point copies per wave and stage (2 bytes each, or one
    // 4-byte pair each in the pre-shuffled layout)
    constexpr int NSZ = (G == 32 && !PK) ? 2 : 1;
    constexpr int Q = XC + 1 + NSZ;              // copies per wave and stage
    // At G = 128 a group spans two stages and ends in the odd one: only odd
    // stages copy scales / zero-points (even stages issue Q - NSZ copies).
    constexpr bool SZ_ALL = G != 128;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave: index inside its K group wg (wave-uniform); the group covers
    // k in [kbase, kbase + K / KSP)
    const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) % NW);
    const int wg = KSP == 1 ? 0 : __builtin_amdgcn_readfirstlane((tid >> 6) / NW);
    const int wm = wave / WN, wn = wave % WN;
    const int nl = lane & 15, kb = lane >> 4;
    const int ngroups = K / G;
    const int Kg = K / KSP;
    const int kbase = wg * Kg;
    const int nstages = (Kg + KS - 1) / KS;

    int m0, n0;
    {
        const int64_t T = ntiles, b = blockIdx.x;
        const int64_t xcd = b & 7, j = b >> 3;
        const int64_t t = tile0 + xcd * (T >> 3) + min(xcd, T & 7) + j;
        const int64_t mtiles = (M + BM - 1) / BM, ntl = (N + BNk - 1) / BNk;
        const int64_t gm = min<int64_t>(4, mtiles);
        const int64_t grp = t / (gm * ntl), r = t - grp * gm * ntl;
        const int64_t gsz = min(gm, mtiles - grp * gm);
        m0 = static_cast<int>((grp * gm + r % gsz) * BM);
        n0 = static_cast<int>((r / gsz) * BNk);
    }

    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t *)&smem[wg][0][0]));
    // x: copy i of wave w fills rows 8 (4w + i) .. +8; lane l row + l / 8,
    // 16-byte slot l % 8 holding k-piece (l % 8) ^ (row % 8)

    uint32_t a_row[XC];
#pragma unroll
    for (int i = 0; i < XC; ++i)
        a_row[i] = static_cast<uint32_t>(min(m0 + (wave * XC + i) * 8 + (lane >> 3), M - 1));
    // codes: lane l of wave w fills row 32 w + l / 2, 16-byte half l % 2,
    // holding k-half (l % 2) ^ ((row / 8) % 2) (swizzle against conflicts)
    const int b_r = wave * 32 + (lane >> 1);
    const int b_half = (lane & 1) ^ ((b_r >> 3) & 1);
    const uint8_t *b_src = codes + static_cast<int64_t>(min(n0 + b_r, N - 1)) * (K >> 1) + b_half * 16;

    // buffer path: descriptors over the block's rows, fixed per-lane offsets
    const int rows_m = min(BM, M - m0), rows_n = min(BNk, N - n0);
    const uint32_t kh = static_cast<uint32_t>(K) >> 1;
    u32x4 xr = {0u, 0u, 0u, 0u}, cr = xr, sr = xr, zr = xr;
    uint32_t xo[2] = {0u, 0u}, co = 0u, so[NSZ > 1 ? NSZ : 1] = {};
    if constexpr (BUF) {
        xr = rsrc_words(x + static_cast<int64_t>(m0) * K, static_cast<uint32_t>(rows_m) * K * 2);
        cr = rsrc_words(codes + static_cast<int64_t>(n0) * kh, static_cast<uint32_t>(rows_n) * kh);
        if constexpr (PK) {
            sr = rsrc_words(sz + static_cast<int64_t>(n0) * ngroups, rows_n * ngroups * 4);
        } else {
            sr = rsrc_words(scales + static_cast<int64_t>(n0) * ngroups, rows_n * ngroups * 2);
            zr = rsrc_words(zeros + static_cast<int64_t>(n0) * ngroups, rows_n * ngroups * 2);
        }
        // x copy i: row 8 (4 w + i) + lane / 8, piece (lane % 8) ^ (row / 2 % 8): the
        // row term of copy i is 32 w + 8 i, so copies of equal i % 2 share the
        // swizzle and differ by 8 rows
        const uint32_t r0 = (wave * 8 * XC + (lane >> 3)) * static_cast<uint32_t>(K);
        xo[0] = (r0 + ((lane & 7) ^ (lane >> 4)) * 8) * 2;
        xo[1] = (r0 + 8 * static_cast<uint32_t>(K) + ((lane & 7) ^ (4 | (lane >> 4))) * 8) * 2;
        co = static_cast<uint32_t>(b_r) * kh + b_half * 16;
        if constexpr (PK) {
            so[0] = static_cast<uint32_t>((64 * wave + lane) & (BNk - 1)) * ngroups * 4;
        } else {
#pragma unroll
            for (int d = 0; d < NSZ; ++d)
                so[d] = static_cast<uint32_t>((64 * (NSZ * wave + d) + lane) & (BNk - 1)) * ngroups * 2;
        }
    }

    auto issue = [&](int kt, int buf) {
        const uint32_t base = lds0 + static_cast<uint32_t>(buf) * STAGE_BYTESk;
        const int k0 = kbase + kt * KS;
        if constexpr (BUF) {
            const uint32_t xs = static_cast<uint32_t>(k0) * 2;
#pragma unroll
            for (int i = 0; i < XC; ++i)
                bcopy16(xr, xo[i & 1] + (i >> 1) * 16 * static_cast<uint32_t>(K) * 2, xs,
                        base + (wave * XC + i) * 1024);
            bcopy16(cr, co, static_cast<uint32_t>(k0) >> 1, base + A_BYTES + wave * 1024);
            if (!SZ_ALL && !(kt & 1)) {
                // G = 128: the stage holds no group end, its scale slots are not read
            } else if constexpr (PK) {
                const int h = (64 * wave) / BNk;
                const int k_end = k0 + (G == 32 ? (h + 1) * 32 : KS);
                const int g = max(0, min(k_end / G - 1, ngroups - 1));
                bcopy4(sr, so[0], static_cast<uint32_t>(g) * 4, base + A_BYTES + B_BYTESk + 256 * wave);
            } else {
#pragma unroll
                for (int d = 0; d < NSZ; ++d) {
                    const int v0 = 64 * (NSZ * wave + d);          // wave-uniform part
                    const int isz = (v0 / BNk) & 1, h = v0 / (2 * BNk);
                    const int k_end = k0 + (G == 32 ? (h + 1) * 32 : KS);
                    const int g = max(0, min(k_end / G - 1, ngroups - 1));
                    bcopy2(isz ? zr : sr, so[d], static_cast<uint32_t>(g) * 2,
                           base + A_BYTES + B_BYTESk + 64 * 4 * (NSZ * wave + d));
                }
            }
            return;
        }
        const int kp0 = min(k0 + ((lane & 7) ^ (lane >> 4)) * 8, K - 8);
        const int kp1 = min(k0 + ((lane & 7) ^ (4 | (lane >> 4))) * 8, K - 8);
#pragma unroll
        for (int i = 0; i < XC; ++i)
            copy16(x + (static_cast<uint64_t>(a_row[i]) * static_cast<uint32_t>(K) +
                        static_cast<uint32_t>((i & 1) ? kp1 : kp0)),
                   base + (wave * XC + i) * 1024);
        // k = min(k0 + 32 * half, K - 32)
        copy16(b_src + min(k0, K - 32 - b_half * 32) / 2, base + A_BYTES + wave * 1024);
        if (!SZ_ALL && !(kt & 1)) {
            // G = 128: no group end in this stage
        } else if constexpr (PK) {
            // (s | z << 16) of the group ends in this stage: value
            // v = 64 w + lane -> row v % 128, end v / 128 (at G >= 64 both
            // ends are the stage's one group end)
            const int v = 64 * wave + lane;
            const int row = v & (BNk - 1), h = v / BNk;
            const int k_end = k0 + (G == 32 ? (h + 1) * 32 : KS);
            const int g = max(0, min(k_end / G - 1, ngroups - 1));
            copy4(sz + static_cast<int64_t>(min(n0 + row, N - 1)) * ngroups + g,
                  base + A_BYTES + B_BYTESk + 256 * wave);
        } else {
            // scales / zero-points of the group ends in this stage: value
            // v = 64 (NSZ w + d) + lane -> row v % 128, s|z (v / 128) % 2, end v / 256
#pragma unroll
            for (int d = 0; d < NSZ; ++d) {
                const int v = 64 * (NSZ * wave + d) + lane;
                const int row = v & (BNk - 1), isz = (v / BNk) & 1, h = v / (2 * BNk);
                const int k_end = k0 + (G == 32 ? (h + 1) * 32 : KS);
                const int g = max(0, min(k_end / G - 1, ngroups - 1));
                const uint16_t *src = (isz ? zeros : scales) +
                                      static_cast<int64_t>(min(n0 + row, N - 1)) * ngroups + g;
                copy2(src, base + A_BYTES + B_BYTESk + 64 * 4 * (NSZ * wave + d));
            }
        }
    };

    // Per-lane byte offsets of the fragments inside a stage buffer, slice 0
    // and 1. x row r = 64 wm + 16 mt + nl holds k-piece p in slot
    // p ^ ((r / 2) % 8) (= p ^ ((nl / 2) % 8): the tile steps keep it); code
    // row r = 64 wn + 16 nt + nl holds its k-half h in half h ^ ((r / 8) % 2)
    // (= h ^ ((nl / 8) % 2)). Kept opaque so that they stay in registers
    // instead of being recomputed in every slice.
    uint32_t la[2], lb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        la[s] = static_cast<uint32_t>((wm * 64 + nl) * 128 + (((s * 4 + kb) ^ ((nl >> 1) & 7)) * 16));
        lb[s] = static_cast<uint32_t>(A_BYTES + (wn * 64 + nl) * 32 + ((s ^ ((nl >> 3) & 1)) * 16) + kb * 4);
        asm volatile("" : "+v"(la[s]), "+v"(lb[s]));
    }
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
        const uint8_t *sb = &smem[wg][buf][0];
        // one add per operand and slice: the per-lane offsets are fixed, the
        // m- / n-tile steps are immediates
        const uint8_t *sa = sb + la[sl];
        const uint8_t *sw = sb + lb[sl];
        bf16x8 a[4], b[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            a[mt] = as_bf16x8(*reinterpret_cast<const u32x4 *>(sa + mt * 16 * 128));
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(sw + nt * 16 * 32);
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
            const uint32_t *szp = reinterpret_cast<const uint32_t *>(sb + A_BYTES + B_BYTESk);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int c = wn * 64 + nt * 16 + nl;
                if constexpr (PK) {
                    const uint32_t pr = szp[h * BNk + c];
                    sv[nt] = bf16_lo(pr);
                    zz[nt] = fmaf(-128.0f, sv[nt], bf16_hi(pr));
                } else {
                    sv[nt] = bf16_to_f32(static_cast<uint16_t>(szp[h * 2 * BNk + c]));
                    zz[nt] = fmaf(-128.0f, sv[nt], bf16_to_f32(static_cast<uint16_t>(szp[h * 2 * BNk + BNk + c])));
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
        // the buffer index is made opaque: left visible, the compiler turns
        // it into a per-lane induction variable that costs two vector ops
        // per fragment read (a scalar offset costs one)
        int buf = kt % NBUF;
        asm volatile("" : "+s"(buf));
        // stage kt + 2 goes into the buffer read in stage kt - 1 (every wave
        // is past the barrier that ended it); past the end it repeats the
        // last stage into a buffer that is not read again
        issue(min(kt + 2, nstages - 1), (kt + 2) % NBUF);
        slice(buf, par_c, IC<0>{});
        if constexpr (G == 32) {
            if (kt * KS + 32 < Kg) slice(buf, par_c, IC<1>{});  // K % 64 == 32: half stage
        } else {
            slice(buf, par_c, IC<1>{});
        }
        // stage kt + 1 has landed (stage kt + 2, of the same parity as kt,
        // may still be in flight; past the end the repeated last stage is odd
        // and issues at least as many copies, so the wait is never short)
        constexpr int QW = (!SZ_ALL && decltype(par_c)::value == 0) ? Q - NSZ : Q;
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
    for (int mt = 0; mt < 4; ++mt) epilogue(mt);

    if constexpr (KSP == 2) {
        // the second K half's sums, through its own (now idle) stage buffers:
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

} // namespace

hipError_t launch_gemm(const uint16_t *x, int64_t M, const uint8_t *codes,
                       const uint16_t *scales, const uint16_t *zeros, const uint32_t *sz,
                       const uint16_t *bias, int64_t N, int64_t K, int G,
                       uint16_t *y, hipStream_t stream) {
    const bool pk = sz != nullptr;
    const bool buf = K < (int64_t(1) << 24);      // 32-bit buffer offsets over 128 rows
    const int64_t mtiles = (M + BM - 1) / BM;
    // 128 x 256 blocks (one per compute unit) when there are enough of them to
    // fill the chip (at least 15/16 of a block per compute unit): measured
    // 2-7 % faster than 128 x 128 blocks on the Gemma3-12B-shaped q, o, gate
    // and down layers at M = 2048, G = 64 and 128, both layouts (even on
    // gate at G = 64, pre-shuffled). With fewer tiles (k and v: half a block
    // per compute unit) and at G = 32 (two scale / zero-point copies per
    // stage) the 128 x 128 block is faster.
    const int64_t wide_tiles = mtiles * ((N + 255) / 256);
    const int64_t cus = compute_units();
    const bool wide = buf && G >= 64 && wide_tiles * 16 >= cus * 15;
    const int64_t bn = wide ? 256 : 128;
    const int64_t tiles = mtiles * ((N + bn - 1) / bn);
    // at most one 128 x 128 tile per compute unit (k and v of the Gemma3-12B
    // shapes at M = 2048: one four-wave block per unit, one wave per SIMD):
    // split K inside eight-wave blocks, each half a multiple of the stage
    // pair and the group
    const bool ksplit = !wide && buf && tiles <= cus && K % (2 * (G > KS ? G : KS)) == 0;
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    // one launch per 2^22 tiles keeps blocks x threads below 2^32
    constexpr int64_t kMaxTiles = int64_t(1) << 22;
    for (int64_t t0 = 0; t0 < tiles; t0 += kMaxTiles) {
        const int64_t nt = min(kMaxTiles, tiles - t0);
        const dim3 grid(static_cast<unsigned>(nt));
        const dim3 block(static_cast<unsigned>(2 * bn * (ksplit ? 2 : 1)));
#define W4_GEMM_LAUNCH(GG, PP)                                                               \
    do {                                                                                     \
        if (buf)                                                                             \
            gemm_kernel<GG, PP, true, 128><<<grid, block, 0, stream>>>(                       \
                x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);                      \
        else                                                                                 \
            gemm_kernel<GG, PP, false, 128><<<grid, block, 0, stream>>>(                      \
                x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);                      \
    } while (0)
        if (ksplit) {
            switch (G) {
            case 32:
                if (pk) gemm_kernel<32, true, true, 128, 2><<<grid, block, 0, stream>>>(
                            x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);
                else gemm_kernel<32, false, true, 128, 2><<<grid, block, 0, stream>>>(
                            x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);
                break;
            case 64:
                if (pk) gemm_kernel<64, true, true, 128, 2><<<grid, block, 0, stream>>>(
                            x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);
                else gemm_kernel<64, false, true, 128, 2><<<grid, block, 0, stream>>>(
                            x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);
                break;
            case 128:
                if (pk) gemm_kernel<128, true, true, 128, 2><<<grid, block, 0, stream>>>(
                            x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);
                else gemm_kernel<128, false, true, 128, 2><<<grid, block, 0, stream>>>(
                            x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);
                break;
            default: return hipErrorInvalidValue;
            }
        } else if (wide) {
            if (G == 64 && pk)
                gemm_kernel<64, true, true, 256><<<grid, block, 0, stream>>>(
                    x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);
            else if (G == 64)
                gemm_kernel<64, false, true, 256><<<grid, block, 0, stream>>>(
                    x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);
            else if (pk)
                gemm_kernel<128, true, true, 256><<<grid, block, 0, stream>>>(
                    x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);
            else
                gemm_kernel<128, false, true, 256><<<grid, block, 0, stream>>>(
                    x, m, codes, scales, zeros, sz, bias, n, k, y, t0, nt);
        } else {
            switch (G) {
            case 32: if (pk) W4_GEMM_LAUNCH(32, true); else W4_GEMM_LAUNCH(32, false); break;
            case 64: if (pk) W4_GEMM_LAUNCH(64, true); else W4_GEMM_LAUNCH(64, false); break;
            case 128: if (pk) W4_GEMM_LAUNCH(128, true); else W4_GEMM_LAUNCH(128, false); break;
            default: return hipErrorInvalidValue;
            }
        }
#undef W4_GEMM_LAUNCH
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

} // namespace w4
