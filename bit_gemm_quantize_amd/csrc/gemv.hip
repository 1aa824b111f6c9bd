// Decode-path W4A16 GEMV (1 <= M <= 16) for gfx950.
//
// y[m][n] = sum_g ( s[n][g] * sum_{k in g} x[m][k] q[n][k]
//                 + z[n][g] * sum_{k in g} x[m][k] ) (+ bias[n])
// ("Optimum Quanto": bf16-int4 matmul, accumulated in float32 and
// dequantized afterwards; bias kept in float.)
//
// The codes are streamed once from HBM. Common to both kernels below:
//   * a tile is 16 output features (rows of the code matrix); the waves that
//     share a tile split K into runs of 128-wide chunks and add their partial
//     sums through LDS;
//   * per chunk, lane l (feature l%16, quarter kb = l/16) loads 16 bytes =
//     32 codes (k = 128c + 32kb ... +32) with one 128-bit load, so a wave
//     load covers 64 contiguous bytes of each of 16 rows; the loads of the
//     next chunks are in flight while the current ones are computed;
//   * codes are expanded in registers to the exact bf16 integers 128 + q and
//     fed with bf16 x (staged in LDS) to the 16x16x32 matrix-core op; the
//     M <= 16 rows of x fill the A operand (rows >= M repeat row M - 1 and
//     are never stored);
//   * each MFMA must contract a single group, so for G = 64 / 32 the four
//     dwords a lane holds are first exchanged across the lane quarters
//     (permlane swaps) so that slot j of every quarter lies in one group;
//   * at the end of a group, in float32:
//         acc += s * acc_g + (z - 128 s) * xsum_g,
//     with xsum_g = sum_{k in g} x[m][k] staged beside x (split kernel) or
//     from a second MFMA against an all-ones B (phased kernel).

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
constexpr int GV_SPLIT_MAX_M = 16;      // split-K kernel: M <= 16 ...
constexpr int GV_SPLIT_WAVES = 8;       // split-K kernel: waves per block
constexpr int GV_SPLIT_MAX_LDS = 160 * 1024;   // ... when its LDS fits one CU

// Codes of U consecutive chunks of one lane, plus the scales and zero-points
// of the batch's U * 128 / G groups for the wave's 16 rows, loaded with
// consecutive lanes on consecutive groups of a row: register r, lane l holds
// (s | z << 16) of row l / 4, group 4r + l % 4 of the batch.
template <int G, int U>
struct Batch {
    static constexpr int GPB = U * 128 / G;     // groups per batch (4 or 8)
    static constexpr int R = GPB / 4;
    u32x4 q[U];
    uint32_t s[R];
    uint32_t z[R];
};

// Issue the loads of one batch: scales/zeros first (needed at the first
// group end), then the codes. All addresses are clamped, never predicated.
template <int G, int U>
__device__ __forceinline__ void load_batch(Batch<G, U> &b, const uint8_t *crow,
                                           const uint16_t *__restrict__ scales,
                                           const uint16_t *__restrict__ zeros,
                                           int row0, int N, int K, int ngroups,
                                           int c, int c_last, int lane) {
    constexpr int GPC = 128 / G;
    const int kb = lane >> 4;
    const int srow = min(row0 + (lane >> 2), N - 1);
#pragma unroll
    for (int r = 0; r < Batch<G, U>::R; ++r) {
        const int g = min(c * GPC + 4 * r + (lane & 3), ngroups - 1);
        const int64_t i = static_cast<int64_t>(srow) * ngroups + g;
        b.s[r] = scales[i];
        b.z[r] = zeros[i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int cc = min(c + u, c_last);
        const int kq = min(cc * 128 + kb * 32, K - 32);
        b.q[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(crow + (kq >> 1)));
    }
}

// (s | z << 16) of group h of the batch for this lane's row (lane & 15),
// fetched from the lane that loaded it; packed[r] = s[r] | z[r] << 16.
__device__ __forceinline__ uint32_t batch_sz(const uint32_t *packed, int h, int lane) {
    const int src = ((lane & 15) * 4 + (h & 3)) * 4;     // byte address of the source lane
    return __builtin_amdgcn_ds_bpermute(src, packed[h >> 2]);
}

// The same batch through buffer loads: the addresses are a per-lane offset
// that never changes (row lane % 16 of the tile, quarter lane / 16) plus a
// wave-uniform part, so a load costs no vector arithmetic. The resource
// covers the tile's valid rows only: reads past them (rows >= N) return 0.
// Reads past the end of a row (the padded last chunk when K % 128 != 0, or
// groups past K / G) land in the next row or return 0; they only meet x = 0
// and xs = 0 and add nothing.
template <int G, int U>
__device__ __forceinline__ void load_batch_buf(Batch<G, U> &b, __amdgpu_buffer_rsrc_t crs,
                                               __amdgpu_buffer_rsrc_t srs,
                                               __amdgpu_buffer_rsrc_t zrs, int cvo, int svo,
                                               int c, int c_last) {
    constexpr int GPC = 128 / G;
    constexpr int OOB = 0x40000000;             // past any resource: reads 0, no traffic
#pragma unroll
    for (int r = 0; r < Batch<G, U>::R; ++r) {
        const int so = (c * GPC + 4 * r) * 2;
        b.s[r] = __builtin_amdgcn_raw_buffer_load_b16(srs, svo, so, 0);
        b.z[r] = __builtin_amdgcn_raw_buffer_load_b16(zrs, svo, so, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // chunks past this wave's segment are never computed: not fetched
        const int so = c + u <= c_last ? (c + u) * 64 : OOB;
        b.q[u] = __builtin_amdgcn_raw_buffer_load_b128(crs, cvo, so, 0);
    }
}

template <int G, int NW>
__global__ __launch_bounds__(NW * 64, 2) void gemv_phased_kernel(
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
        load_batch<G, U>(b, crow, scales, zeros, n_base, N, K, ngroups, c, c_last, lane);
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
            uint32_t packed[Batch<G, U>::R];
#pragma unroll
            for (int r = 0; r < Batch<G, U>::R; ++r) packed[r] = (b.s[r] & 0xFFFFu) | (b.z[r] << 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool first = (j % SPG) == 0;
                const int ka = cc * 128 + slot_koff<G>(j, kb) - k_phase;
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(&xl[mrow * kp + ka]));
                uint32_t w[4];
                unpack8_bias128_il(b.q[u][j], w, uc);
                xsg = mfma16x16x32(a, ones, first ? zero4 : xsg);
                accg = mfma16x16x32(a, as_bf16x8(w[0], w[1], w[2], w[3]),
                                    first ? zero4 : accg);
                if ((j % SPG) == SPG - 1) {
                    const uint32_t szv = batch_sz(packed, u * GPC + j / SPG, lane);
                    const float sv = bf16_lo(szv);
                    const float zz = fmaf(-128.0f, sv, bf16_hi(szv));
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
        const int npieces = M * per_row;        // at most GV_X_ELEMS / 8
        {
            // all of a thread's pieces are loaded first (pieces past K read 0
            // from outside the resource), then interleaved into LDS
            constexpr int XP = GV_X_ELEMS / 8 / (NW * 64);
            const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t *>(x), 0, M * K * 2, 0x00020000);
            u32x4 xv[XP];
#pragma unroll
            for (int j = 0; j < XP; ++j) {
                xv[j] = u32x4{0u, 0u, 0u, 0u};
                if (j * NW * 64 >= npieces) break;  // uniform
                const int e = static_cast<int>(threadIdx.x) + j * NW * 64;
                const int m = e / per_row;
                const int kk = (e - m * per_row) * 8;
                const int off = (e < npieces && k_phase + kk < K) ? (m * K + k_phase + kk) * 2
                                                                  : 0x40000000;
                xv[j] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < XP; ++j) {
                const int e = static_cast<int>(threadIdx.x) + j * NW * 64;
                if (e >= npieces) break;
                const int m = e / per_row;
                const int kk = (e - m * per_row) * 8;
                *reinterpret_cast<u32x4 *>(&xl[m * kp + kk]) = interleave8_bf16(xv[j]);
            }
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

// Persistent split-K kernel for 1 <= M <= 16 when x fits in LDS: x[0:M, :]
// is staged in LDS (interleaved, zero padded to whole chunks) together with
// the per-group sums xs[g][m] = sum_{k in g} x[m][k]; each wave stages the K
// segment it reads.
//
// The 8 waves of a block work on T = 8 / S tiles of 16 rows at a time; the
// S waves of a tile split its K range (S = 1, 2, 4 or 8, chosen by the host
// so that the grid has enough waves in flight: narrow layers split K more).
// A wave streams its (tile, K segment) items with the codes of the next two
// items in flight while the current one is computed. With S > 1 the partial
// sums of a tile meet in LDS (one barrier per block step, double buffered);
// with S = 1 each wave stores its tile directly. Lane (nl, kb) holds output
// rows 4 kb .. 4 kb + 3 of column nl; rows >= M are computed (their A rows
// repeat row M - 1) and never stored.
template <int G, int S>
__global__ __launch_bounds__(GV_SPLIT_WAVES * 64, 2) void gemv_split_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int N, int K, uint16_t *__restrict__ y) {
    constexpr int NW = GV_SPLIT_WAVES;
    constexpr int T = NW / S;                   // tiles per block step
    constexpr int SPG = G / 32;
    constexpr int GPC = 128 / G;
    constexpr int U = G == 32 ? 2 : 4;
    constexpr int LPG = G / 8;                  // staging lanes per group
    // dynamic LDS: x [M][kr] bf16 | xs [kr/G][mr] f32 | red [2][NW][mr][16] f32
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
    const int nl = lane & 15;
    const int kb = lane >> 4;
    const int ts = wave / S, sg = wave % S;
    const int nchunk = (K + 127) >> 7;
    const int kr = nchunk * 128;                // LDS row length (zero padded)
    const int mr = (M + 3) & ~3;                // rows of xs and red
    uint16_t *xl = reinterpret_cast<uint16_t *>(smem);
    float *xs = reinterpret_cast<float *>(smem + static_cast<size_t>(M) * kr * 2);
    float *red = xs + static_cast<size_t>(kr / G) * mr;
    const int ngroups = K / G;
    const int ntiles = (N + 15) >> 4;
    const int nsteps = (ntiles + T - 1) / T;    // block steps in the grid
    const int my_steps = (nsteps - static_cast<int>(blockIdx.x) + gridDim.x - 1) / gridDim.x;
    const int mrow = nl < M ? nl : M - 1;
    const int kq = min(kb, (M - 1) >> 2);       // xs rows read by this lane (>= M: dead)
    const Unpack128 uc = unpack128_consts();

    // this wave's K segment (whole chunks); every wave runs nb batches per
    // step (the longest segment's count), shorter segments skip the rest
    const int cb = sg * nchunk / S;
    const int ce = (sg + 1) * nchunk / S;
    const int c_last = max(cb, ce - 1);
    const int nb = ((nchunk + S - 1) / S + U - 1) / U;
    const int nitems = my_steps * nb;

    auto tile_of = [&](int st, int slot) {
        return (static_cast<int>(blockIdx.x) + st * static_cast<int>(gridDim.x)) * T + slot;
    };
    // Loads are unconditional: items past the end reload the last one; the
    // last block step may hold fewer tiles, its extra slots repeat the last.
    const int cvo = nl * (K >> 1) + kb * 16;                  // code byte offset
    const int svo = ((lane >> 2) * ngroups + (lane & 3)) * 2;  // s / z byte offset
    auto load = [&](Batch<G, U> &b, int item) {
        // items past the end (issued by the fixed-depth pipeline) get an
        // empty resource: their loads return 0 without touching memory
        const bool live = item < nitems;
        item = min(item, nitems - 1);
        const int st = item / nb;
        const int c = cb + (item - st * nb) * U;
        const int tile = min(tile_of(st, ts), ntiles - 1);
        const int rows = live ? min(16, N - tile * 16) : 0;
        const int64_t row0 = static_cast<int64_t>(tile) * 16;
        const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(codes + row0 * (K >> 1)), 0, rows * (K >> 1), 0x00020000);
        const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(scales + row0 * ngroups), 0, rows * ngroups * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(zeros + row0 * ngroups), 0, rows * ngroups * 2, 0x00020000);
        load_batch_buf<G, U>(b, crs, srs, zrs, cvo, svo, c, c_last);
    };

    // x staging, per wave: a wave stages only the K segment it reads (rows
    // 0..M-1, whole chunks), so no block barrier is needed before the first
    // step; waves that share a segment (T > 1) write identical values. The
    // segment is cut in runs of 64 pieces of 16 bytes (one per lane) along
    // each row; the first XR runs are issued ahead of the codes of the first
    // two items, so the wait for x leaves the codes in flight.
    Batch<G, U> b0, b1, b2;
    {
        constexpr int XR = 16;                  // runs per round
        const int seg_pr = (ce - cb) * 16;      // pieces per row of the segment
        const int rpr = (seg_pr + 63) >> 6;     // runs per row
        const int nruns = M * rpr;
        const int k0 = cb * 128;
        const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(x), 0, M * K * 2, 0x00020000);
        u32x4 xv[XR];
        // run i covers row i / rpr, pieces 64 (i % rpr) + lane; pieces past
        // the segment or past K are out of the resource: they read 0 and
        // fetch nothing
        auto issue = [&](int r0) {
            int m = r0 / rpr, q = r0 - m * rpr;
#pragma unroll
            for (int j = 0; j < XR; ++j) {
                if (r0 + j >= nruns) break;     // uniform
                const int p = q * 64 + lane;
                const int kk = k0 + p * 8;
                const int off = (p < seg_pr && kk < K) ? (m * K + kk) * 2 : 0x40000000;
                xv[j] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
                if (++q == rpr) { q = 0; ++m; }
            }
        };
        auto put = [&](int r0) {
            int m = r0 / rpr, q = r0 - m * rpr;
#pragma unroll
            for (int j = 0; j < XR; ++j) {
                if (r0 + j >= nruns) break;     // uniform
                const int p = q * 64 + lane;
                const int kk = k0 + p * 8;
                const bool ok = p < seg_pr;
                const u32x4 v = xv[j];
                if (ok) *reinterpret_cast<u32x4 *>(&xl[m * kr + kk]) = interleave8_bf16(v);
                float sum = (bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y)) +
                            (bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w));
                // a group's LPG pieces sit in consecutive lanes of one run
                // (LPG divides 16, runs start at multiples of 512 k), so
                // they reduce with DPP moves
                sum = group_sum<LPG>(sum);
                if (ok && (lane & (LPG - 1)) == 0) xs[(kk / G) * mr + m] = sum;
                if (++q == rpr) { q = 0; ++m; }
            }
        };
        issue(0);
        // items past the end get an empty resource (nitems >= 1 always)
        load(b0, 0);
        load(b1, 1);
        put(0);
        for (int r0 = XR; r0 < nruns; r0 += XR) {
            issue(r0);
            put(r0);
        }
        __builtin_amdgcn_wave_barrier();
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    auto step = [&](Batch<G, U> &b, int item) {
        const int st = item / nb;
        const int bi = item - st * nb;
        const int c = cb + bi * U;
        uint32_t packed[Batch<G, U>::R];
#pragma unroll
        for (int r = 0; r < Batch<G, U>::R; ++r) packed[r] = (b.s[r] & 0xFFFFu) | (b.z[r] << 16);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = c + u;
            if (cc >= ce) break;                // uniform across the wave
            align_groups<G>(b.q[u]);
            f32x4 accg = zero4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool first = (j % SPG) == 0;
                const int ka = cc * 128 + slot_koff<G>(j, kb);
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(&xl[mrow * kr + ka]));
                uint32_t w[4];
                unpack8_bias128_il(b.q[u][j], w, uc);
                accg = mfma16x16x32(a, as_bf16x8(w[0], w[1], w[2], w[3]),
                                    first ? zero4 : accg);
                if ((j % SPG) == SPG - 1) {
                    const uint32_t szv = batch_sz(packed, u * GPC + j / SPG, lane);
                    const float sv = bf16_lo(szv);
                    const float zz = fmaf(-128.0f, sv, bf16_hi(szv));
                    const f32x4 xg = *reinterpret_cast<const f32x4 *>(
                        &xs[(cc * GPC + j / SPG) * mr + 4 * kq]);
                    // All four MFMA results are consumed (also for M = 1):
                    // leaving some of them dead lets the register allocator
                    // reuse an MFMA destination register while the MFMA is
                    // still writing it, which gave wrong results.
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[i] = fmaf(sv, accg[i], fmaf(zz, xg[i], acc[i]));
                }
            }
        }
        if (bi != nb - 1) return;               // end of this block step
        if constexpr (S == 1) {
            const int col = tile_of(st, ts) * 16 + nl;
            if (col < N) {
                const float bv = bias ? bf16_to_f32(bias[col]) : 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * kb + i < M)
                        y[static_cast<int64_t>(4 * kb + i) * N + col] =
                            static_cast<uint16_t>(f32_to_bf16_rne(acc[i] + bv));
            }
            acc = zero4;
        } else {
            const int par = st & 1;
            float *rw = red + (static_cast<size_t>(par * NW + wave) * mr) * 16;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * kb + i < M) rw[(4 * kb + i) * 16 + nl] = acc[i];
            acc = zero4;
            __syncthreads();
            for (int e = threadIdx.x; e < T * M * 16; e += NW * 64) {
                const int slot = e / (M * 16);
                const int rem = e - slot * (M * 16);
                const int m = rem >> 4;
                const int nn = rem & 15;
                const float *rp = red + (static_cast<size_t>(par * NW + slot * S) * mr + m) * 16 + nn;
                float sum = 0.f;
#pragma unroll
                for (int w = 0; w < S; ++w) sum += rp[w * mr * 16];
                const int col = tile_of(st, slot) * 16 + nn;
                if (col < N) {
                    if (bias) sum += bf16_to_f32(bias[col]);
                    y[static_cast<int64_t>(m) * N + col] =
                        static_cast<uint16_t>(f32_to_bf16_rne(sum));
                }
            }
        }
    };

    for (int i = 0; i < nitems; i += 3) {
        load(b2, i + 2);
        step(b0, i);
        if (i + 1 >= nitems) break;
        load(b0, i + 3);
        step(b1, i + 1);
        if (i + 2 >= nitems) break;
        load(b1, i + 4);
        step(b2, i + 2);
    }
}

int compute_units() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cus[dev] = v;
    }
    return cus[dev];
}

// LDS a workgroup may use on the current device (160 KB on gfx950).
size_t max_lds_per_block() {
    static size_t lds[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64 * 1024;
    if (lds[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            v = 64 * 1024;
        lds[dev] = static_cast<size_t>(v < GV_SPLIT_MAX_LDS ? v : GV_SPLIT_MAX_LDS);
    }
    return lds[dev];
}

// Dynamic LDS of the split kernel for (M, K).
size_t split_lds_bytes(int M, int K, int G) {
    const size_t kr = static_cast<size_t>((K + 127) / 128) * 128;
    const size_t mr = static_cast<size_t>((M + 3) & ~3);
    return static_cast<size_t>(M) * kr * 2 + (kr / G) * mr * 4 + 2 * GV_SPLIT_WAVES * mr * 16 * 4;
}

template <int G, int S>
hipError_t launch_split_s(const uint16_t *x, int M, const uint8_t *codes,
                          const uint16_t *scales, const uint16_t *zeros,
                          const uint16_t *bias, int N, int K, uint16_t *y,
                          hipStream_t stream) {
    auto kern = gemv_split_kernel<G, S>;
    static bool attr_set[64] = {false};         // per device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev < 0 || dev >= 64 || !attr_set[dev]) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(max_lds_per_block()));
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) attr_set[dev] = true;
    }
    const size_t lds = split_lds_bytes(M, K, G);
    // resident blocks per compute unit: LDS (160 KB) and 2 blocks of 8 waves
    int per_cu = static_cast<int>(static_cast<size_t>(GV_SPLIT_MAX_LDS) / lds);
    per_cu = per_cu < 1 ? 1 : (per_cu > 2 ? 2 : per_cu);
    const int ntiles = (N + 15) / 16;
    constexpr int T = GV_SPLIT_WAVES / S;
    const int nsteps = (ntiles + T - 1) / T;
    const int slots = compute_units() * per_cu;
    const int blocks = nsteps < slots ? nsteps : slots;
    kern<<<dim3(blocks), dim3(GV_SPLIT_WAVES * 64), lds, stream>>>(x, M, codes, scales, zeros,
                                                                   bias, N, K, y);
    return hipGetLastError();
}

// K split: 8 waves per tile (measured best for the decode layers: wide
// layers keep 8-way splits too, the persistent grid streams their tiles),
// fewer when K has fewer than 8 chunks.
template <int G>
hipError_t launch_split(const uint16_t *x, int M, const uint8_t *codes,
                        const uint16_t *scales, const uint16_t *zeros,
                        const uint16_t *bias, int N, int K, uint16_t *y,
                        hipStream_t stream) {
    const int nchunk = (K + 127) / 128;
    if (nchunk >= 8)
        return launch_split_s<G, 8>(x, M, codes, scales, zeros, bias, N, K, y, stream);
    if (nchunk >= 4)
        return launch_split_s<G, 4>(x, M, codes, scales, zeros, bias, N, K, y, stream);
    if (nchunk >= 2)
        return launch_split_s<G, 2>(x, M, codes, scales, zeros, bias, N, K, y, stream);
    return launch_split_s<G, 1>(x, M, codes, scales, zeros, bias, N, K, y, stream);
}

template <int G>
hipError_t launch_gemv_g(const uint16_t *x, int M, const uint8_t *codes,
                         const uint16_t *scales, const uint16_t *zeros,
                         const uint16_t *bias, int N, int K, uint16_t *y,
                         hipStream_t stream) {
    const int ntiles = (N + 15) / 16;
    if (M <= GV_SPLIT_MAX_M && split_lds_bytes(M, K, G) <= max_lds_per_block()) {
        return launch_split<G>(x, M, codes, scales, zeros, bias, N, K, y, stream);
    }
    gemv_phased_kernel<G, GV_WAVES><<<dim3(ntiles), dim3(GV_WAVES * 64), 0, stream>>>(
        x, M, codes, scales, zeros, bias, N, K, y);
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
