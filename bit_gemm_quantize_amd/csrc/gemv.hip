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

#include <atomic>

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
// Padding (bf16 elements) after each staged x row: an A-fragment read has
// 16 lanes on 16 rows at one column; with rows 16 bytes apart modulo the
// 256-byte bank period they fall in different banks instead of one.
constexpr int GV_X_PAD = 8;
constexpr int GV_SPLIT_MAX_M = 16;      // split-K kernel: M <= 16 ...
constexpr int GV_SPLIT_WAVES = 8;       // split-K kernel: waves per block
constexpr int GV_SPLIT_MAX_LDS = 160 * 1024;   // ... when its LDS fits one CU

// Codes of U consecutive chunks of one lane, plus the scales and zero-points
// of the batch's U * 128 / G groups for the wave's 16 rows, loaded with
// consecutive lanes on consecutive groups of a row: register r, lane l holds
// (s | z << 16) of row l / 4, group 4r + l % 4 of the batch.
template <int G, int U>
struct Batch {
    static constexpr int GPB = U * 128 / G;     // groups per batch (2, 4 or 8)
    static constexpr int R = (GPB + 3) / 4;     // (GPB = 2: lanes l % 4 >= 2 unused)
    u32x4 q[U];
    uint32_t s[R];
    uint32_t z[R];
};

// Issue the loads of one batch: scales/zeros first (needed at the first
// group end), then the codes. All addresses are clamped, never predicated.
template <int G, int U, bool PK>
__device__ __forceinline__ void load_batch(Batch<G, U> &b, const uint8_t *crow,
                                           const uint16_t *__restrict__ scales,
                                           const uint16_t *__restrict__ zeros,
                                           const uint32_t *__restrict__ sz,
                                           int row0, int N, int K, int ngroups,
                                           int c, int c_last, int lane) {
    constexpr int GPC = 128 / G;
    const int kb = lane >> 4;
    const int srow = min(row0 + (lane >> 2), N - 1);
#pragma unroll
    for (int r = 0; r < Batch<G, U>::R; ++r) {
        const int g = min(c * GPC + 4 * r + (lane & 3), ngroups - 1);
        const int64_t i = static_cast<int64_t>(srow) * ngroups + g;
        if constexpr (PK) {                     // one (s | z << 16) word
            b.s[r] = sz[i];
            b.z[r] = b.s[r] >> 16;
        } else {
            b.s[r] = scales[i];
            b.z[r] = zeros[i];
        }
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
template <int G, int U, bool PK>
__device__ __forceinline__ void load_batch_buf(Batch<G, U> &b, __amdgpu_buffer_rsrc_t crs,
                                               __amdgpu_buffer_rsrc_t srs,
                                               __amdgpu_buffer_rsrc_t zrs, int cvo, int svo,
                                               int c, int c_last) {
    constexpr int GPC = 128 / G;
    constexpr int OOB = 0x40000000;             // past any resource: reads 0, no traffic
#pragma unroll
    for (int r = 0; r < Batch<G, U>::R; ++r) {
        const int so = (c * GPC + 4 * r) * 2;
        if constexpr (PK) {                     // srs covers the (s | z << 16) words
            b.s[r] = __builtin_amdgcn_raw_buffer_load_b32(srs, 2 * svo, 2 * so, 0);
            b.z[r] = b.s[r] >> 16;
        } else {
            b.s[r] = __builtin_amdgcn_raw_buffer_load_b16(srs, svo, so, 0);
            b.z[r] = __builtin_amdgcn_raw_buffer_load_b16(zrs, svo, so, 0);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // chunks past this wave's segment are never computed: not fetched
        const int so = c + u <= c_last ? (c + u) * 64 : OOB;
        b.q[u] = __builtin_amdgcn_raw_buffer_load_b128(crs, cvo, so, W4_CPOL_STREAM);
    }
}

template <int G, int NW, bool PK>
__global__ __launch_bounds__(NW * 64, 2) void gemv_phased_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint32_t *__restrict__ sz, const uint16_t *__restrict__ bias, int N, int K,
    uint16_t *__restrict__ y) {
    constexpr int SPG = G / 32;                 // slots per group: 4, 2 or 1
    constexpr int GPC = 128 / G;                // groups per chunk: 1, 2 or 4
    constexpr int U = G == 32 ? 2 : 4;          // chunks per batch
    __shared__ __attribute__((aligned(16))) uint16_t xl[GV_X_ELEMS + 16 * GV_X_PAD];
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
    const int kps = kp + GV_X_PAD;              // LDS row stride

    // Loads are unconditional (clamped addresses), so the compiler can count
    // the loads in flight and wait only for the batch being computed.
    auto load = [&](Batch<G, U> &b, int c, int c_last) {
        load_batch<G, U, PK>(b, crow, scales, zeros, sz, n_base, N, K, ngroups, c, c_last, lane);
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
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(&xl[mrow * kps + ka]));
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
                // pre-shuffled codes expand in natural k order: x stays as is
                *reinterpret_cast<u32x4 *>(&xl[m * kps + kk]) = PK ? xv[j] : interleave8_bf16(xv[j]);
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
// is staged in LDS (zero padded to whole chunks) together with the
// per-group sums xs[g][m] = sum_{k in g} x[m][k]; each wave stages the K
// segment it reads. Two staging forms:
//   NAT = false (small M): through registers, 8 values per 16 bytes put in
//     the interleaved order of the 7-op code expansion, group sums from the
//     loaded values, rows padded by 16 bytes against bank conflicts;
//   NAT = true (larger M, where that staging costs more than it saves):
//     global -> LDS copies with no register round trip, natural order (9-op
//     expansion), 16-byte pieces of row m stored at piece ^ (m % 16) inside
//     each 256-byte chunk so that the 16 rows of a fragment read fall in
//     different banks, group sums by matrix-core products with ones.
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
template <int G, int S, bool NAT, bool PK>
__global__ __launch_bounds__(GV_SPLIT_WAVES * 64, 2) void gemv_split_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint32_t *__restrict__ sz, const uint16_t *__restrict__ bias, int N, int K,
    uint16_t *__restrict__ y) {
    constexpr int NW = GV_SPLIT_WAVES;
    constexpr int T = NW / S;                   // tiles per block step
    constexpr int SPG = G / 32;
    constexpr int GPC = 128 / G;
    constexpr int U = G == 32 ? 2 : 4;
    constexpr int LPG = G / 8;                  // staging lanes per group
    constexpr int R = Batch<G, U>::R;
    constexpr int MR = GV_SPLIT_MAX_M;          // rows of xs and red
    // dynamic LDS: x [M][kr + pad] bf16 | xs [kr/G][MR] f32 | red [2][NW][MR][16] f32
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
    const int nl = lane & 15;
    const int kb = lane >> 4;
    const int ts = wave / S, sg = wave % S;
    const int nchunk = (K + 127) >> 7;
    const int kr = nchunk * 128;                // x row length (zero padded)
    const int krs = NAT ? kr : kr + GV_X_PAD;   // LDS row stride
    uint16_t *xl = reinterpret_cast<uint16_t *>(smem);
    float *xs = reinterpret_cast<float *>(smem + static_cast<size_t>(M) * krs * 2);
    float *red = xs + static_cast<size_t>(kr / G) * MR;
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

    // Per-lane operand addresses; a chunk adds a wave-uniform offset and a
    // slot j a constant one. slot_koff(j, kb) - slot_koff(0, kb) does not
    // depend on kb.
    const uint16_t *xa = &xl[mrow * krs + slot_koff<G>(0, kb)];
    // NAT: byte offset of the lane's fragment j in chunk 0 (swizzled piece)
    uint32_t xo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        xo[j] = (mrow * krs + ((slot_koff<G>(j, kb) >> 3) ^ (mrow & 15)) * 8) * 2;
    const float *xsa = xs + 4 * kq;
    const int cvo = nl * (K >> 1) + kb * 16;                  // code byte offset
    const int svo = ((lane >> 2) * ngroups + (lane & 3)) * 2;  // s / z byte offset

    // Items are loaded and computed in order: (block step st, batch bi).
    // Items past the end (issued by the fixed-depth pipeline) and tiles past
    // N get an empty resource: their loads return 0 without touching memory.
    int ld_st = 0, ld_bi = 0;
    auto load_next = [&](Batch<G, U> &b, uint32_t &bv) {
        const int tl = (static_cast<int>(blockIdx.x) + ld_st * static_cast<int>(gridDim.x)) * T + ts;
        const int rows = (ld_st < my_steps && tl < ntiles) ? min(16, N - tl * 16) : 0;
        const int64_t row0 = static_cast<int64_t>(min(tl, ntiles - 1)) * 16;
        const int c = cb + ld_bi * U;
        const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(codes + row0 * (K >> 1)), 0, rows * (K >> 1), 0x00020000);
        const __amdgpu_buffer_rsrc_t srs =
            PK ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(sz + row0 * ngroups), 0,
                                                   rows * ngroups * 4, 0x00020000)
               : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(scales + row0 * ngroups),
                                                   0, rows * ngroups * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t zrs =
            PK ? srs
               : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(zeros + row0 * ngroups),
                                                   0, rows * ngroups * 2, 0x00020000);
        load_batch_buf<G, U, PK>(b, crs, srs, zrs, cvo, svo, c, c_last);
        // bias of column nl (0 without bias: empty resource)
        const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(bias ? bias + row0 : bias), 0, bias ? rows * 2 : 0, 0x00020000);
        bv = __builtin_amdgcn_raw_buffer_load_b16(brs, nl * 2, 0, 0);
        if (++ld_bi == nb) { ld_bi = 0; ++ld_st; }
    };

    // x staging, per wave: a wave stages only the K segment it reads (rows
    // 0..M-1, whole chunks), so no block barrier is needed before the first
    // step; waves that share a segment (T > 1) write identical values. The
    // segment is cut in runs of 64 pieces of 16 bytes (one per lane) along
    // each row; the first XR runs are issued ahead of the codes of the first
    // two items, so the wait for x leaves the codes in flight.
    Batch<G, U> b0, b1, b2;
    uint32_t bv0, bv1, bv2;
    if constexpr (NAT) {
        // one copy per run of 64 pieces along a row; lane l of the run fills
        // piece position l, i.e. fetches piece l ^ (m % 16) of the run
        const int seg_pr = (ce - cb) * 16;      // pieces per row of the segment
        const int rpr = (seg_pr + 63) >> 6;     // runs per row
        const int k0 = cb * 128;
        const uint32_t xl0 = lds_address(smem);
        for (int m = 0; m < M; ++m) {
            const uint16_t *xrow = x + static_cast<int64_t>(m) * K;
            for (int q = 0; q < rpr; ++q) {
                // pieces past K (last chunk) are not copied but cleared below
                const int kk = k0 + (q * 64 + (lane ^ (m & 15))) * 8;
                if (q * 64 + lane < seg_pr && kk < K)
                    lds_dma16(xrow + kk, xl0 + (m * krs + k0) * 2 + q * 1024);
            }
        }
        load_next(b0, bv0);
        load_next(b1, bv1);
        // the copies are older than the loads of b0 and b1: per item R scale /
        // zero-point words (pre-shuffled) or 2R halves, U code pieces, 1 bias
        constexpr int LPI = (PK ? R : 2 * R) + U + 1;
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"(2 * LPI) : "memory");
        if ((K & 127) != 0 && ce == nchunk && ce > cb) {
            // zero the pieces of the last chunk that lie past K
            const int p = lane & 15;            // logical piece in the chunk
            if ((nchunk - 1) * 128 + p * 8 >= K) {
                for (int m = lane >> 4; m < M; m += 4)
                    *reinterpret_cast<u32x4 *>(
                        &xl[m * krs + (nchunk - 1) * 128 + ((p ^ (m & 15)) * 8)]) =
                        u32x4{0u, 0u, 0u, 0u};
            }
        }
        // group sums of the segment: fragments against ones; lane (nl, kb)
        // receives rows 4 kb .. 4 kb + 3 (all columns equal)
        const bf16x8 ones = bf16x8_ones();
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        for (int cc = cb; cc < ce; ++cc) {
            f32x4 sg4 = z4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(
                    reinterpret_cast<const uint8_t *>(xl) + xo[j] + cc * 256);
                sg4 = mfma16x16x32(as_bf16x8(a), ones, (j % SPG) == 0 ? z4 : sg4);
                if ((j % SPG) == SPG - 1 && nl == 0)
                    *reinterpret_cast<f32x4 *>(&xs[(cc * GPC + j / SPG) * MR + 4 * kb]) = sg4;
            }
        }
        __builtin_amdgcn_wave_barrier();
    } else {
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
                if (ok) *reinterpret_cast<u32x4 *>(&xl[m * krs + kk]) = PK ? v : interleave8_bf16(v);
                float sum = (bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y)) +
                            (bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w));
                // a group's LPG pieces sit in consecutive lanes of one run
                // (LPG divides 16, runs start at multiples of 512 k), so
                // they reduce with DPP moves
                sum = group_sum<LPG>(sum);
                if (ok && (lane & (LPG - 1)) == 0) xs[(kk / G) * MR + m] = sum;
                if (++q == rpr) { q = 0; ++m; }
            }
        };
        issue(0);
        load_next(b0, bv0);
        load_next(b1, bv1);
        put(0);
        for (int r0 = XR; r0 < nruns; r0 += XR) {
            issue(r0);
            put(r0);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // the outputs of a block step this thread sums (S > 1): T * M * 16 of
    // them over the block, at most RI per thread
    constexpr int RI = (T * MR * 16 + NW * 64 - 1) / (NW * 64);
    bool red_live[RI];
    int red_slot[RI], red_m[RI], red_nn[RI];
#pragma unroll
    for (int it = 0; it < RI; ++it) {
        const int e = static_cast<int>(threadIdx.x) + it * NW * 64;
        red_live[it] = e < T * M * 16;
        red_slot[it] = e / (M * 16);
        const int rem = e - red_slot[it] * (M * 16);
        red_m[it] = rem >> 4;
        red_nn[it] = rem & 15;
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    int sp_st = 0, sp_bi = 0;
    auto step = [&](Batch<G, U> &b, uint32_t bvr) {
        const int st = sp_st, bi = sp_bi;
        if (++sp_bi == nb) { sp_bi = 0; ++sp_st; }
        const int c = cb + bi * U;
        // scales and zero-points of the batch as float: s and z - 128 s
        float svr[R], zzr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            svr[r] = __uint_as_float(b.s[r] << 16);
            zzr[r] = fmaf(-128.0f, svr[r], __uint_as_float(b.z[r] << 16));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = c + u;
            if (cc >= ce) break;                // uniform across the wave
            align_groups<G>(b.q[u]);
            // the chunk's LDS reads first: x fragments, group sums, and the
            // scale / zero-point of column nl for each group
            const uint16_t *xc = xa + cc * 128;
            const float *xsc = xsa + cc * GPC * MR;
            u32x4 av[4];
            f32x4 xg[GPC];
            float sg_[GPC], zg[GPC];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (NAT)
                    av[j] = *reinterpret_cast<const u32x4 *>(
                        reinterpret_cast<const uint8_t *>(xl) + xo[j] + cc * 256);
                else
                    av[j] = *reinterpret_cast<const u32x4 *>(xc + slot_koff<G>(j, 0) -
                                                             slot_koff<G>(0, 0));
            }
#pragma unroll
            for (int g = 0; g < GPC; ++g) {
                const int h = u * GPC + g;      // group of the batch
                xg[g] = *reinterpret_cast<const f32x4 *>(xsc + g * MR);
                const int src = (nl * 4 + (h & 3)) * 4;
                sg_[g] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                       src, __builtin_bit_cast(int, svr[h >> 2])));
                zg[g] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                      src, __builtin_bit_cast(int, zzr[h >> 2])));
            }
            f32x4 accg = zero4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool first = (j % SPG) == 0;
                uint32_t w[4];
                if constexpr (NAT && !PK)
                    unpack8_bias128(b.q[u][j], w, uc);
                else                            // interleaved x, or pre-shuffled codes
                    unpack8_bias128_il(b.q[u][j], w, uc);
                accg = mfma16x16x32(as_bf16x8(av[j]), as_bf16x8(w[0], w[1], w[2], w[3]),
                                    first ? zero4 : accg);
                if ((j % SPG) == SPG - 1) {
                    const int g = j / SPG;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[i] = fmaf(sg_[g], accg[i], fmaf(zg[g], xg[g][i], acc[i]));
                }
            }
        }
        if (bi != nb - 1) return;               // end of this block step
        // bias of column nl, added once per tile (by the waves of K segment 0)
        if (sg == 0) {
            const float bvf = bf16_to_f32(static_cast<uint16_t>(bvr));
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += bvf;
        }
        if constexpr (S == 1) {
            const int col = ((static_cast<int>(blockIdx.x) + st * static_cast<int>(gridDim.x)) * T + ts) * 16 + nl;
            if (col < N) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * kb + i < M)
                        y[static_cast<int64_t>(4 * kb + i) * N + col] =
                            static_cast<uint16_t>(f32_to_bf16_rne(acc[i]));
            }
            acc = zero4;
        } else {
            const int par = st & 1;
            float *rw = red + (par * NW + wave) * MR * 16;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * kb + i < M) rw[(4 * kb + i) * 16 + nl] = acc[i];
            acc = zero4;
            __syncthreads();
            const int tile0 = (static_cast<int>(blockIdx.x) + st * static_cast<int>(gridDim.x)) * T;
#pragma unroll
            for (int it = 0; it < RI; ++it) {
                if (!red_live[it]) continue;
                const int slot = red_slot[it], m = red_m[it], nn = red_nn[it];
                const float *rp = red + ((par * NW + slot * S) * MR + m) * 16 + nn;
                float sum = 0.f;
#pragma unroll
                for (int w = 0; w < S; ++w) sum += rp[w * MR * 16];
                const int col = (tile0 + slot) * 16 + nn;
                if (col < N)
                    y[static_cast<int64_t>(m) * N + col] =
                        static_cast<uint16_t>(f32_to_bf16_rne(sum));
            }
        }
    };

    const int nitems = my_steps * nb;
    for (int i = 0; i < nitems; i += 3) {
        load_next(b2, bv2);
        step(b0, bv0);
        if (i + 1 >= nitems) break;
        load_next(b0, bv0);
        step(b1, bv1);
        if (i + 2 >= nitems) break;
        load_next(b1, bv1);
        step(b2, bv2);
    }
}

// Persistent split-K kernel for 1 <= M <= 16 whose x fragments come from
// global memory (L2) instead of LDS: used when x does not fit in LDS. Same
// (tile, K segment) decomposition and cross-wave reduction as the split
// kernel; items are 2 chunks; K is a multiple of 128 (no partial chunk
// whose x would have to read 0 past K). The codes of the next two items and the x
// fragments of the next one are in flight while an item is computed; loads
// complete in issue order, so the order codes(t), x(t), codes(t+1), ...
// lets the wait for x(t) leave codes(t + 1), codes(t + 2) in flight. Group
// sums come from the matrix cores (fragments against ones); x and the codes
// are expanded in natural order.
template <int G, int S, bool PK>
__global__ __launch_bounds__(GV_SPLIT_WAVES * 64, 2) void gemv_direct_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint32_t *__restrict__ sz, const uint16_t *__restrict__ bias, int N, int K,
    uint16_t *__restrict__ y) {
    constexpr int NW = GV_SPLIT_WAVES;
    constexpr int T = NW / S;                   // tiles per block step
    constexpr int SPG = G / 32;
    constexpr int GPC = 128 / G;
    constexpr int U = 2;
    constexpr int R = Batch<G, U>::R;
    constexpr int MR = GV_SPLIT_MAX_M;
    constexpr int OOB = 0x40000000;
    __shared__ __attribute__((aligned(16))) float red[2][NW][MR][16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
    const int nl = lane & 15;
    const int kb = lane >> 4;
    const int ts = wave / S, sg = wave % S;
    const int nchunk = (K + 127) >> 7;
    const int ngroups = K / G;
    const int ntiles = (N + 15) >> 4;
    const int nsteps = (ntiles + T - 1) / T;
    const int my_steps = (nsteps - static_cast<int>(blockIdx.x) + gridDim.x - 1) / gridDim.x;
    const int mrow = nl < M ? nl : M - 1;
    const Unpack128 uc = unpack128_consts();
    const bf16x8 ones = bf16x8_ones();

    const int cb = sg * nchunk / S;
    const int ce = (sg + 1) * nchunk / S;
    const int c_last = max(cb, ce - 1);
    const int nb = ((nchunk + S - 1) / S + U - 1) / U;

    const int cvo = nl * (K >> 1) + kb * 16;
    const int svo = ((lane >> 2) * ngroups + (lane & 3)) * 2;
    const int xvo = (mrow * K + slot_koff<G>(0, kb)) * 2;     // x byte offset
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x), 0, M * K * 2, 0x00020000);

    int ld_st = 0, ld_bi = 0;                   // next item whose codes load
    auto load_codes = [&](Batch<G, U> &b, uint32_t &bv) {
        const int tl = (static_cast<int>(blockIdx.x) + ld_st * static_cast<int>(gridDim.x)) * T + ts;
        const int rows = (ld_st < my_steps && tl < ntiles) ? min(16, N - tl * 16) : 0;
        const int64_t row0 = static_cast<int64_t>(min(tl, ntiles - 1)) * 16;
        const int c = cb + ld_bi * U;
        const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(codes + row0 * (K >> 1)), 0, rows * (K >> 1), 0x00020000);
        const __amdgpu_buffer_rsrc_t srs =
            PK ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(sz + row0 * ngroups), 0,
                                                   rows * ngroups * 4, 0x00020000)
               : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(scales + row0 * ngroups),
                                                   0, rows * ngroups * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t zrs =
            PK ? srs
               : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(zeros + row0 * ngroups),
                                                   0, rows * ngroups * 2, 0x00020000);
        load_batch_buf<G, U, PK>(b, crs, srs, zrs, cvo, svo, c, c_last);
        const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(bias ? bias + row0 : bias), 0, bias ? rows * 2 : 0, 0x00020000);
        bv = __builtin_amdgcn_raw_buffer_load_b16(brs, nl * 2, 0, 0);
        if (++ld_bi == nb) { ld_bi = 0; ++ld_st; }
    };
    int xl_st = 0, xl_bi = 0;                   // next item whose x loads
    auto load_x = [&](u32x4 (&a)[U][4]) {
        const bool live = xl_st < my_steps;
        const int c = cb + xl_bi * U;
        if (++xl_bi == nb) { xl_bi = 0; ++xl_st; }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = c + u;
            // chunks outside the segment (or items past the end): nothing
            const int so = (live && cc < ce) ? cc * 256 : OOB;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                a[u][j] = __builtin_amdgcn_raw_buffer_load_b128(
                    xrs, xvo, so + (slot_koff<G>(j, 0) - slot_koff<G>(0, 0)) * 2, 0);
        }
    };

    // the outputs of a block step this thread sums (S > 1): T * M * 16 of
    // them over the block, at most RI per thread
    constexpr int RI = (T * MR * 16 + NW * 64 - 1) / (NW * 64);
    bool red_live[RI];
    int red_slot[RI], red_m[RI], red_nn[RI];
#pragma unroll
    for (int it = 0; it < RI; ++it) {
        const int e = static_cast<int>(threadIdx.x) + it * NW * 64;
        red_live[it] = e < T * M * 16;
        red_slot[it] = e / (M * 16);
        const int rem = e - red_slot[it] * (M * 16);
        red_m[it] = rem >> 4;
        red_nn[it] = rem & 15;
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    int sp_st = 0, sp_bi = 0;
    auto step = [&](Batch<G, U> &b, uint32_t bvr, u32x4 (&a)[U][4]) {
        const int st = sp_st, bi = sp_bi;
        if (++sp_bi == nb) { sp_bi = 0; ++sp_st; }
        const int c = cb + bi * U;
        float svr[R], zzr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            svr[r] = __uint_as_float(b.s[r] << 16);
            zzr[r] = fmaf(-128.0f, svr[r], __uint_as_float(b.z[r] << 16));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int cc = c + u;
            if (cc >= ce) break;                // uniform across the wave
            align_groups<G>(b.q[u]);
            float sg_[GPC], zg[GPC];
#pragma unroll
            for (int g = 0; g < GPC; ++g) {
                const int h = u * GPC + g;
                const int src = (nl * 4 + (h & 3)) * 4;
                sg_[g] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                       src, __builtin_bit_cast(int, svr[h >> 2])));
                zg[g] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                      src, __builtin_bit_cast(int, zzr[h >> 2])));
            }
            f32x4 accg = zero4, xsg = zero4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool first = (j % SPG) == 0;
                uint32_t w[4];
                if constexpr (PK)
                    unpack8_bias128_il(b.q[u][j], w, uc);   // natural k order
                else
                    unpack8_bias128(b.q[u][j], w, uc);
                xsg = mfma16x16x32(as_bf16x8(a[u][j]), ones, first ? zero4 : xsg);
                accg = mfma16x16x32(as_bf16x8(a[u][j]), as_bf16x8(w[0], w[1], w[2], w[3]),
                                    first ? zero4 : accg);
                if ((j % SPG) == SPG - 1) {
                    const int g = j / SPG;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[i] = fmaf(sg_[g], accg[i], fmaf(zg[g], xsg[i], acc[i]));
                }
            }
        }
        if (bi != nb - 1) return;               // end of this block step
        if (sg == 0) {
            const float bvf = bf16_to_f32(static_cast<uint16_t>(bvr));
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += bvf;
        }
        if constexpr (S == 1) {
            const int col = ((static_cast<int>(blockIdx.x) + st * static_cast<int>(gridDim.x)) * T + ts) * 16 + nl;
            if (col < N) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * kb + i < M)
                        y[static_cast<int64_t>(4 * kb + i) * N + col] =
                            static_cast<uint16_t>(f32_to_bf16_rne(acc[i]));
            }
            acc = zero4;
        } else {
            const int par = st & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * kb + i < M) red[par][wave][4 * kb + i][nl] = acc[i];
            acc = zero4;
            __syncthreads();
            const int tile0 = (static_cast<int>(blockIdx.x) + st * static_cast<int>(gridDim.x)) * T;
#pragma unroll
            for (int it = 0; it < RI; ++it) {
                if (!red_live[it]) continue;
                const int slot = red_slot[it], m = red_m[it], nn = red_nn[it];
                float sum = 0.f;
#pragma unroll
                for (int w = 0; w < S; ++w) sum += red[par][slot * S + w][m][nn];
                const int col = (tile0 + slot) * 16 + nn;
                if (col < N)
                    y[static_cast<int64_t>(m) * N + col] =
                        static_cast<uint16_t>(f32_to_bf16_rne(sum));
            }
        }
    };

    Batch<G, U> b0, b1, b2;
    uint32_t bv0, bv1, bv2;
    u32x4 a0[U][4], a1[U][4], a2[U][4];
    load_codes(b0, bv0);
    load_x(a0);
    load_codes(b1, bv1);
    const int nitems = my_steps * nb;
    for (int i = 0; i < nitems; i += 3) {
        load_x(a1);
        load_codes(b2, bv2);
        step(b0, bv0, a0);
        if (i + 1 >= nitems) break;
        load_x(a2);
        load_codes(b0, bv0);
        step(b1, bv1, a1);
        if (i + 2 >= nitems) break;
        load_x(a0);
        load_codes(b1, bv1);
        step(b2, bv2, a2);
    }
}


constexpr int kMaxDevices = 64;

// Lets `kern` use up to the device's LDS limit as dynamic LDS (the default
// cap is lower); set once per device and kernel.
template <typename Kern>
hipError_t allow_large_lds(Kern kern) {
    static std::atomic<unsigned long long> done{0};    // bit per device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const unsigned long long bit = (dev >= 0 && dev < kMaxDevices) ? 1ull << dev : 0;
    if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(max_lds_per_block()));
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_relaxed);
    return e;
}

// ---------------------------------------------------------- M = 1, 2
// Decode GEMV for one or two activation rows, with the products on the
// vector ALUs (bf16 pair dot products accumulated in float32). At such M
// the matrix-core layout below carries 14 or 15 padding rows and ties each
// load to 16 rows x 64 bytes; here a wave takes R consecutive output rows
// and one 2048-wide K segment, lane l covering k = 2048 s + 32 l .. +32 (16
// code bytes), so every load of a row is 1 KB contiguous and the blocks of
// a launch sweep memory in order. A block holds RG row groups x NSB segment
// waves; a wave whose row needs more than NSB segments takes every NSB-th.
//   * x: the lane's 32 values of each of the MR activation rows stay in
//     registers for all R weight rows. Loaded directly (4 x 16 bytes per lane and row), or
//     (XLDS) as four contiguous 1 KB runs per row passed through a per-wave
//     LDS slab one row at a time, which pays once the row spans several
//     segments. Plain codes expand in the interleaved order (0,4), (1,5),
//     (2,6), (3,7), so x is permuted to match; pre-shuffled codes expand in
//     natural order. Each code word is expanded once and meets all MR rows.
//   * per weight row, activation row and lane (its 32 codes lie in one
//     group), in float32:
//       v += s * sum x (128 + q) + (z - 128 s) * sum x.
//   * the R partial sums of each activation row are reduced across the wave
//     with lane swaps and DPP, then across the segment waves of the row
//     through LDS.
constexpr int GV1_MAX_WAVES = 16;         // waves per block (1024 threads)
constexpr int GV1_SEG = 2048;             // k per wave segment
// segment waves per row group: a row spanning more segments gives each wave
// every 8th (32768-wide rows: M = 1 and M = 2 13 % faster than one wave per
// segment; the Llama-3-8B decode rows span at most 7)
constexpr int GV1_SEG_WAVES = 8;

// Sum over the 64 lanes of four row partials; every lane of quarter r ends
// with row r's sum.
__device__ __forceinline__ float reduce_rows4(float v0, float v1, float v2, float v3) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
    const float u02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
    const float u13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(u02), __float_as_uint(u13), false, false);
    return group_sum<16>(__uint_as_float(c[0]) + __uint_as_float(c[1]));
}

template <int G, int R, bool XLDS, bool PK, int MR>
__global__ __launch_bounds__(GV1_MAX_WAVES * 64) void gemv1_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint32_t *__restrict__ sz, const uint16_t *__restrict__ bias, int N, int K,
    uint16_t *__restrict__ y, int nseg, int nsb, int rg) {
    static_assert(R % 4 == 0, "rows per wave");
    static_assert(MR == 1 || MR == 2, "activation rows");
    constexpr int GPS = GV1_SEG / G;          // groups per segment: 16, 32, 64
    constexpr int P = R * GPS / 64;           // scale / zero-point values per lane
    // dynamic LDS: partial row sums [waves][R][MR] f32, then (XLDS) 4 KB per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t g1_smem[];
    float *red = reinterpret_cast<float *>(g1_smem);
    uint8_t *g1_slab = g1_smem + GV1_MAX_WAVES * R * MR * 4;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sw = wave % nsb, rgi = wave / nsb;
    const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * rg + rgi) * R;
    const uint32_t rows = static_cast<uint32_t>(max<int64_t>(0, min<int64_t>(R, N - row0)));
    const uint32_t ngroups = static_cast<uint32_t>(K / G);
    const uint32_t kh = static_cast<uint32_t>(K) >> 1;
    constexpr uint32_t OOB = 0x80000000u;   // past every resource: reads 0
    const __amdgpu_buffer_rsrc_t crs = buf_rsrc(codes + row0 * kh, rows * kh);
    const __amdgpu_buffer_rsrc_t srs =
        PK ? buf_rsrc(sz + row0 * ngroups, rows * ngroups * 4)
           : buf_rsrc(scales + row0 * ngroups, rows * ngroups * 2);
    const __amdgpu_buffer_rsrc_t zrs = PK ? srs : buf_rsrc(zeros + row0 * ngroups, rows * ngroups * 2);
    // one resource per activation row
    __amdgpu_buffer_rsrc_t xrs[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m)
        xrs[m] = buf_rsrc(x + static_cast<int64_t>(m) * K, static_cast<uint32_t>(K) * 2);
    const uint32_t ones = 0x3F803F80u;      // bf16 pair (1, 1)
    const Unpack128 uc = unpack128_consts();

    float v[R][MR];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) v[r][m] = 0.f;

    for (int seg = sw; seg < nseg; seg += nsb) {
        const uint32_t k0 = static_cast<uint32_t>(seg) * GV1_SEG + 32u * lane;
        const bool ok = k0 < static_cast<uint32_t>(K);
        // x first (needed first), then scales / zero-points, then the codes
        u32x4 xv[MR][4];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            if constexpr (XLDS) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {   // piece p = lane + 64 i of the segment (8 k)
                    const uint32_t kx = static_cast<uint32_t>(seg) * GV1_SEG + 8u * (lane + 64 * i);
                    xv[m][i] = __builtin_amdgcn_raw_buffer_load_b128(
                        xrs[m], kx < static_cast<uint32_t>(K) ? kx * 2 : OOB, 0, 0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xv[m][i] = __builtin_amdgcn_raw_buffer_load_b128(xrs[m], ok ? (k0 + 8 * i) * 2 : OOB,
                                                                     0, 0);
            }
        }
        // (issued before the codes: loads complete in order, so each row can
        // be finished as soon as its own codes arrive)
        // Scales / zero-points of the segment's GPS groups for the R rows, P
        // per lane: lane l holds value e = l + 64 p, i.e. row e / GPS, group
        // e % GPS. Row r's value for this lane's group is then in register
        // p = r GPS / 64 of lane (r GPS + group) % 64 (fetched below with a
        // lane permute): 2P (plain) or P (pre-shuffled) loads per wave instead
        // of 2R or R.
        uint32_t sreg[P], zreg[P];
#pragma unroll
        for (int pp = 0; pp < P; ++pp) {
            const uint32_t e = static_cast<uint32_t>(lane) + 64u * pp;
            const uint32_t gs = static_cast<uint32_t>(seg) * GPS + e % GPS;   // group in the row
            const uint32_t vo = (e / GPS) * ngroups + gs;
            if constexpr (PK) {
                sreg[pp] = __builtin_amdgcn_raw_buffer_load_b32(srs, gs < ngroups ? vo * 4 : OOB, 0, 0);
                zreg[pp] = 0;
            } else {
                const uint32_t so = gs < ngroups ? vo * 2 : OOB;
                sreg[pp] = __builtin_amdgcn_raw_buffer_load_b16(srs, so, 0, 0);
                zreg[pp] = __builtin_amdgcn_raw_buffer_load_b16(zrs, so, 0, 0);
            }
        }
        u32x4 q[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            q[r] = __builtin_amdgcn_raw_buffer_load_b128(crs, ok ? (k0 >> 1) + r * kh : OOB, 0,
                                                         W4_CPOL_STREAM);
        if constexpr (XLDS) {
            // piece p -> slot 4 (p / 4) + ((p % 4) ^ ((p / 16) % 4)): the four
            // reads below (lane l: pieces 4 l .. 4 l + 3) are conflict-free.
            // One activation row at a time through the same slab (a wave's
            // LDS operations complete in issue order).
            u32x4 *slab = reinterpret_cast<u32x4 *>(g1_slab) + wave * 256;
#pragma unroll
            for (int m = 0; m < MR; ++m) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int p = lane + 64 * i;
                    slab[4 * (p >> 2) + ((p & 3) ^ ((p >> 4) & 3))] =
                        PK ? xv[m][i] : interleave8_bf16(xv[m][i]);
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[m][i] = slab[4 * lane + (i ^ ((lane >> 2) & 3))];
                __builtin_amdgcn_wave_barrier();
            }
        } else if constexpr (!PK) {
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[m][i] = interleave8_bf16(xv[m][i]);
        }
        float xs[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            xs[m] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xs[m] = dot2_bf16(xv[m][i].x, ones, xs[m]);
                xs[m] = dot2_bf16(xv[m][i].y, ones, xs[m]);
                xs[m] = dot2_bf16(xv[m][i].z, ones, xs[m]);
                xs[m] = dot2_bf16(xv[m][i].w, ones, xs[m]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float p0[MR], p1[MR];
#pragma unroll
            for (int m = 0; m < MR; ++m) p0[m] = p1[m] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t w[4];
                unpack8_bias128_il(q[r][i], w, uc);   // pairs (q0,q4).. plain, (q0,q1).. pre-shuffled
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    p0[m] = dot2_bf16(xv[m][i].x, w[0], p0[m]);
                    p1[m] = dot2_bf16(xv[m][i].y, w[1], p1[m]);
                    p0[m] = dot2_bf16(xv[m][i].z, w[2], p0[m]);
                    p1[m] = dot2_bf16(xv[m][i].w, w[3], p1[m]);
                }
            }
            // this lane's group: lane / (G / 32); source lane of row r's value
            const int src = ((r * GPS) % 64 + lane / (G / 32)) * 4;
            float s, z;
            if constexpr (PK) {
                const uint32_t w = static_cast<uint32_t>(
                    __builtin_amdgcn_ds_bpermute(src, static_cast<int>(sreg[(r * GPS) / 64])));
                s = bf16_lo(w);
                z = bf16_hi(w);
            } else {
                s = bf16_to_f32(static_cast<uint16_t>(
                    __builtin_amdgcn_ds_bpermute(src, static_cast<int>(sreg[(r * GPS) / 64]))));
                z = bf16_to_f32(static_cast<uint16_t>(
                    __builtin_amdgcn_ds_bpermute(src, static_cast<int>(zreg[(r * GPS) / 64]))));
            }
            const float zz = fmaf(-128.0f, s, z);
#pragma unroll
            for (int m = 0; m < MR; ++m) v[r][m] = fmaf(s, p0[m] + p1[m], fmaf(zz, xs[m], v[r][m]));
        }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int r = 0; r < R; r += 4) {
            const float t = reduce_rows4(v[r][m], v[r + 1][m], v[r + 2][m], v[r + 3][m]);
            if ((lane & 15) == 0) red[(wave * R + r + (lane >> 4)) * MR + m] = t;
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

// M <= GV1_MAX_M: four rows per wave; x loaded directly while a row spans at
// most two segments (K <= 4096), through LDS beyond (measured on the
// Llama-3-8B decode shapes and the 32768-square layer; eight rows per wave
// were slower at M = 1). At M = 2 the kernel beats the matrix-core split
// kernel on every decode layer (4-28 %); four activation rows per lane
// (M = 3, 4) made it vector-bound and slower on the wide layers, so those
// stay on the split kernel.
constexpr int GV1_MAX_M = 2;

template <int G, bool PK, int MR>
hipError_t launch_gemv1_mr(const uint16_t *x, const uint8_t *codes, const uint16_t *scales,
                           const uint16_t *zeros, const uint32_t *sz, const uint16_t *bias,
                           int N, int K, uint16_t *y, hipStream_t stream) {
    const int nseg = (K + GV1_SEG - 1) / GV1_SEG;
    const int nsb = nseg < GV1_SEG_WAVES ? nseg : GV1_SEG_WAVES;
    const int rg = nsb >= 4 ? 1 : 4 / nsb;             // about four waves per block
    const bool xlds = nseg > 2;
    constexpr int R = 4;
    const int64_t rows_per_block = static_cast<int64_t>(rg) * R;
    const unsigned blocks = static_cast<unsigned>((N + rows_per_block - 1) / rows_per_block);
    const dim3 block(static_cast<unsigned>(rg * nsb * 64));
    const size_t red_bytes = static_cast<size_t>(GV1_MAX_WAVES) * R * MR * 4;
    if (xlds) {
        const hipError_t e = allow_large_lds(gemv1_kernel<G, R, true, PK, MR>);
        if (e != hipSuccess) return e;
        gemv1_kernel<G, R, true, PK, MR><<<dim3(blocks), block,
                                           red_bytes + static_cast<size_t>(rg * nsb) * 4096, stream>>>(
            x, codes, scales, zeros, sz, bias, N, K, y, nseg, nsb, rg);
    } else {
        gemv1_kernel<G, R, false, PK, MR><<<dim3(blocks), block, red_bytes, stream>>>(
            x, codes, scales, zeros, sz, bias, N, K, y, nseg, nsb, rg);
    }
    return hipGetLastError();
}

template <int G, bool PK>
hipError_t launch_gemv1(const uint16_t *x, int M, const uint8_t *codes, const uint16_t *scales,
                        const uint16_t *zeros, const uint32_t *sz, const uint16_t *bias,
                        int N, int K, uint16_t *y, hipStream_t stream) {
    if (M == 1) return launch_gemv1_mr<G, PK, 1>(x, codes, scales, zeros, sz, bias, N, K, y, stream);
    return launch_gemv1_mr<G, PK, 2>(x, codes, scales, zeros, sz, bias, N, K, y, stream);
}

// The split kernel stages x through LDS copies (NAT) from this M on.
constexpr int GV_NAT_MIN_M = 5;

// Dynamic LDS of the split kernel for (M, K).
size_t split_lds_bytes(int M, int K, int G) {
    const size_t kr = static_cast<size_t>((K + 127) / 128) * 128;
    const size_t krs = M >= GV_NAT_MIN_M ? kr : kr + GV_X_PAD;
    return static_cast<size_t>(M) * krs * 2 + (kr / G) * GV_SPLIT_MAX_M * 4 +
           2 * GV_SPLIT_WAVES * GV_SPLIT_MAX_M * 16 * 4;
}

template <int G, int S, bool NAT, bool PK>
hipError_t launch_split_s(const uint16_t *x, int M, const uint8_t *codes,
                          const uint16_t *scales, const uint16_t *zeros, const uint32_t *sz,
                          const uint16_t *bias, int N, int K, uint16_t *y,
                          hipStream_t stream) {
    auto kern = gemv_split_kernel<G, S, NAT, PK>;
    const hipError_t e = allow_large_lds(kern);
    if (e != hipSuccess) return e;
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
                                                                   sz, bias, N, K, y);
    return hipGetLastError();
}

// K split: 8 waves per tile (measured best for the decode layers: wide
// layers keep 8-way splits too, the persistent grid streams their tiles),
// fewer when K has fewer than 8 chunks.
template <int G, bool PK>
hipError_t launch_split(const uint16_t *x, int M, const uint8_t *codes,
                        const uint16_t *scales, const uint16_t *zeros, const uint32_t *sz,
                        const uint16_t *bias, int N, int K, uint16_t *y,
                        hipStream_t stream) {
    const int nchunk = (K + 127) / 128;
    if (M >= GV_NAT_MIN_M) {
        if (nchunk >= 8)
            return launch_split_s<G, 8, true, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
        if (nchunk >= 4)
            return launch_split_s<G, 4, true, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
        if (nchunk >= 2)
            return launch_split_s<G, 2, true, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
        return launch_split_s<G, 1, true, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
    }
    if (nchunk >= 8)
        return launch_split_s<G, 8, false, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
    if (nchunk >= 4)
        return launch_split_s<G, 4, false, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
    if (nchunk >= 2)
        return launch_split_s<G, 2, false, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
    return launch_split_s<G, 1, false, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
}

template <int G, int S, bool PK>
hipError_t launch_direct_s(const uint16_t *x, int M, const uint8_t *codes,
                           const uint16_t *scales, const uint16_t *zeros, const uint32_t *sz,
                           const uint16_t *bias, int N, int K, uint16_t *y,
                           hipStream_t stream) {
    const int ntiles = (N + 15) / 16;
    constexpr int T = GV_SPLIT_WAVES / S;
    const int nsteps = (ntiles + T - 1) / T;
    const int slots = compute_units();
    const int blocks = nsteps < slots ? nsteps : slots;
    gemv_direct_kernel<G, S, PK><<<dim3(blocks), dim3(GV_SPLIT_WAVES * 64), 0, stream>>>(
        x, M, codes, scales, zeros, sz, bias, N, K, y);
    return hipGetLastError();
}

template <int G, bool PK>
hipError_t launch_direct(const uint16_t *x, int M, const uint8_t *codes,
                         const uint16_t *scales, const uint16_t *zeros, const uint32_t *sz,
                         const uint16_t *bias, int N, int K, uint16_t *y,
                         hipStream_t stream) {
    const int nchunk = (K + 127) / 128;
    if (nchunk >= 8)
        return launch_direct_s<G, 8, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
    if (nchunk >= 4)
        return launch_direct_s<G, 4, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
    if (nchunk >= 2)
        return launch_direct_s<G, 2, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
    return launch_direct_s<G, 1, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
}

template <int G, bool PK>
hipError_t launch_gemv_g(const uint16_t *x, int M, const uint8_t *codes,
                         const uint16_t *scales, const uint16_t *zeros, const uint32_t *sz,
                         const uint16_t *bias, int N, int K, uint16_t *y,
                         hipStream_t stream) {
    const int ntiles = (N + 15) / 16;
    if (M <= GV1_MAX_M) return launch_gemv1<G, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
    if (M <= GV_SPLIT_MAX_M && split_lds_bytes(M, K, G) <= max_lds_per_block()) {
        return launch_split<G, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
    }
    if (M <= GV_SPLIT_MAX_M && K % 128 == 0)
        return launch_direct<G, PK>(x, M, codes, scales, zeros, sz, bias, N, K, y, stream);
    gemv_phased_kernel<G, GV_WAVES, PK><<<dim3(ntiles), dim3(GV_WAVES * 64), 0, stream>>>(
        x, M, codes, scales, zeros, sz, bias, N, K, y);
    return hipGetLastError();
}

} // namespace

// Per-device values computed on first use. Threads that race on the first
// call compute the same value; relaxed atomics keep the reads whole.
int compute_units() {
    static std::atomic<int> cus[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int v = cus[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cus[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// LDS a workgroup may use on the current device (160 KB on gfx950).
size_t max_lds_per_block() {
    static std::atomic<int> lds[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 64 * 1024;
    int v = lds[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
            v <= 0)
            v = 64 * 1024;
        v = v < GV_SPLIT_MAX_LDS ? v : GV_SPLIT_MAX_LDS;
        lds[dev].store(v, std::memory_order_relaxed);
    }
    return static_cast<size_t>(v);
}

hipError_t launch_gemv(const uint16_t *x, int M, const uint8_t *codes,
                       const uint16_t *scales, const uint16_t *zeros, const uint32_t *sz,
                       const uint16_t *bias, int64_t N, int64_t K, int G,
                       uint16_t *y, hipStream_t stream) {
    const int n = static_cast<int>(N), k = static_cast<int>(K);
    const bool pk = sz != nullptr;
#define W4_GEMV_LAUNCH(GG) \
    (pk ? launch_gemv_g<GG, true>(x, M, codes, scales, zeros, sz, bias, n, k, y, stream) \
        : launch_gemv_g<GG, false>(x, M, codes, scales, zeros, sz, bias, n, k, y, stream))
    switch (G) {
    case 32: return W4_GEMV_LAUNCH(32);
    case 64: return W4_GEMV_LAUNCH(64);
    case 128: return W4_GEMV_LAUNCH(128);
    default: return hipErrorInvalidValue;
    }
#undef W4_GEMV_LAUNCH
}

} // namespace w4
