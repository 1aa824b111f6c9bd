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
constexpr int GV_STREAM_MAX_M = 4;      // persistent kernel: M <= 4
constexpr int GV_STREAM_WAVES = 8;      // persistent kernel: waves per block
constexpr int GV_STREAM_MAX_LDS = GV_X_ELEMS * 2 + (GV_X_ELEMS / 32) * 4 * 4 +
                                  2 * GV_STREAM_WAVES * 4 * 16 * 4;

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
        for (int e = threadIdx.x; e < M * per_row; e += NW * 64) {
            const int m = e / per_row;
            const int kk = (e - m * per_row) * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (k_phase + kk < K)
                v = *reinterpret_cast<const u32x4 *>(x + static_cast<int64_t>(m) * K + k_phase + kk);
            *reinterpret_cast<u32x4 *>(&xl[m * kp + kk]) = interleave8_bf16(v);
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

// Persistent variant for M <= 4 and M * K small enough to keep x in LDS:
// one block per compute unit stages x once (interleaved, zero padded to
// whole chunks) together with the per-group sums xs[g][m] = sum_{k in g}
// x[m][k], then streams 16-row tiles blockIdx.x, blockIdx.x + gridDim.x, ...
// Each wave keeps the same run of K chunks for every tile, and the codes of
// the next (tile, batch) are in flight while the current one is computed.
// One barrier per tile combines the waves' partial sums (double-buffered).
// Only lanes 0..15 (rows 0..3 of the MFMA output) carry live outputs.
template <int G, int NW>
__global__ __launch_bounds__(NW * 64, 2) void gemv_stream_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int N, int K, uint16_t *__restrict__ y) {
    constexpr int SPG = G / 32;
    constexpr int GPC = 128 / G;
    constexpr int U = G == 32 ? 2 : 4;
    constexpr int LPG = G / 8;                  // staging lanes per group
    // dynamic LDS: x [M][kr] bf16 | xs [kr/G][4] f32 | red [2][NW][4][16] f32
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nl = lane & 15;
    const int kb = lane >> 4;
    const int nchunk = (K + 127) >> 7;
    const int kr = nchunk * 128;                // LDS row length (zero padded)
    uint16_t *xl = reinterpret_cast<uint16_t *>(smem);
    float(*xs)[GV_STREAM_MAX_M] = reinterpret_cast<float(*)[GV_STREAM_MAX_M]>(
        smem + static_cast<size_t>(M) * kr * 2);
    float(*red)[NW][GV_STREAM_MAX_M][16] = reinterpret_cast<float(*)[NW][GV_STREAM_MAX_M][16]>(
        smem + static_cast<size_t>(M) * kr * 2 + static_cast<size_t>(kr / G) * GV_STREAM_MAX_M * 4);
    const int ngroups = K / G;
    const int ntiles = (N + 15) >> 4;
    const int my_tiles = (ntiles - static_cast<int>(blockIdx.x) + gridDim.x - 1) / gridDim.x;
    const int mrow = nl < M ? nl : M - 1;
    const Unpack128 uc = unpack128_consts();

    const int cb = wave * nchunk / NW;
    const int ce = (wave + 1) * nchunk / NW;
    const int c_last = max(cb, ce - 1);
    const int nb = ((nchunk + NW - 1) / NW + U - 1) / U;
    const int nitems = my_tiles * nb;

    auto load = [&](Batch<G, U> &b, int item) {
        const int t = item / nb;
        const int c = cb + (item - t * nb) * U;
        const int tile = blockIdx.x + t * gridDim.x;
        const int n = min(tile * 16 + nl, N - 1);
        load_batch<G, U>(b, codes + static_cast<int64_t>(n) * (K >> 1), scales, zeros,
                         tile * 16, N, K, ngroups, c, c_last, lane);
    };

    // issue the first loads, then stage x and its group sums
    Batch<G, U> b0, b1;
    if (nitems > 0) load(b0, 0);
    const int per_row = kr >> 3;                // 16-byte pieces per row
    for (int e = threadIdx.x; e < M * per_row; e += NW * 64) {
        // a group's LPG pieces are consecutive lanes (M * per_row and the
        // stride are multiples of LPG), so they reduce with DPP moves
        const int m = e / per_row;
        const int kk = (e - m * per_row) * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (kk < K)
            v = *reinterpret_cast<const u32x4 *>(x + static_cast<int64_t>(m) * K + kk);
        *reinterpret_cast<u32x4 *>(&xl[m * kr + kk]) = interleave8_bf16(v);
        float sum = (bf16_lo(v.x) + bf16_hi(v.x)) + (bf16_lo(v.y) + bf16_hi(v.y)) +
                    (bf16_lo(v.z) + bf16_hi(v.z)) + (bf16_lo(v.w) + bf16_hi(v.w));
        sum = group_sum<LPG>(sum);
        if (((e & (LPG - 1)) == 0)) xs[kk / G][m] = sum;
    }
    __syncthreads();

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    auto step = [&](Batch<G, U> &b, int item) {
        const int t = item / nb;
        const int bi = item - t * nb;
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
                    const int h = u * GPC + j / SPG;
                    const uint32_t szv = batch_sz(packed, h, lane);
                    const float sv = bf16_lo(szv);
                    const float zz = fmaf(-128.0f, sv, bf16_hi(szv));
                    const f32x4 xg = *reinterpret_cast<const f32x4 *>(&xs[cc * GPC + j / SPG][0]);
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
        if (bi == nb - 1) {                     // end of tile t: combine waves
            const int par = t & 1;
            if (kb == 0) {
#pragma unroll
                for (int i = 0; i < GV_STREAM_MAX_M; ++i)
                    if (i < M) red[par][wave][i][nl] = acc[i];
            }
            acc = zero4;
            __syncthreads();
            const int tile = blockIdx.x + t * gridDim.x;
            for (int e = threadIdx.x; e < M * 16; e += NW * 64) {
                const int m = e >> 4;
                const int nn = e & 15;
                float sum = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) sum += red[par][w][m][nn];
                const int col = tile * 16 + nn;
                if (col < N) {
                    if (bias) sum += bf16_to_f32(bias[col]);
                    y[static_cast<int64_t>(m) * N + col] =
                        static_cast<uint16_t>(f32_to_bf16_rne(sum));
                }
            }
        }
    };

    int i = 0;
    while (i < nitems) {
        if (i + 1 < nitems) load(b1, i + 1);
        step(b0, i);
        if (++i >= nitems) break;
        if (i + 1 < nitems) load(b0, i + 1);
        step(b1, i);
        ++i;
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

template <int G>
hipError_t launch_stream(const uint16_t *x, int M, const uint8_t *codes,
                         const uint16_t *scales, const uint16_t *zeros,
                         const uint16_t *bias, int N, int K, uint16_t *y,
                         hipStream_t stream) {
    constexpr int NW = GV_STREAM_WAVES;
    auto kern = gemv_stream_kernel<G, NW>;
    static bool attr_set[64] = {false};         // per device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (dev < 0 || dev >= 64 || !attr_set[dev]) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 GV_STREAM_MAX_LDS);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) attr_set[dev] = true;
    }
    const int ntiles = (N + 15) / 16;
    const int kr = (K + 127) / 128 * 128;
    const size_t lds = static_cast<size_t>(M) * kr * 2 +
                       static_cast<size_t>(kr / G) * GV_STREAM_MAX_M * 4 +
                       2 * NW * GV_STREAM_MAX_M * 16 * 4;
    // resident blocks per compute unit: LDS (160 KB) and 2 blocks of NW waves
    int per_cu = static_cast<int>((160 * 1024) / lds);
    per_cu = per_cu < 1 ? 1 : (per_cu > 2 ? 2 : per_cu);
    const int slots = compute_units() * per_cu;
    const int blocks = ntiles < slots ? ntiles : slots;
    kern<<<dim3(blocks), dim3(NW * 64), lds, stream>>>(x, M, codes, scales, zeros, bias, N, K, y);
    return hipGetLastError();
}

template <int G>
hipError_t launch_gemv_g(const uint16_t *x, int M, const uint8_t *codes,
                         const uint16_t *scales, const uint16_t *zeros,
                         const uint16_t *bias, int N, int K, uint16_t *y,
                         hipStream_t stream) {
    const int ntiles = (N + 15) / 16;
    const int kr = (K + 127) / 128 * 128;
    if (M <= GV_STREAM_MAX_M && static_cast<int64_t>(M) * kr <= GV_X_ELEMS) {
        return launch_stream<G>(x, M, codes, scales, zeros, bias, N, K, y, stream);
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
