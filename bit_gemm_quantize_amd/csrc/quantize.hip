// Group-wise asymmetric int4 quantizer for gfx950.
//
// Method: "Optimum Quanto", "Design overview / Tensors" - below 8 bits each
// group is projected affinely, with an offset, onto the 4-bit range and
// mapped by rounding half to even; "Modules" - groups run along the input
// dimension of each output row. Per row n and group g, in IEEE binary32:
//   lo = min + 0, hi = max + 0, s = bf16_rne((hi - lo) / 15), z = lo,
//   q = s == 0 ? 0 : clamp(rint((w - lo) / s), 0, 15).
//
// Layout of the work: W[N, K] is streamed as a flat array of 16-byte chunks
// (8 bf16). K is a multiple of G, so group f of the flat array is (n, g) =
// (f / (K/G), f % (K/G)) and the scale/zero arrays [N, K/G] are indexed by
// the flat group number; likewise codes are the flat chunk number times 4
// bytes. A group is G/8 consecutive lanes (4, 8 or 16, aligned inside a
// 16-lane DPP row), which reduce min/max with DPP moves.
//
// Exactness: the scale uses a correctly rounded binary32 divide (built with
// correctly rounded division; no fp contraction in this file). Codes use
// t = (w - lo) * rcp(s): with s in [2^-100, 2^100] the hardware reciprocal is
// within 1 ulp, so |t - fl((w - lo) / s)| < 4e-6 for t <= 15.06. When t is
// farther than 2^-16 from a half-integer, rint(t) equals rint of the
// correctly rounded quotient; otherwise (and for extreme scales) the lane
// recomputes every element of its chunk with the true divide.
#pragma clang fp contract(off)

#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

constexpr int QT_THREADS = 256;
constexpr int QT_UNROLL = 4;

template <int G>
__device__ __forceinline__ void quantize_chunk(u32x4 d, int64_t c,
                                               uint32_t *__restrict__ codes,
                                               uint16_t *__restrict__ scales,
                                               uint16_t *__restrict__ zeros) {
    constexpr int LPG = G / 8;                 // lanes per group
    float v[8];
    v[0] = bf16_lo(d.x); v[1] = bf16_hi(d.x);
    v[2] = bf16_lo(d.y); v[3] = bf16_hi(d.y);
    v[4] = bf16_lo(d.z); v[5] = bf16_hi(d.z);
    v[6] = bf16_lo(d.w); v[7] = bf16_hi(d.w);

    float mn = v[0], mx = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        mn = fminf(mn, v[i]);
        mx = fmaxf(mx, v[i]);
    }
    group_minmax<LPG>(mn, mx);
    const float lo = mn + 0.0f;                // -0 -> +0
    const float hi = mx + 0.0f;
    const float range = hi - lo;
    const float s32 = range / 15.0f;           // correctly rounded
    const uint32_t sb = f32_to_bf16_rne(s32);
    const float s = __uint_as_float(sb << 16);
    const uint32_t zb = __float_as_uint(lo) >> 16;

    uint32_t packed = 0;
    if (s != 0.0f) {
        const float r = __builtin_amdgcn_rcpf(s);
        bool exact = !(s >= 0x1p-100f && s <= 0x1p100f);
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float t = (v[i] - lo) * r;
            const float f = __builtin_amdgcn_fractf(t);
            exact |= !(fabsf(f - 0.5f) > 0x1p-16f);
            q[i] = __builtin_rintf(t);
        }
        if (exact) {
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = __builtin_rintf((v[i] - lo) / s);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float qc = fminf(fmaxf(q[i], 0.0f), 15.0f);
            packed |= static_cast<uint32_t>(qc) << (4 * i);
        }
    }
    __builtin_nontemporal_store(packed, codes + c);
    if ((c & (LPG - 1)) == 0) {
        const int64_t grp = c / LPG;
        scales[grp] = static_cast<uint16_t>(sb);
        zeros[grp] = static_cast<uint16_t>(zb);
    }
}

template <int G>
__global__ __launch_bounds__(QT_THREADS) void quantize_kernel(
    const u32x4 *__restrict__ W, int64_t nchunk, uint32_t *__restrict__ codes,
    uint16_t *__restrict__ scales, uint16_t *__restrict__ zeros) {
    // Every chunk index of a group shares the in/out-of-range decision:
    // nchunk and the grid stride are multiples of the lanes per group.
    const int64_t stride = static_cast<int64_t>(gridDim.x) * QT_THREADS;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * QT_THREADS + threadIdx.x;
         base < nchunk; base += stride * QT_UNROLL) {
        u32x4 d[QT_UNROLL];
#pragma unroll
        for (int u = 0; u < QT_UNROLL; ++u) {
            const int64_t c = base + u * stride;
            if (c < nchunk) d[u] = __builtin_nontemporal_load(W + c);
        }
#pragma unroll
        for (int u = 0; u < QT_UNROLL; ++u) {
            const int64_t c = base + u * stride;
            if (c < nchunk) quantize_chunk<G>(d[u], c, codes, scales, zeros);
        }
    }
}

} // namespace

hipError_t launch_quantize(const uint16_t *W, int64_t N, int64_t K, int G,
                           uint8_t *codes, uint16_t *scales, uint16_t *zeros,
                           hipStream_t stream) {
    const int64_t nchunk = N * K / 8;
    int64_t blocks = (nchunk + QT_THREADS * QT_UNROLL - 1) / (QT_THREADS * QT_UNROLL);
    const int64_t max_blocks = 256 * 16;       // 16 blocks per compute unit
    if (blocks > max_blocks) blocks = max_blocks;
    const dim3 grid(static_cast<unsigned>(blocks)), block(QT_THREADS);
    const u32x4 *w4p = reinterpret_cast<const u32x4 *>(W);
    uint32_t *c32 = reinterpret_cast<uint32_t *>(codes);
    switch (G) {
    case 32: quantize_kernel<32><<<grid, block, 0, stream>>>(w4p, nchunk, c32, scales, zeros); break;
    case 64: quantize_kernel<64><<<grid, block, 0, stream>>>(w4p, nchunk, c32, scales, zeros); break;
    case 128: quantize_kernel<128><<<grid, block, 0, stream>>>(w4p, nchunk, c32, scales, zeros); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace w4
