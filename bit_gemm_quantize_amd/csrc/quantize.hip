// Group-wise asymmetric int4 quantizer for gfx950.
//
// Method: "Optimum Quanto", "Design overview / Tensors" - below 8 bits each
// group is projected affinely, with an offset, onto the 4-bit range and
// mapped by rounding half to even; "Modules" - groups run along the input
// dimension of each output row. Per row n and group g, in IEEE binary32:
//   lo = min + 0, hi = max + 0, s = bf16_rne((hi - lo) / 15), z = lo,
//   q = s == 0 ? 0 : clamp(rint((w - lo) / s), 0, 15).
//
// Layout of the work: W[N, K] is streamed as a flat array of 32-byte chunks
// (16 bf16, one chunk per lane and step). K is a multiple of G, so group f of
// the flat array is (n, g) = (f / (K/G), f % (K/G)) and the scale/zero arrays
// [N, K/G] are indexed by the flat group number; likewise codes are the flat
// chunk number times 8 bytes. A group is G/16 consecutive lanes (2, 4 or 8,
// aligned inside a DPP row), which reduce min/max with DPP moves.
//
// Exactness: the scale uses a correctly rounded binary32 divide (built with
// correctly rounded division; no fp contraction in this file). Codes use
// t = (w - lo) * rcp(s): with s in [2^-100, 2^100] the hardware reciprocal is
// within 1 ulp, so |t - fl((w - lo) / s)| < 4e-6 for t <= 15.06. When t is
// farther than 2^-16 from a half-integer, rint(t) equals rint of the
// correctly rounded quotient; otherwise (and for extreme scales) the lane
// recomputes every element of its chunk with the true divide. On the fast
// path 0 <= t <= 15.06 (w - lo <= hi - lo, and (hi - lo)/s <= 15 (1 + 2^-8)),
// so rint(t) is already inside [0, 15].
#pragma clang fp contract(off)

#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

constexpr int QT_THREADS = 256;
constexpr int QT_UNROLL = 2;

// One lane quantizes 16 consecutive elements (two 16-byte loads); a group is
// G/16 consecutive lanes (2, 4 or 8 inside one DPP row).
template <int G>
__device__ __forceinline__ void quantize16(const u32x4 d0, const u32x4 d1, int64_t c,
                                          u32x2 *__restrict__ codes,
                                          uint16_t *__restrict__ scales,
                                          uint16_t *__restrict__ zeros) {
    constexpr int LPG = G / 16;
    float v[16];
    const uint32_t w[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
    float mn = fminf(v[0], v[1]), mx = fmaxf(v[0], v[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
        mn = fminf(mn, fminf(v[i], v[i + 1]));
        mx = fmaxf(mx, fmaxf(v[i], v[i + 1]));
    }
    if constexpr (LPG >= 2) {
        mn = fminf(mn, dpp_f32<DPP_QUAD_XOR1>(mn));
        mx = fmaxf(mx, dpp_f32<DPP_QUAD_XOR1>(mx));
    }
    if constexpr (LPG >= 4) {
        mn = fminf(mn, dpp_f32<DPP_QUAD_XOR2>(mn));
        mx = fmaxf(mx, dpp_f32<DPP_QUAD_XOR2>(mx));
    }
    if constexpr (LPG >= 8) {
        mn = fminf(mn, dpp_f32<DPP_ROW_HALF_MIRROR>(mn));
        mx = fmaxf(mx, dpp_f32<DPP_ROW_HALF_MIRROR>(mx));
    }
    const float lo = mn + 0.0f;                // -0 -> +0
    const float hi = mx + 0.0f;
    const float range = hi - lo;
    const float s32 = range / 15.0f;           // correctly rounded
    const uint32_t sb = f32_to_bf16_rne(s32);
    const float s = __uint_as_float(sb << 16);
    const uint32_t zb = __float_as_uint(lo) >> 16;

    uint32_t out0 = 0, out1 = 0;
    if (s != 0.0f) {
        const float r = __builtin_amdgcn_rcpf(s);
        bool exact = !(s >= 0x1p-100f && s <= 0x1p100f);
        float q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float t = (v[i] - lo) * r;
            q[i] = __builtin_rintf(t);
            // t within 2^-16 of a half-integer: the reciprocal may have
            // decided the rounding; redo the chunk with the true divide.
            exact |= fabsf(t - q[i]) > 0.5f - 0x1p-16f;
        }
        if (exact) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                q[i] = fminf(fmaxf(__builtin_rintf((v[i] - lo) / s), 0.0f), 15.0f);
        }
        // bytes q[2j] + 16 q[2j+1] (exact small integers), four per dword
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out0 = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(16.0f, q[2 * j + 1], q[2 * j]), j, out0);
            out1 = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(16.0f, q[2 * j + 9], q[2 * j + 8]), j, out1);
        }
    }
    __builtin_nontemporal_store(u32x2{out0, out1}, codes + c);
    if ((c & (LPG - 1)) == 0) {
        const int64_t grp = c / LPG;
        scales[grp] = static_cast<uint16_t>(sb);
        zeros[grp] = static_cast<uint16_t>(zb);
    }
}

template <int G>
__global__ __launch_bounds__(QT_THREADS) void quantize_kernel(
    const u32x4 *__restrict__ W, int64_t nchunk, u32x2 *__restrict__ codes,
    uint16_t *__restrict__ scales, uint16_t *__restrict__ zeros) {
    // nchunk counts 16-element chunks. Every chunk of a group shares the
    // in/out-of-range decision: nchunk and the grid stride are multiples of
    // the lanes per group.
    const int64_t stride = static_cast<int64_t>(gridDim.x) * QT_THREADS;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * QT_THREADS + threadIdx.x;
         base < nchunk; base += stride * QT_UNROLL) {
        u32x4 d[QT_UNROLL][2];
#pragma unroll
        for (int u = 0; u < QT_UNROLL; ++u) {
            const int64_t c = base + u * stride;
            if (c < nchunk) {
                d[u][0] = __builtin_nontemporal_load(W + 2 * c);
                d[u][1] = __builtin_nontemporal_load(W + 2 * c + 1);
            }
        }
#pragma unroll
        for (int u = 0; u < QT_UNROLL; ++u) {
            const int64_t c = base + u * stride;
            if (c < nchunk) quantize16<G>(d[u][0], d[u][1], c, codes, scales, zeros);
        }
    }
}

} // namespace

hipError_t launch_quantize(const uint16_t *W, int64_t N, int64_t K, int G,
                           uint8_t *codes, uint16_t *scales, uint16_t *zeros,
                           hipStream_t stream) {
    const int64_t nchunk = N * K / 16;
    int64_t blocks = (nchunk + QT_THREADS * QT_UNROLL - 1) / (QT_THREADS * QT_UNROLL);
    const int64_t max_blocks = 256 * 8;        // 8 blocks per compute unit
    if (blocks > max_blocks) blocks = max_blocks;
    const dim3 grid(static_cast<unsigned>(blocks)), block(QT_THREADS);
    const u32x4 *w4p = reinterpret_cast<const u32x4 *>(W);
    u32x2 *c64 = reinterpret_cast<u32x2 *>(codes);
    switch (G) {
    case 32: quantize_kernel<32><<<grid, block, 0, stream>>>(w4p, nchunk, c64, scales, zeros); break;
    case 64: quantize_kernel<64><<<grid, block, 0, stream>>>(w4p, nchunk, c64, scales, zeros); break;
    case 128: quantize_kernel<128><<<grid, block, 0, stream>>>(w4p, nchunk, c64, scales, zeros); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace w4
