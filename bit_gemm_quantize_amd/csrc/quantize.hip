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
// aligned inside a DPP row), which reduce min/max with DPP ops.
//
// Exactness: the scale is the correctly rounded binary32 quotient (a
// multiply by RN(1/15) and one fma correction, which reproduces the IEEE
// divide for every positive finite range; no fp contraction in this file).
// Codes use
// t = w * rcp(s) - lo * rcp(s) (one fma): with s in [2^-100, 2^100] the
// hardware reciprocal is within 1 ulp, so t is within 15.06 * 2^-21 plus the
// rounding of lo * rcp(s) of the correctly rounded quotient. When every t of
// the chunk is farther than that bound (with a margin) from a half-integer,
// rint(t) equals rint of the correctly rounded quotient; otherwise (and for
// extreme scales) the lane recomputes its chunk with the true divide. On the
// fast path -2^-20 < t <= 15.06 ((hi - lo)/s <= 15 (1 + 2^-8)), so rint(t)
// is already one of 0..15 (or -0).
#pragma clang fp contract(off)

#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

constexpr int QT_THREADS = 256;
constexpr int QT_UNROLL = 2;

// min / max of three floats in one VALU op. Written in asm so that the
// compiler does not add canonicalising copies of the bit-cast inputs (all
// inputs here are finite).
__device__ __forceinline__ float min3f(float a, float b, float c) {
    float d;
    asm("v_min3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}
// max(|a|, |b|, c)
__device__ __forceinline__ float max3_abs2(float a, float b, float c) {
    float d;
    asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// min / max of a and the same register of a partner lane, in one DPP op:
// xor 1 / xor 2 inside each quad, or the mirror inside each half row. The
// two wait states a DPP read needs after a VALU write of its source are
// inside the asm.
#define W4_DPP_MINMAX(name, op, ctrl)                                                   \
    __device__ __forceinline__ float name(float a) {                                    \
        float d;                                                                        \
        asm("s_nop 1\n\t" op " %0, %1, %1 " ctrl " row_mask:0xf bank_mask:0xf"        \
            : "=v"(d) : "v"(a));                                                        \
        return d;                                                                       \
    }
W4_DPP_MINMAX(min_xor1, "v_min_f32_dpp", "quad_perm:[1,0,3,2]")
W4_DPP_MINMAX(max_xor1, "v_max_f32_dpp", "quad_perm:[1,0,3,2]")
W4_DPP_MINMAX(min_xor2, "v_min_f32_dpp", "quad_perm:[2,3,0,1]")
W4_DPP_MINMAX(max_xor2, "v_max_f32_dpp", "quad_perm:[2,3,0,1]")
W4_DPP_MINMAX(min_hmirror, "v_min_f32_dpp", "row_half_mirror")
W4_DPP_MINMAX(max_hmirror, "v_max_f32_dpp", "row_half_mirror")
#undef W4_DPP_MINMAX

// One lane quantizes 16 consecutive elements (two 16-byte loads); a group is
// G/16 consecutive lanes (2, 4 or 8 inside one DPP row). FAKE: instead of
// codes, scales and zero-points, write the dequantized weights
// bf16_rne(fl32(q s + z)) (32 bytes per lane).
template <int G, bool FAKE>
__device__ __forceinline__ void quantize16(const u32x4 d0, const u32x4 d1, int64_t c,
                                          u32x2 *__restrict__ codes,
                                          uint16_t *__restrict__ scales,
                                          uint16_t *__restrict__ zeros,
                                          u32x4 *__restrict__ what) {
    constexpr int LPG = G / 16;
    float v[16];
    const uint32_t w[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
    float mn = min3f(v[0], v[1], v[2]);
    float mx = max3f(v[0], v[1], v[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) {
        mn = min3f(mn, v[i], v[i + 1]);
        mx = max3f(mx, v[i], v[i + 1]);
    }
    mn = min3f(mn, v[15], v[15]);
    mx = max3f(mx, v[15], v[15]);
    if constexpr (LPG >= 2) {
        mn = min_xor1(mn);
        mx = max_xor1(mx);
    }
    if constexpr (LPG >= 4) {
        mn = min_xor2(mn);
        mx = max_xor2(mx);
    }
    if constexpr (LPG >= 8) {
        mn = min_hmirror(mn);
        mx = max_hmirror(mx);
    }
    const float lo = mn + 0.0f;                // -0 -> +0
    const float hi = mx + 0.0f;
    const float range = hi - lo;
    // range / 15 correctly rounded: q0 = range * RN(1/15) and one fma
    // correction (equal to the IEEE quotient for every positive finite
    // binary32 range, denormals included; checked exhaustively)
    const float q0 = range * (1.0f / 15.0f);
    const float s32 = fmaf(fmaf(-15.0f, q0, range), 1.0f / 15.0f, q0);
    const uint32_t sb = f32_to_bf16_rne(s32);
    const float s = __uint_as_float(sb << 16);
    const uint32_t zb = __float_as_uint(lo) >> 16;

    uint32_t out0 = 0, out1 = 0;
    float q[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = 0.0f;
    if (s != 0.0f) {
        // Fast path: t = w * r + c with r = rcp(s), c = -lo * r. Its error
        // against fl(fl(w - lo) / s) is below 15.06 * 2^-21 + |c| * 2^-23, so
        // when every t is farther than 2^-16 + |c| * 2^-22 from a
        // half-integer, rint(t) is the exact code. Otherwise (or for
        // extreme scales) the chunk is redone with the true divide.
        const float r = __builtin_amdgcn_rcpf(s);
        const float cst = -lo * r;
        const bool extreme = !(s >= 0x1p-100f && s <= 0x1p100f);
        const float margin = 0.5f - (0x1p-16f + fabsf(cst) * 0x1p-22f);
        float dmax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const float t0 = fmaf(v[i], r, cst);
            const float t1 = fmaf(v[i + 1], r, cst);
            q[i] = __builtin_rintf(t0);
            q[i + 1] = __builtin_rintf(t1);
            dmax = max3_abs2(t0 - q[i], t1 - q[i + 1], dmax);
        }
        if (extreme || !(dmax < margin)) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                q[i] = fminf(fmaxf(__builtin_rintf((v[i] - lo) / s), 0.0f), 15.0f);
        }
        if constexpr (!FAKE) {
            // bytes q[2j] + 16 q[2j+1] (exact small integers), four per
            // dword; a fast-path q may be -0 (t a hair below 0): it converts
            // to 0
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                out0 = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(16.0f, q[2 * j + 1], q[2 * j]), j, out0);
                out1 = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(16.0f, q[2 * j + 9], q[2 * j + 8]), j, out1);
            }
        }
    }
    if constexpr (FAKE) {
        // q s is exact (4-bit q, bf16 s), so fma(q, s, z) is fl32(q s + z);
        // a fast-path q of -0 gives z exactly
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            o[j] = f32_to_bf16_rne(fmaf(q[2 * j], s, lo)) |
                   (f32_to_bf16_rne(fmaf(q[2 * j + 1], s, lo)) << 16);
        __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, what + 2 * c);
        __builtin_nontemporal_store(u32x4{o[4], o[5], o[6], o[7]}, what + 2 * c + 1);
        return;
    }
    __builtin_nontemporal_store(u32x2{out0, out1}, codes + c);
    // The first lane of each group stores the group's scale and zero-point
    // (a lane mask, not a branch: every chunk issues the same stores, so the
    // loop waits only for the loads it needs).
    if ((c & (LPG - 1)) == 0) {
        const int64_t grp = c / LPG;
        scales[grp] = static_cast<uint16_t>(sb);
        zeros[grp] = static_cast<uint16_t>(zb);
    }
}

template <int G, bool FAKE>
__global__ __launch_bounds__(QT_THREADS) void quantize_kernel(
    const u32x4 *__restrict__ W, int64_t nchunk, u32x2 *__restrict__ codes,
    uint16_t *__restrict__ scales, uint16_t *__restrict__ zeros, u32x4 *__restrict__ what) {
    // nchunk counts 16-element chunks; a thread takes chunks c, c + stride,
    // ... and loads the next one before quantizing the current one. Every
    // chunk of a group shares the in/out-of-range decision (nchunk and the
    // stride are multiples of the lanes per group). Loads use a clamped
    // index so they are never predicated.
    const int64_t stride = static_cast<int64_t>(gridDim.x) * QT_THREADS;
    const int64_t last = nchunk - 1;
    int64_t c = static_cast<int64_t>(blockIdx.x) * QT_THREADS + threadIdx.x;
    if (c >= nchunk) return;
    u32x4 a0, a1, b0, b1;
    auto load = [&](u32x4 &d0, u32x4 &d1, int64_t i) {
        const int64_t il = i < last ? i : last;
        d0 = __builtin_nontemporal_load(W + 2 * il);
        d1 = __builtin_nontemporal_load(W + 2 * il + 1);
    };
    // The first chunk is peeled so that the loop is entered, and re-entered,
    // with the same operations outstanding (the next chunk's loads, then the
    // current chunk's stores): the waits inside stay exact.
    load(a0, a1, c);
    int64_t c1 = c + stride;
    load(b0, b1, c1);
    quantize16<G, FAKE>(a0, a1, c, codes, scales, zeros, what);
    while (c1 < nchunk) {
        const int64_t c2 = c1 + stride;
        load(a0, a1, c2);
        quantize16<G, FAKE>(b0, b1, c1, codes, scales, zeros, what);
        if (c2 >= nchunk) break;
        c1 = c2 + stride;
        load(b0, b1, c1);
        quantize16<G, FAKE>(a0, a1, c2, codes, scales, zeros, what);
    }
}

} // namespace

namespace {

template <bool FAKE>
hipError_t launch_q(const uint16_t *W, int64_t N, int64_t K, int G, uint8_t *codes,
                    uint16_t *scales, uint16_t *zeros, uint16_t *what, hipStream_t stream) {
    const int64_t nchunk = N * K / 16;
    int64_t blocks = (nchunk + QT_THREADS * QT_UNROLL - 1) / (QT_THREADS * QT_UNROLL);
    const int64_t max_blocks = 256 * 8;        // 8 blocks per compute unit
    if (blocks > max_blocks) blocks = max_blocks;
    const dim3 grid(static_cast<unsigned>(blocks)), block(QT_THREADS);
    const u32x4 *w4p = reinterpret_cast<const u32x4 *>(W);
    u32x2 *c64 = reinterpret_cast<u32x2 *>(codes);
    u32x4 *wh = reinterpret_cast<u32x4 *>(what);
    switch (G) {
    case 32: quantize_kernel<32, FAKE><<<grid, block, 0, stream>>>(w4p, nchunk, c64, scales, zeros, wh); break;
    case 64: quantize_kernel<64, FAKE><<<grid, block, 0, stream>>>(w4p, nchunk, c64, scales, zeros, wh); break;
    case 128: quantize_kernel<128, FAKE><<<grid, block, 0, stream>>>(w4p, nchunk, c64, scales, zeros, wh); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_quantize(const uint16_t *W, int64_t N, int64_t K, int G,
                           uint8_t *codes, uint16_t *scales, uint16_t *zeros,
                           hipStream_t stream) {
    return launch_q<false>(W, N, K, G, codes, scales, zeros, nullptr, stream);
}

hipError_t launch_fake_quant(const uint16_t *W, int64_t N, int64_t K, int G, uint16_t *what,
                             hipStream_t stream) {
    return launch_q<true>(W, N, K, G, nullptr, nullptr, nullptr, what, stream);
}

} // namespace w4
