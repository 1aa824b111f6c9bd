// Group-wise asymmetric int4 quantizer for gfx950.
//
// Method: "Optimum Quanto", "Design overview / Tensors" - below 8 bits each
// group is projected affinely, with an offset, onto the 4-bit range and
// mapped by rounding half to even; "Modules" - groups run along the input
// dimension of each output row. Per row n and group g, in IEEE binary32:
//   lo = min + 0, hi = max + 0, s = bf16_rne((hi - lo) / 15), z = lo,
//   q = s == 0 ? 0 : clamp(rint((w - lo) / s), 0, 15).
//
// Layout of the work: W[N, K] is streamed as a flat array of 16-byte pieces
// (8 bf16; two pieces per lane and step, 1 KB apart). K is a multiple of G,
// so group f of the flat array is (n, g) = (f / (K/G), f % (K/G)) and the
// scale/zero arrays [N, K/G] are indexed by the flat group number; likewise
// codes are the flat piece number times 4 bytes. A group is G/8 consecutive
// lanes (4, 8 or 16, aligned inside a DPP row), which reduce min/max with
// DPP ops.
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
// xor 1 / xor 2 inside each quad, or the mirror inside each half row or row. The
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
W4_DPP_MINMAX(min_mirror, "v_min_f32_dpp", "row_mirror")
W4_DPP_MINMAX(max_mirror, "v_max_f32_dpp", "row_mirror")
#undef W4_DPP_MINMAX

// One lane quantizes 8 consecutive elements (one 16-byte load), the first
// at flat index e0; a group is G/8 consecutive lanes (4, 8 or 16: inside one
// DPP row). FAKE: instead of codes, scales and zero-points, write the
// dequantized weights bf16_rne(fl32(q s + z)) (16 bytes per lane). Lanes
// past the end (live false) compute on a clamped copy and store nothing.
template <int G, bool FAKE>
__device__ __forceinline__ void quantize8(const u32x4 d, int64_t e0, bool live,
                                         uint32_t *__restrict__ codes,
                                         uint16_t *__restrict__ scales,
                                         uint16_t *__restrict__ zeros,
                                         u32x4 *__restrict__ what) {
    constexpr int LPG = G / 8;
    const float v[8] = {bf16_lo(d.x), bf16_hi(d.x), bf16_lo(d.y), bf16_hi(d.y),
                        bf16_lo(d.z), bf16_hi(d.z), bf16_lo(d.w), bf16_hi(d.w)};
    float mn = min3f(v[0], v[1], v[2]);
    float mx = max3f(v[0], v[1], v[2]);
    mn = min3f(mn, v[3], v[4]);
    mx = max3f(mx, v[3], v[4]);
    mn = min3f(mn, v[5], v[6]);
    mx = max3f(mx, v[5], v[6]);
    mn = min3f(mn, v[7], v[7]);
    mx = max3f(mx, v[7], v[7]);
    mn = min_xor1(mn);
    mx = max_xor1(mx);
    mn = min_xor2(mn);
    mx = max_xor2(mx);
    if constexpr (LPG >= 8) {
        mn = min_hmirror(mn);
        mx = max_hmirror(mx);
    }
    if constexpr (LPG >= 16) {
        mn = min_mirror(mn);
        mx = max_mirror(mx);
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

    uint32_t out = 0;
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = 0.0f;
    if (s != 0.0f) {
        // Fast path: t = w * r + c with r = rcp(s), c = -lo * r. Its error
        // against fl(fl(w - lo) / s) is below 15.06 * 2^-21 + |c| * 2^-23, so
        // when every t is farther than 2^-16 + |c| * 2^-22 from a
        // half-integer, rint(t) is the exact code. Otherwise (or for
        // extreme scales) the lane's elements are redone with the true divide.
        const float r = __builtin_amdgcn_rcpf(s);
        const float cst = -lo * r;
        const bool extreme = !(s >= 0x1p-100f && s <= 0x1p100f);
        const float margin = 0.5f - (0x1p-16f + fabsf(cst) * 0x1p-22f);
        float dmax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            const float t0 = fmaf(v[i], r, cst);
            const float t1 = fmaf(v[i + 1], r, cst);
            q[i] = __builtin_rintf(t0);
            q[i + 1] = __builtin_rintf(t1);
            dmax = max3_abs2(t0 - q[i], t1 - q[i + 1], dmax);
        }
        if (extreme || !(dmax < margin)) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                q[i] = fminf(fmaxf(__builtin_rintf((v[i] - lo) / s), 0.0f), 15.0f);
        }
        if constexpr (!FAKE) {
            // bytes q[2j] + 16 q[2j+1] (exact small integers); a fast-path q
            // may be -0 (t a hair below 0): it converts to 0
#pragma unroll
            for (int j = 0; j < 4; ++j)
                out = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(16.0f, q[2 * j + 1], q[2 * j]), j, out);
        }
    }
    if (!live) return;
    if constexpr (FAKE) {
        // q s is exact (4-bit q, bf16 s), so fma(q, s, z) is fl32(q s + z);
        // a fast-path q of -0 gives z exactly
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = f32_to_bf16_rne(fmaf(q[2 * j], s, lo)) |
                   (f32_to_bf16_rne(fmaf(q[2 * j + 1], s, lo)) << 16);
        __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, what + e0 / 8);
        return;
    }
    __builtin_nontemporal_store(out, codes + e0 / 8);
    // the first lane of each group stores the group's scale and zero-point
    if (((e0 / 8) & (LPG - 1)) == 0) {
        scales[e0 / G] = static_cast<uint16_t>(sb);
        zeros[e0 / G] = static_cast<uint16_t>(zb);
    }
}

// W is streamed in wave chunks of 1024 elements (2 KB): lane l quantizes
// the 16-byte pieces l and 64 + l of the chunk, so each load and each store
// instruction of a wave covers one contiguous span (1 KB of W, 256 bytes of
// codes). Groups never straddle the halves (512 is a multiple of G).
template <int G, bool FAKE>
__global__ __launch_bounds__(QT_THREADS) void quantize_kernel(
    const u32x4 *__restrict__ W, int64_t nelem, uint32_t *__restrict__ codes,
    uint16_t *__restrict__ scales, uint16_t *__restrict__ zeros, u32x4 *__restrict__ what) {
    // A wave takes chunks w, w + stride, ... and loads the next one before
    // quantizing the current one. Loads use clamped indices so they are
    // never predicated; stores are masked by the element count.
    constexpr int WPB = QT_THREADS / 64;
    const int lane = threadIdx.x & 63;
    const int64_t npiece = nelem / 8;          // nelem % 32 == 0
    const int64_t nw = (nelem + 1023) / 1024;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * WPB;
    int64_t w = static_cast<int64_t>(blockIdx.x) * WPB + (threadIdx.x >> 6);
    if (w >= nw) return;                       // whole waves
    u32x4 a0, a1, b0, b1;
    auto load = [&](u32x4 &d0, u32x4 &d1, int64_t wi) {
        const int64_t wl = wi < nw ? wi : nw - 1;
        const int64_t p0 = 128 * wl + lane, p1 = p0 + 64;
        d0 = __builtin_nontemporal_load(W + (p0 < npiece ? p0 : npiece - 1));
        d1 = __builtin_nontemporal_load(W + (p1 < npiece ? p1 : npiece - 1));
    };
    auto work = [&](const u32x4 &d0, const u32x4 &d1, int64_t wi) {
        const int64_t p0 = 128 * wi + lane, p1 = p0 + 64;
        quantize8<G, FAKE>(d0, 8 * p0, p0 < npiece, codes, scales, zeros, what);
        quantize8<G, FAKE>(d1, 8 * p1, p1 < npiece, codes, scales, zeros, what);
    };
    // The first chunk is peeled so that the loop is entered, and re-entered,
    // with the same operations outstanding (the next chunk's loads, then the
    // current chunk's stores): the waits inside stay exact.
    load(a0, a1, w);
    int64_t w1 = w + stride;
    load(b0, b1, w1);
    work(a0, a1, w);
    while (w1 < nw) {
        const int64_t w2 = w1 + stride;
        load(a0, a1, w2);
        work(b0, b1, w1);
        if (w2 >= nw) break;
        w1 = w2 + stride;
        load(b0, b1, w1);
        work(a0, a1, w2);
    }
}

// Several weights in one launch (the layers of a block): the wave chunks of
// all jobs form one index space, job j owning chunks first[j] ..
// first[j + 1] - 1; a wave looks its chunk's job up (wave-uniform) and
// works as quantize_kernel does.
struct QuantBatch {
    const u32x4 *W[W4_QUANT_BATCH_MAX];
    uint32_t *codes[W4_QUANT_BATCH_MAX];
    uint16_t *scales[W4_QUANT_BATCH_MAX];
    uint16_t *zeros[W4_QUANT_BATCH_MAX];
    int64_t npiece[W4_QUANT_BATCH_MAX];
    int64_t first[W4_QUANT_BATCH_MAX + 1];
    int njobs;
};

template <int G>
__global__ __launch_bounds__(QT_THREADS) void quantize_batch_kernel(const QuantBatch b) {
    constexpr int WPB = QT_THREADS / 64;
    const int lane = threadIdx.x & 63;
    const int64_t nw = b.first[b.njobs];
    const int64_t stride = static_cast<int64_t>(gridDim.x) * WPB;
    int64_t w = static_cast<int64_t>(blockIdx.x) * WPB +
                __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    if (w >= nw) return;                       // whole waves
    auto job_of = [&](int64_t wi) {
        int j = 0;
#pragma unroll
        for (int i = 1; i < W4_QUANT_BATCH_MAX; ++i)
            if (i < b.njobs && wi >= b.first[i]) j = i;
        return j;
    };
    u32x4 a0, a1, b0, b1;
    auto load = [&](u32x4 &d0, u32x4 &d1, int64_t wi) {
        const int64_t wl = wi < nw ? wi : nw - 1;
        const int j = job_of(wl);
        const int64_t np = b.npiece[j];
        const int64_t p0 = 128 * (wl - b.first[j]) + lane, p1 = p0 + 64;
        d0 = __builtin_nontemporal_load(b.W[j] + (p0 < np ? p0 : np - 1));
        d1 = __builtin_nontemporal_load(b.W[j] + (p1 < np ? p1 : np - 1));
    };
    auto work = [&](const u32x4 &d0, const u32x4 &d1, int64_t wi) {
        const int j = job_of(wi);
        const int64_t np = b.npiece[j];
        const int64_t p0 = 128 * (wi - b.first[j]) + lane, p1 = p0 + 64;
        quantize8<G, false>(d0, 8 * p0, p0 < np, b.codes[j], b.scales[j], b.zeros[j], nullptr);
        quantize8<G, false>(d1, 8 * p1, p1 < np, b.codes[j], b.scales[j], b.zeros[j], nullptr);
    };
    load(a0, a1, w);
    int64_t w1 = w + stride;
    load(b0, b1, w1);
    work(a0, a1, w);
    while (w1 < nw) {
        const int64_t w2 = w1 + stride;
        load(a0, a1, w2);
        work(b0, b1, w1);
        if (w2 >= nw) break;
        w1 = w2 + stride;
        load(b0, b1, w1);
        work(a0, a1, w2);
    }
}

} // namespace

hipError_t launch_quantize_batch(const w4_quant_job *jobs, int njobs, int G,
                                 hipStream_t stream) {
    QuantBatch b = {};
    b.njobs = njobs;
    b.first[0] = 0;
    for (int j = 0; j < njobs; ++j) {
        const int64_t nelem = jobs[j].N * jobs[j].K;
        b.W[j] = reinterpret_cast<const u32x4 *>(jobs[j].W);
        b.codes[j] = reinterpret_cast<uint32_t *>(jobs[j].codes);
        b.scales[j] = jobs[j].scales;
        b.zeros[j] = jobs[j].zeros;
        b.npiece[j] = nelem / 8;
        b.first[j + 1] = b.first[j] + (nelem + 1023) / 1024;
    }
    for (int j = njobs; j < W4_QUANT_BATCH_MAX; ++j) b.first[j + 1] = b.first[njobs];
    const int64_t nw = b.first[njobs];
    constexpr int64_t WPB = QT_THREADS / 64;
    int64_t blocks = (nw + WPB * QT_UNROLL - 1) / (WPB * QT_UNROLL);
    // 24 blocks per compute unit (more than stay resident: finer-grained
    // work toward the end of the launch; 8 per unit measured ≈ 10% slower)
    const int64_t max_blocks = static_cast<int64_t>(compute_units()) * 24;
    if (blocks > max_blocks) blocks = max_blocks;
    if (blocks < 1) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(blocks)), block(QT_THREADS);
    switch (G) {
    case 32: quantize_batch_kernel<32><<<grid, block, 0, stream>>>(b); break;
    case 64: quantize_batch_kernel<64><<<grid, block, 0, stream>>>(b); break;
    case 128: quantize_batch_kernel<128><<<grid, block, 0, stream>>>(b); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

namespace {

template <bool FAKE>
hipError_t launch_q(const uint16_t *W, int64_t N, int64_t K, int G, uint8_t *codes,
                    uint16_t *scales, uint16_t *zeros, uint16_t *what, hipStream_t stream) {
    const int64_t nelem = N * K;
    const int64_t nw = (nelem + 1023) / 1024;  // wave chunks
    constexpr int64_t WPB = QT_THREADS / 64;
    int64_t blocks = (nw + WPB * QT_UNROLL - 1) / (WPB * QT_UNROLL);
    // 24 blocks per compute unit (more than stay resident: finer-grained
    // work toward the end of the launch; 8 per unit measured ≈ 10% slower)
    const int64_t max_blocks = static_cast<int64_t>(compute_units()) * 24;
    if (blocks > max_blocks) blocks = max_blocks;
    const dim3 grid(static_cast<unsigned>(blocks)), block(QT_THREADS);
    const u32x4 *w4p = reinterpret_cast<const u32x4 *>(W);
    uint32_t *c32 = reinterpret_cast<uint32_t *>(codes);
    u32x4 *wh = reinterpret_cast<u32x4 *>(what);
    switch (G) {
    case 32: quantize_kernel<32, FAKE><<<grid, block, 0, stream>>>(w4p, nelem, c32, scales, zeros, wh); break;
    case 64: quantize_kernel<64, FAKE><<<grid, block, 0, stream>>>(w4p, nelem, c32, scales, zeros, wh); break;
    case 128: quantize_kernel<128, FAKE><<<grid, block, 0, stream>>>(w4p, nelem, c32, scales, zeros, wh); break;
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
