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
// 16-byte pieces per lane and wave chunk (1 KB per wave and piece): two
// keep 8 waves per SIMD resident; four measured no faster.
constexpr int QT_PPL = 2;

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

// One lane quantizes 8 consecutive elements (one 16-byte load); a group is
// G/8 consecutive lanes (4, 8 or 16: inside one DPP row). Returns, without
// storing anything: r.x = the 8 codes (4 bits each, element 0 in the low
// nibble), r.y = the group's scale | zero-point << 16 (bf16 bits); FAKE:
// the dequantized weights bf16_rne(fl32(q s + z)) (16 bytes). Every lane
// of the group must take part (the min / max reduction reads its partners).
template <int G, bool FAKE>
__device__ __forceinline__ u32x4 quantize8(const u32x4 d) {
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
    if constexpr (FAKE) {
        // q s is exact (4-bit q, bf16 s), so fma(q, s, z) is fl32(q s + z);
        // a fast-path q of -0 gives z exactly
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = f32_to_bf16_rne(fmaf(q[2 * j], s, lo)) |
                   (f32_to_bf16_rne(fmaf(q[2 * j + 1], s, lo)) << 16);
        return u32x4{o[0], o[1], o[2], o[3]};
    }
    return u32x4{out, sb | (zb << 16), 0u, 0u};
}

// Waits until the loads into d have landed (a use of the registers makes the
// compiler wait for them here, before any later memory operation is issued).
template <int PPL>
__device__ __forceinline__ void wait_for(const u32x4 (&d)[PPL]) {
#pragma unroll
    for (int j = 0; j < PPL; ++j) asm volatile("" ::"v"(d[j]));
}

// The streaming loop shared by the quantizers. W is a sequence of wave
// chunks of 64 PPL 16-byte pieces (512 PPL elements): lane l takes pieces
// l, l + 64, ..., so every load and store instruction of a wave covers one
// contiguous span (groups never straddle them: 512 is a multiple of G). A
// wave takes chunks w, w + stride, ...
//
// Order of a step: wait for the current chunk's loads, issue the next
// chunk's loads and the previous chunk's stores, then quantize the current
// chunk (results kept in registers until the next step), so that the
// stores complete under a whole step of arithmetic. Src supplies ctx(wi)
// (the chunk's buffer descriptors, built once per chunk in scalar
// registers), load(ctx, j) and store(ctx, j, r) for piece j of the chunk.
template <int G, bool FAKE, int PPL, class Src>
__device__ __forceinline__ void quantize_stream(const Src &src, int64_t w, int64_t nw,
                                                int64_t stride) {
    using Ctx = typename Src::Ctx;
    u32x4 a[PPL], b[PPL], r[PPL];
    auto ctx = [&](int64_t wi) { return src.ctx(wi < nw ? wi : nw - 1); };
    auto load = [&](u32x4 (&d)[PPL], const Ctx &c, int64_t wi) {
        if (wi < nw) {                        // wave-uniform
#pragma unroll
            for (int j = 0; j < PPL; ++j) d[j] = src.load(c, j);
        }
    };
    auto quant = [&](const u32x4 (&d)[PPL]) {
#pragma unroll
        for (int j = 0; j < PPL; ++j) r[j] = quantize8<G, FAKE>(d[j]);
    };
    auto store = [&](const Ctx &c) {
#pragma unroll
        for (int j = 0; j < PPL; ++j) src.store(c, j, r[j]);
    };
    const Ctx c0 = ctx(w);
    load(a, c0, w);
    int64_t w1 = w + stride;
    Ctx c1 = ctx(w1);
    load(b, c1, w1);
    quant(a);
    Ctx cp = c0;                              // the chunk r belongs to
    while (w1 < nw) {
        const int64_t w2 = w1 + stride;
        wait_for(b);
        const Ctx c2 = ctx(w2);
        load(a, c2, w2);
        store(cp);
        quant(b);
        cp = c1;
        if (w2 >= nw) break;
        w1 = w2 + stride;
        wait_for(a);
        c1 = ctx(w1);
        load(b, c1, w1);
        store(cp);
        quant(a);
        cp = c2;
    }
    store(cp);
}

// Loads and stores of one wave chunk go through buffer descriptors whose base
// is the chunk's first byte (wave-uniform, scalar registers) and whose size
// is the chunk's valid bytes: the per-lane offsets are constants, lanes past
// the end of the weight load zeros (a whole group of them, since nelem is a
// multiple of G: scale 0, nothing stored) and their stores are dropped, and
// only the first lane of a group stores its scale and zero-point (the other
// lanes' offsets lie outside every descriptor).
constexpr uint32_t QT_OOB = 0x80000000u;

struct ChunkCtx {
    __amdgpu_buffer_rsrc_t w;       // the chunk's weights
    __amdgpu_buffer_rsrc_t c;       // its codes (FAKE: its dequantized weights)
    __amdgpu_buffer_rsrc_t s, z;    // its groups' scales / zero-points
};

template <int G, bool FAKE, int PPL>
struct ChunkIO {
    static constexpr int64_t CH = 512 * PPL;   // elements per wave chunk
    static constexpr int LPG = G / 8;          // lanes per group
    // descriptors of chunk c of a weight of nelem elements
    __device__ static __forceinline__ ChunkCtx ctx(const uint16_t *W, uint8_t *codes,
                                                   uint16_t *scales, uint16_t *zeros,
                                                   uint16_t *what, int64_t nelem, int64_t c) {
        const int64_t e0 = c * CH;
        const int64_t n = min<int64_t>(CH, nelem - e0);   // valid elements
        ChunkCtx x;
        x.w = buf_rsrc(W + e0, static_cast<uint32_t>(n * 2));
        if constexpr (FAKE) {
            x.c = buf_rsrc(what + e0, static_cast<uint32_t>(n * 2));
            x.s = x.z = x.c;
        } else {
            x.c = buf_rsrc(codes + e0 / 2, static_cast<uint32_t>(n / 2));
            x.s = buf_rsrc(scales + e0 / G, static_cast<uint32_t>(n / G) * 2);
            x.z = buf_rsrc(zeros + e0 / G, static_cast<uint32_t>(n / G) * 2);
        }
        return x;
    }
    __device__ static __forceinline__ u32x4 load(const ChunkCtx &x, int lane, int j) {
        return __builtin_amdgcn_raw_buffer_load_b128(x.w, (lane + 64 * j) * 16, 0, W4_CPOL_STREAM);
    }
    __device__ static __forceinline__ void store(const ChunkCtx &x, int lane, int j, const u32x4 r) {
        const int p = lane + 64 * j;                        // piece in the chunk
        if constexpr (FAKE) {
            __builtin_amdgcn_raw_buffer_store_b128(r, x.c, p * 16, 0, W4_CPOL_STREAM);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(r.x, x.c, p * 4, 0, W4_CPOL_STREAM);
            const uint32_t go = lane % LPG == 0 ? (p / LPG) * 2 : QT_OOB;
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(r.y), x.s, go, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(r.y >> 16), x.z, go, 0, 0);
        }
    }
};

// One weight of nelem elements.
template <int G, bool FAKE, int PPL>
struct FlatSrc {
    using Ctx = ChunkCtx;
    const uint16_t *W;
    uint8_t *codes;
    uint16_t *scales;
    uint16_t *zeros;
    uint16_t *what;
    int64_t nelem;
    int lane;
    __device__ __forceinline__ Ctx ctx(int64_t wi) const {
        return ChunkIO<G, FAKE, PPL>::ctx(W, codes, scales, zeros, what, nelem, wi);
    }
    __device__ __forceinline__ u32x4 load(const Ctx &c, int j) const {
        return ChunkIO<G, FAKE, PPL>::load(c, lane, j);
    }
    __device__ __forceinline__ void store(const Ctx &c, int j, const u32x4 r) const {
        ChunkIO<G, FAKE, PPL>::store(c, lane, j, r);
    }
};

template <int G, bool FAKE, int PPL>
__global__ __launch_bounds__(QT_THREADS) void quantize_kernel(
    const uint16_t *__restrict__ W, int64_t nelem, uint8_t *__restrict__ codes,
    uint16_t *__restrict__ scales, uint16_t *__restrict__ zeros, uint16_t *__restrict__ what) {
    constexpr int WPB = QT_THREADS / 64;
    const int64_t nw = (nelem + 512 * PPL - 1) / (512 * PPL);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * WPB;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * WPB +
                      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    if (w >= nw) return;                       // whole waves
    const FlatSrc<G, FAKE, PPL> src{W, codes, scales, zeros, what, nelem,
                                    static_cast<int>(threadIdx.x & 63)};
    quantize_stream<G, FAKE, PPL>(src, w, nw, stride);
}

// Several weights in one launch (the layers of a block): the wave chunks of
// all jobs form one index space, job j owning chunks first[j] ..
// first[j + 1] - 1; a wave looks its chunk's job up (wave-uniform).
struct QuantBatch {
    const uint16_t *W[W4_QUANT_BATCH_MAX];
    uint8_t *codes[W4_QUANT_BATCH_MAX];
    uint16_t *scales[W4_QUANT_BATCH_MAX];
    uint16_t *zeros[W4_QUANT_BATCH_MAX];
    int64_t nelem[W4_QUANT_BATCH_MAX];
    int64_t first[W4_QUANT_BATCH_MAX + 1];
    int njobs;
};

template <int G, int PPL>
struct BatchSrc {
    using Ctx = ChunkCtx;
    const QuantBatch *b;
    int lane;
    __device__ __forceinline__ Ctx ctx(int64_t wi) const {
        int j = 0;
#pragma unroll
        for (int i = 1; i < W4_QUANT_BATCH_MAX; ++i)
            if (i < b->njobs && wi >= b->first[i]) j = i;
        return ChunkIO<G, false, PPL>::ctx(b->W[j], b->codes[j], b->scales[j], b->zeros[j],
                                           nullptr, b->nelem[j], wi - b->first[j]);
    }
    __device__ __forceinline__ u32x4 load(const Ctx &c, int j) const {
        return ChunkIO<G, false, PPL>::load(c, lane, j);
    }
    __device__ __forceinline__ void store(const Ctx &c, int j, const u32x4 r) const {
        ChunkIO<G, false, PPL>::store(c, lane, j, r);
    }
};

template <int G, int PPL>
__global__ __launch_bounds__(QT_THREADS) void quantize_batch_kernel(const QuantBatch b) {
    constexpr int WPB = QT_THREADS / 64;
    const int64_t nw = b.first[b.njobs];
    const int64_t stride = static_cast<int64_t>(gridDim.x) * WPB;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * WPB +
                      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    if (w >= nw) return;                       // whole waves
    const BatchSrc<G, PPL> src{&b, static_cast<int>(threadIdx.x & 63)};
    quantize_stream<G, false, PPL>(src, w, nw, stride);
}

} // namespace

namespace {

// Wave chunks per launch: 24 blocks of 4 waves per compute unit at most
// (more than stay resident: finer-grained work toward the end of the
// launch), fewer when the weight has fewer chunks.
int64_t quant_blocks(int64_t nw) {
    constexpr int64_t WPB = QT_THREADS / 64;
    int64_t blocks = (nw + WPB * QT_UNROLL - 1) / (WPB * QT_UNROLL);
    const int64_t max_blocks = static_cast<int64_t>(compute_units()) * 24;
    return blocks > max_blocks ? max_blocks : blocks;
}

template <int PPL>
hipError_t launch_batch(const w4_quant_job *jobs, int njobs, int G, hipStream_t stream) {
    QuantBatch b = {};
    b.njobs = njobs;
    b.first[0] = 0;
    for (int j = 0; j < njobs; ++j) {
        const int64_t nelem = jobs[j].N * jobs[j].K;
        b.W[j] = jobs[j].W;
        b.codes[j] = jobs[j].codes;
        b.scales[j] = jobs[j].scales;
        b.zeros[j] = jobs[j].zeros;
        b.nelem[j] = nelem;
        b.first[j + 1] = b.first[j] + (nelem + 512 * PPL - 1) / (512 * PPL);
    }
    for (int j = njobs; j < W4_QUANT_BATCH_MAX; ++j) b.first[j + 1] = b.first[njobs];
    const int64_t blocks = quant_blocks(b.first[njobs]);
    if (blocks < 1) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(blocks)), block(QT_THREADS);
    switch (G) {
    case 32: quantize_batch_kernel<32, PPL><<<grid, block, 0, stream>>>(b); break;
    case 64: quantize_batch_kernel<64, PPL><<<grid, block, 0, stream>>>(b); break;
    case 128: quantize_batch_kernel<128, PPL><<<grid, block, 0, stream>>>(b); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool FAKE, int PPL>
hipError_t launch_q(const uint16_t *W, int64_t N, int64_t K, int G, uint8_t *codes,
                    uint16_t *scales, uint16_t *zeros, uint16_t *what, hipStream_t stream) {
    const int64_t nelem = N * K;
    const int64_t blocks = quant_blocks((nelem + 512 * PPL - 1) / (512 * PPL));
    if (blocks < 1) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(blocks)), block(QT_THREADS);
    switch (G) {
    case 32: quantize_kernel<32, FAKE, PPL><<<grid, block, 0, stream>>>(W, nelem, codes, scales, zeros, what); break;
    case 64: quantize_kernel<64, FAKE, PPL><<<grid, block, 0, stream>>>(W, nelem, codes, scales, zeros, what); break;
    case 128: quantize_kernel<128, FAKE, PPL><<<grid, block, 0, stream>>>(W, nelem, codes, scales, zeros, what); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace

hipError_t launch_quantize_batch(const w4_quant_job *jobs, int njobs, int G,
                                 hipStream_t stream) {
    return launch_batch<QT_PPL>(jobs, njobs, G, stream);
}

hipError_t launch_quantize(const uint16_t *W, int64_t N, int64_t K, int G,
                           uint8_t *codes, uint16_t *scales, uint16_t *zeros,
                           hipStream_t stream) {
    return launch_q<false, QT_PPL>(W, N, K, G, codes, scales, zeros, nullptr, stream);
}

hipError_t launch_fake_quant(const uint16_t *W, int64_t N, int64_t K, int G, uint16_t *what,
                             hipStream_t stream) {
    return launch_q<true, QT_PPL>(W, N, K, G, nullptr, nullptr, nullptr, what, stream);
}

} // namespace w4
