// Device helpers shared by the gfx950 kernels of the W4A16 library.
//
// bf16 values travel as raw 16-bit patterns. Codes are 4-bit unsigned
// integers, two per byte, low nibble = even k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_lo(uint32_t pair) {   // element 0
    return __uint_as_float(pair << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t pair) {   // element 1
    return __uint_as_float(pair & 0xFFFF0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// binary32 -> bf16, round to nearest, ties to even (finite inputs; a carry
// into the exponent is the correct rounding up).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// ------------------------------------------------------------- DPP reduce
// Min/max across aligned lane groups of 4, 8 or 16 lanes with DPP moves
// (quad permutes, then half-row and row mirrors; each step leaves every
// lane of the group holding the partial result of its whole sub-group).

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(
        0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

constexpr int DPP_QUAD_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141; // lane i <- lane 7-i within 8
constexpr int DPP_ROW_MIRROR = 0x140;      // lane i <- lane 15-i within 16

template <int LANES>
__device__ __forceinline__ void group_minmax(float &mn, float &mx) {
    static_assert(LANES == 4 || LANES == 8 || LANES == 16, "group lanes");
    mn = fminf(mn, dpp_f32<DPP_QUAD_XOR1>(mn));
    mx = fmaxf(mx, dpp_f32<DPP_QUAD_XOR1>(mx));
    mn = fminf(mn, dpp_f32<DPP_QUAD_XOR2>(mn));
    mx = fmaxf(mx, dpp_f32<DPP_QUAD_XOR2>(mx));
    if constexpr (LANES >= 8) {
        mn = fminf(mn, dpp_f32<DPP_ROW_HALF_MIRROR>(mn));
        mx = fmaxf(mx, dpp_f32<DPP_ROW_HALF_MIRROR>(mx));
    }
    if constexpr (LANES >= 16) {
        mn = fminf(mn, dpp_f32<DPP_ROW_MIRROR>(mn));
        mx = fmaxf(mx, dpp_f32<DPP_ROW_MIRROR>(mx));
    }
}

// Sum across aligned lane groups of 4, 8 or 16 lanes (every lane of the
// group receives the group's sum).
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(LANES == 4 || LANES == 8 || LANES == 16, "group lanes");
    v += dpp_f32<DPP_QUAD_XOR1>(v);
    v += dpp_f32<DPP_QUAD_XOR2>(v);
    if constexpr (LANES >= 8) v += dpp_f32<DPP_ROW_HALF_MIRROR>(v);
    if constexpr (LANES >= 16) v += dpp_f32<DPP_ROW_MIRROR>(v);
    return v;
}

// ----------------------------------------------------------- code unpack
// (a & mask) | c: the compiler selects one v_and_or_b32 for it. It must
// stay plain code: a VALU op written as inline asm is invisible to the
// compiler's hazard checks, and placed next to a matrix-core op that reads
// or writes the same registers it gave wrong, run-to-run varying results.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
    return (a & mask) | c;
}

// Constants of the nibble expansion, materialised once per kernel.
struct Unpack128 {
    uint32_t mask;     // 0x000F000F (scalar)
    uint32_t bias;     // 0x43004300 (vector)
};
__device__ __forceinline__ Unpack128 unpack128_consts() {
    Unpack128 u;
    u.mask = __builtin_amdgcn_readfirstlane(0x000F000Fu);
    u.bias = 0x43004300u;
    asm volatile("" : "+v"(u.bias));   // keep it in a VGPR
    return u;
}

// One dword of 8 codes (k = 0..7, natural order) -> four bf16 pairs holding
// the exact integers 128 + q: bf16 0x4300 is 128.0 and its 7 mantissa bits
// count in units of 1, so 0x4300 | q == 128 + q for q in 0..15.
// out[i] = (128 + q[2i]) | (128 + q[2i+1]) << 16.
__device__ __forceinline__ void unpack8_bias128(uint32_t w, uint32_t out[4],
                                                const Unpack128 &c) {
    const uint32_t w4 = w >> 4;
    // byte0 <- w.byte i (q[2i] in its low nibble), byte2 <- (w>>4).byte i
    // (q[2i+1] in its low nibble), bytes 1 and 3 <- 0.
    out[0] = and_or(__builtin_amdgcn_perm(w4, w, 0x0C040C00u), c.mask, c.bias);
    out[1] = and_or(__builtin_amdgcn_perm(w4, w, 0x0C050C01u), c.mask, c.bias);
    out[2] = and_or(__builtin_amdgcn_perm(w4, w, 0x0C060C02u), c.mask, c.bias);
    out[3] = and_or(__builtin_amdgcn_perm(w4, w, 0x0C070C03u), c.mask, c.bias);
}

// One dword of 8 codes -> four bf16 pairs of 128 + q in the interleaved
// order (q0,q4), (q1,q5), (q2,q6), (q3,q7): k = 0,4,1,5,2,6,3,7. The other
// MFMA operand must list its 8 values in the same order (see
// interleave8_bf16). 7 VALU ops instead of 9.
__device__ __forceinline__ void unpack8_bias128_il(uint32_t w, uint32_t out[4],
                                                   const Unpack128 &c) {
    out[0] = and_or(w, c.mask, c.bias);
    out[1] = and_or(w >> 4, c.mask, c.bias);
    out[2] = and_or(w >> 8, c.mask, c.bias);
    out[3] = and_or(w >> 12, c.mask, c.bias);
}

// 8 consecutive bf16 (k = 0..7, as 4 dwords of pairs) -> the interleaved
// order k = 0,4,1,5,2,6,3,7 used by unpack8_bias128_il.
__device__ __forceinline__ u32x4 interleave8_bf16(u32x4 v) {
    u32x4 r;
    r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);   // (x0, x4)
    r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);   // (x1, x5)
    r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);   // (x2, x6)
    r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);   // (x3, x7)
    return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u32x4 u = {a, b, c, d};
    return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) {
    return __builtin_bit_cast(bf16x8, u);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// c + a.lo * b.lo + a.hi * b.hi for two bf16 pairs, accumulated in float32
// (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// Buffer resource over [p, p + bytes): loads at offsets past `bytes` return 0
// and fetch nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}

// Cache-policy operand for weights a kernel reads exactly once (the GEMVs):
// nt, streaming, so the lines are not kept in L2 and the reused operands (x,
// scales) stay there.
constexpr int W4_CPOL_STREAM = 2;

// bf16 1.0 in every element.
__device__ __forceinline__ bf16x8 bf16x8_ones() {
    return as_bf16x8(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
}

// 16 bytes per lane, global -> LDS: lane l writes LDS byte address lds
// (wave-uniform) + 16 l; inactive lanes write nothing. No output registers:
// the caller waits with an explicit s_waitcnt vmcnt before reading LDS.
__device__ __forceinline__ void lds_dma16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 : : "v"(g), "s"(lds) : "memory", "m0");
}

// LDS byte address of a __shared__ object.
template <typename P>
__device__ __forceinline__ uint32_t lds_address(P *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) const uint8_t *)(p)));
}

// D = A(16x32) * B(32x16) + C on the bf16 matrix cores.
// Lane l supplies A[l%16][8*(l/16) .. +8) and B[8*(l/16) .. +8)[l%16];
// it receives D[4*(l/16) + i][l%16] in element i.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

} // namespace w4
