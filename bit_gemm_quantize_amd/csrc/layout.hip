// Pre-shuffled weight layout for gfx950: a one-time repack of the plain
// int4 format.
//
// codes_ps[n, 4j .. 4j + 4) is one little-endian 32-bit word holding the
// eight codes of k = 8j .. 8j + 7 with the even-k codes in nibbles 0..3 and
// the odd-k codes in nibbles 4..7:
//   nibble i = q[n, 8j + 2i], nibble 4 + i = q[n, 8j + 2i + 1]   (i = 0..3).
// (w >> 4i) & 0x000F000F then holds the pair (q[8j + 2i], q[8j + 2i + 1]) in
// natural order, so the exact-integer bf16 expansion 0x4300 | q costs one
// shift and one and-or per pair without reordering the activations.
// sz[n, g] = scales[n, g] | zeros[n, g] << 16: one 4-byte load per group.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

__device__ __forceinline__ uint32_t preshuffle_word(uint32_t w) {
    const uint32_t e = w & 0x0F0F0F0Fu;          // q0, q2, q4, q6 in the bytes' low nibbles
    const uint32_t o = (w >> 4) & 0x0F0F0F0Fu;   // q1, q3, q5, q7
    const uint32_t e2 = e | (e >> 4);            // byte 0: q0 | q2 << 4, byte 2: q4 | q6 << 4
    const uint32_t o2 = o | (o >> 4);            // byte 0: q1 | q3 << 4, byte 2: q5 | q7 << 4
    return (e2 & 0xFFu) | ((e2 >> 8) & 0xFF00u) | ((o2 & 0xFFu) << 16) | ((o2 << 8) & 0xFF000000u);
}

// one 16-byte piece (four words) of codes per thread, grid-stride
__global__ __launch_bounds__(256) void repack_codes_kernel(const u32x4 *__restrict__ in,
                                                           u32x4 *__restrict__ out, int64_t n16) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const u32x4 v = in[i];
        out[i] = u32x4{preshuffle_word(v.x), preshuffle_word(v.y), preshuffle_word(v.z),
                       preshuffle_word(v.w)};
    }
}

__global__ __launch_bounds__(256) void pair_sz_kernel(const uint16_t *__restrict__ s,
                                                      const uint16_t *__restrict__ z,
                                                      uint32_t *__restrict__ sz, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * 256)
        sz[i] = static_cast<uint32_t>(s[i]) | (static_cast<uint32_t>(z[i]) << 16);
}

} // namespace

hipError_t launch_repack(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros,
                         int64_t N, int64_t K, int G, uint8_t *codes_ps, uint32_t *sz,
                         hipStream_t stream) {
    // K is a multiple of G >= 32, so every row is a whole number of 16-byte pieces
    const int64_t n16 = N * K / 32;
    const int64_t ng = N * (K / G);
    const int64_t cap = static_cast<int64_t>(compute_units()) * 8;
    const int64_t w1 = (n16 + 255) / 256, w2 = (ng + 255) / 256;
    const int b1 = static_cast<int>(w1 < cap ? w1 : cap);
    const int b2 = static_cast<int>(w2 < cap ? w2 : cap);
    repack_codes_kernel<<<dim3(b1), dim3(256), 0, stream>>>(
        reinterpret_cast<const u32x4 *>(codes), reinterpret_cast<u32x4 *>(codes_ps), n16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    pair_sz_kernel<<<dim3(b2), dim3(256), 0, stream>>>(scales, zeros, sz, ng);
    return hipGetLastError();
}

} // namespace w4
