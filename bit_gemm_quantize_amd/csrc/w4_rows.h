// Helpers shared by the row-run decode kernels of the int8 weight-only and
// W4A8 paths (a wave holds partial sums of four output rows in every lane).
#pragma once

#include "w4_device.h"

namespace w4 {

// Sum over the 64 lanes of four row partials; every lane of quarter r ends
// with row r's sum.
__device__ __forceinline__ float sum_rows4(float v0, float v1, float v2, float v3) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
    const float u02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
    const float u13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(u02), __float_as_uint(u13), false, false);
    return group_sum<16>(__uint_as_float(c[0]) + __uint_as_float(c[1]));
}

} // namespace w4
