// The quantizer computes its scale (hi - lo) / 15 as
//   q0 = a * y, q1 = fma(fma(-15, q0, a), y, q0),  y = RN(1/15),
// instead of a divide. This program checks, for every positive finite
// binary32 a (denormals included), that q1 is the correctly rounded IEEE
// quotient, and that both round to the same bf16. Prints the mismatch counts.
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <omp.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t b(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
int main(void) {
    const float y = 1.0f / 15.0f;
    long bad = 0, bad16 = 0;
    uint32_t first = 0;
    #pragma omp parallel for reduction(+:bad,bad16) schedule(static)
    for (long i = 0; i <= 0x7F7FFFFFL; ++i) {
        const float a = f((uint32_t)i);
        volatile float ref = a / 15.0f;
        const float q0 = a * y;
        const float r = fmaf(-15.0f, q0, a);
        const float q1 = fmaf(r, y, q0);
        if (b(q1) != b(ref)) { bad++; }
        // bf16 round to nearest even of both
        uint32_t u1 = b(q1), ur = b(ref);
        uint32_t h1 = (u1 + 0x7FFF + ((u1 >> 16) & 1)) >> 16;
        uint32_t hr = (ur + 0x7FFF + ((ur >> 16) & 1)) >> 16;
        if (h1 != hr) bad16++;
    }
    printf("y=%a mismatches fp32=%ld bf16=%ld\n", y, bad, bad16);
    return 0;
}
