/* The device token quantizer divides by the group scale as q = x * r, r = 1 / s (one IEEE
 * division per group), corrected once by the exact remainder: y = copysign(fma(e, r, q), x)
 * with e = fma(-q, s, x). This program checks that the code of y equals the code of the IEEE
 * quotient x / s -- the quotient the oracle encodes -- for every finite positive bf16 amax
 * and every bf16 x with |x| <= amax (both signs, zeros and subnormals included), with
 * s = max(amax, eps) / Qmax (eps = 1e-10; Qmax = 448 for e4m3fn, 127 for int8) and with s
 * rounded up to a power of two (the UE8M0 scale format). The encoders are the oracle's.
 * Prints the number of mismatching codes (0 expected); the first few mismatches go to stderr.
 * Build: gcc -O2 -fopenmp -ffp-contract=off quotient_codes.c -loracle -lm */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint8_t orc_e4m3_encode(float x);
int8_t orc_int8_encode(float x);

static float bf16_value(uint32_t bits) {
    const uint32_t u = bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* the smallest power of two >= v (v > 0, normal) */
static float pow2_ceil(float v) {
    int ex;
    const float m = frexpf(v, &ex);   /* v = m * 2^ex, m in [0.5, 1) */
    return ldexpf(1.0f, m == 0.5f ? ex - 1 : ex);
}

int main(void) {
    const float eps = 1e-10f;
    long long bad = 0;
    for (int mode = 0; mode < 4; ++mode) {
        const int int8 = mode & 1, ue8m0 = mode >> 1;
        const float qmax = int8 ? 127.0f : 448.0f;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad)
        for (uint32_t ab = 1; ab < 0x7F80u; ++ab) {          /* finite positive amax */
            const float amax = bf16_value(ab);
            float s = (amax > eps ? amax : eps) / qmax;
            if (ue8m0) s = pow2_ceil(s);
            const float r = 1.0f / s;
            for (uint32_t xb = 0; xb <= ab; ++xb) {
                for (uint32_t sign = 0; sign < 2; ++sign) {
                    const float x = bf16_value(xb | (sign << 15));
                    const float ieee = x / s;
                    const float q = x * r;
                    const float e = fmaf(-q, s, x);
                    const float y = copysignf(fmaf(e, r, q), x);
                    const int differ = int8 ? orc_int8_encode(y) != orc_int8_encode(ieee)
                                            : orc_e4m3_encode(y) != orc_e4m3_encode(ieee);
                    if (differ) {
#pragma omp critical
                        if (bad < 5)
                            fprintf(stderr, "int8=%d ue8m0=%d amax=%a x=%a ieee=%a corrected=%a\n",
                                    int8, ue8m0, amax, x, ieee, y);
                        ++bad;
                    }
                }
            }
        }
    }
    printf("%lld\n", bad);
    return 0;
}
