/*
 * Exhaustive pin of the oracle's fp32 -> e4m3fn encoder (test helper, CPU only).
 *
 * For every one of the 2^32 fp32 bit patterns, the oracle's code must equal the answer of a
 * brute-force search written from the format definition alone: among the 127 non-negative
 * finite e4m3fn values (m * 2^-9 for exponent field 0, (8 + m) * 2^(E - 10) otherwise,
 * E = 1..15 except the NaN pattern E = 15, m = 7) take the one nearest to |x|, on a tie the
 * one whose code is even; magnitudes at or above 448 saturate to 448; keep the sign of x;
 * NaN maps to 0x7F. Prints the number of mismatches and the first few.
 * Usage: e4m3_exhaustive [start_hi16 end_hi16]   (range of the top 16 bits, default all)
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint8_t orc_e4m3_encode(float x);

static double vals[127];

static uint8_t brute(float x) {
    if (isnan(x)) return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs((double)x);
    if (a >= 448.0) return sign | 0x7E;
    /* vals[] ascends with the code: bisect for the last value <= a, then compare the two
     * neighbours around a */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (vals[mid] <= a) lo = mid; else hi = mid - 1;
    }
    int best = lo;
    if (lo < 126) {
        double dl = a - vals[lo], dh = vals[lo + 1] - a;
        if (dh < dl || (dh == dl && ((lo + 1) & 1) == 0)) best = lo + 1;
    }
    return sign | (uint8_t)best;
}

int main(int argc, char** argv) {
    for (int c = 0; c < 127; ++c) {
        int E = c >> 3, m = c & 7;
        vals[c] = E == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), E - 10);
    }
    long lo = 0, hi = 65536;
    if (argc == 3) { lo = atol(argv[1]); hi = atol(argv[2]); }
    long long bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(+ : bad)
    for (long h = lo; h < hi; ++h) {
        for (uint32_t l = 0; l < 65536; ++l) {
            uint32_t u = ((uint32_t)h << 16) | l;
            float x;
            memcpy(&x, &u, 4);
            uint8_t a = orc_e4m3_encode(x), b = brute(x);
            if (a != b) {
                if (bad < 5) {
#pragma omp critical
                    fprintf(stderr, "mismatch x=%a (0x%08x): oracle 0x%02x brute 0x%02x\n", x, u, a, b);
                }
                ++bad;
            }
        }
    }
    printf("%lld\n", bad);
    return bad != 0;
}
