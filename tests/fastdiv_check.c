/*
 * Exhaustive check of the division scheme the activation kernel uses for
 * bf16 inputs (host test; no GPU):
 *     y  = RN(1 / s)                 (one IEEE binary32 division per channel)
 *     q0 = RN(x * y)
 *     q1 = RN(q0 + RN-exact(x - q0 * s) * y)   i.e. fma(fma(-q0, s, x), y, q0)
 * must equal RN(x / s), the correctly rounded IEEE quotient, whenever
 * 2^-50 <= |q0| <= 2^120 (the kernel divides exactly otherwise; x = 0 is
 * exact as well).
 *
 * Every operation is a correctly rounded binary32 operation, so scaling x
 * and s by powers of two scales every intermediate exactly as long as none
 * of them underflows or overflows, which the guard on |q0| (with s in the
 * floored range of the method) ensures. It therefore suffices to check
 * x in [1, 2) with an 8-bit significand (every bf16 significand) against
 * every binary32 significand of s in [1, 2): 128 * 2^23 = 2^30 cases,
 * covering quotients in (1/2, 2), both result binades. A second pass checks
 * random x, s with random exponents inside the guard.
 *
 * Build: gcc -O2 -mfma -fopenmp -ffp-contract=off (fmaf is the hardware
 * fused multiply-add). Prints the number of mismatches; exit status 0 iff
 * there are none.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

static int fast_ok(float x, float s, float* out) {
    float y = 1.0f / s;
    float q0 = x * y;
    float e = fmaf(-q0, s, x);
    float q1 = fmaf(e, y, q0);
    *out = q1;
    float a = fabsf(q0);
    return (a >= 0x1p-50f && a <= 0x1p120f) || q0 == 0.0f;
}

int main(void) {
#ifndef __FMA__
    printf("no hardware FMA on this host: skipped\n");
    return 77;
#endif
    long long bad = 0, guarded_out = 0;
#pragma omp parallel for reduction(+ : bad, guarded_out) schedule(static)
    for (uint32_t sm = 0; sm < (1u << 23); ++sm) {
        float s = from_bits(0x3F800000u | sm);            /* s in [1, 2) */
        for (uint32_t xm = 0; xm < 128; ++xm) {
            float x = from_bits(0x3F800000u | (xm << 16)); /* bf16 x in [1, 2) */
            float q1;
            if (!fast_ok(x, s, &q1)) { ++guarded_out; continue; }
            float q = x / s;
            if (q1 != q) ++bad;
            /* the negative operand gives the negated results */
            float qn;
            fast_ok(-x, s, &qn);
            if (qn != -q) ++bad;
        }
    }
    printf("exhaustive: %lld mismatches, %lld outside the guard (of %lld)\n", bad, guarded_out,
           128LL << 23);
    /* random exponents inside the guard */
    uint64_t st = 0x9E3779B97F4A7C15ull;
    long long rbad = 0, rn = 0;
    for (long i = 0; i < 20000000; ++i) {
        st ^= st << 13; st ^= st >> 7; st ^= st << 17;
        uint32_t xm = (uint32_t)(st & 0x7F), xe = 127 - 50 + (uint32_t)((st >> 8) % 121);
        uint32_t sm = (uint32_t)((st >> 16) & 0x7FFFFF), se = 127 - 27 + (uint32_t)((st >> 40) % 60);
        float x = from_bits((xe << 23) | (xm << 16) | ((st >> 63) << 31));
        float s = from_bits((se << 23) | sm);
        float q1;
        if (!fast_ok(x, s, &q1)) continue;
        ++rn;
        if (q1 != x / s) ++rbad;
    }
    printf("random exponents: %lld mismatches of %lld\n", rbad, rn);
    return (bad || rbad) ? 1 : 0;
}
