/* Exhaustive check of the quotient sequence the device codec uses for the
 * column scales c = m / Qb (div_by_qmax in the library's codec): for every
 * positive finite fp32 m,
 *     q0 = RN(m * r),  e = fma(-q0, Qb, m),  q1 = fma(e, r, q0),  r = RN(1/Qb)
 * must be RN(m / Qb), the correctly rounded quotient.  Every operation of the
 * sequence is one IEEE fp32 operation, so the CPU's results are the GPU's.
 * q1 >= 0 is RN(m / Qb) exactly when the residual d = m - q1 Qb (exact in
 * fp64: q1 Qb has at most 31 significant bits) satisfies |d| < h, or
 * |d| == h with q1's significand even, where h = ulp(q1) Qb / 2 and ulp(q1)
 * is the spacing of fp32 values at q1 (2^-149 below the normal range).
 * Prints "Qb mismatches" per constant.
 * Build: gcc -O2 -fopenmp -ffp-contract=off division_check.c -lm */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_to_float(uint32_t u)
{
    float x;
    memcpy(&x, &u, 4);
    return x;
}

static uint32_t float_to_bits(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return u;
}

static double pow2(int e)  /* 2^e as a double, e in the normal fp64 range */
{
    const uint64_t b = (uint64_t)(e + 1023) << 52;
    double d;
    memcpy(&d, &b, 8);
    return d;
}

int main(void)
{
    const float qbs[3] = {127.0f, 31.0f, 7.0f};
    for (int k = 0; k < 3; k++) {
        const float qb = qbs[k];
        const float r = (float)(1.0 / (double)qb);
        unsigned long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
        for (long long i = 1; i < 0x7f800000LL; i++) {
            const float m = bits_to_float((uint32_t)i);
            const float q0 = m * r;
            const float q1 = fmaf(fmaf(-q0, qb, m), r, q0);
            const uint32_t qbits = float_to_bits(q1);
            const int ex = (int)(qbits >> 23);                 /* q1 >= 0: sign bit clear */
            const double ulp = pow2((ex > 0 ? ex : 1) - 150);
            const double d = fabs((double)m - (double)q1 * (double)qb);
            const double h = 0.5 * ulp * (double)qb;
            const int ok = (d < h) || (d == h && (qbits & 1u) == 0);
            bad += !ok;
        }
        printf("%g %llu\n", qb, bad);
    }
    return 0;
}
