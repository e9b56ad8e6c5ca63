/* Exhaustive check of the per-block reciprocal division used by the quantize
 * kernel for bf16 and fp16 inputs (CPU only; this is a proof of the kernel's
 * arithmetic, not part of the oracle).
 *
 * For every pair (x, a) of the input format with a > 0 finite and |x| <= a,
 * inside the region where the kernel takes the fast path,
 *     block:   2^-36 <= a <= 2^64
 *     element: |x| >= a * 2^-64      (so x = 0 is outside: the kernel divides
 *                                     such elements with the IEEE sequence)
 * it compares
 *     r  = RN(1/a)                (once per block, IEEE division)
 *     q0 = RN(x*r)
 *     e  = RN(x - q0*a)           (fused multiply-add; exact in this region)
 *     q1 = RN(q0 + e*r)           (fused multiply-add)
 * with the correctly rounded quotient RN(x/a).  This is Markstein's correction
 * step (P. Markstein, "Computation of elementary functions on the IBM RISC
 * System/6000 processor", IBM J. Res. Dev. 34(1), 1990).  Outside the region the
 * residual e can underflow or the quotient is subnormal and the step is not
 * exact, which is why the kernel falls back there.
 *
 * The reciprocal itself is not an IEEE division in the kernel: it is the
 * hardware's approximate reciprocal y (within 1 ulp of 1/a) refined by one
 * correction step, r = RN(y + RN(1 - a*y)*y) with two fused multiply-adds.  For
 * every a of the fast region and every binary32 y within 2 ulp of 1/a (twice the
 * hardware's error bound) the program checks r == RN(1/a) first.
 *
 * usage: div_check bf16|fp16      prints "recips R recip_mismatches M1" and
 *                                 "pairs P fast F mismatches M"; exit 0 iff M1 == M == 0
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#define A_MIN_EXP (-36)
#define A_MAX_EXP 64
#define X_REL_EXP (-64)

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static float bf16_to_f(uint16_t h) { return from_bits((uint32_t)h << 16); }
static float fp16_to_f(uint16_t h) {
    uint32_t s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), (int)e - 25);
    return s ? -v : v;
}

int main(int argc, char** argv) {
    int is_bf16 = !(argc > 1 && strcmp(argv[1], "fp16") == 0);
    uint32_t top = is_bf16 ? 0x7F7F : 0x7BFF;   /* largest finite positive pattern */
    const float a_lo = ldexpf(1.0f, A_MIN_EXP), a_hi = ldexpf(1.0f, A_MAX_EXP);
    unsigned long long pairs = 0, fast = 0, bad = 0, recips = 0, rbad = 0;
    for (uint32_t ab = 1; ab <= top; ++ab) {
        float a = is_bf16 ? bf16_to_f((uint16_t)ab) : fp16_to_f((uint16_t)ab);
        if (!(a >= a_lo && a <= a_hi)) continue;
        volatile float one = 1.0f;
        const float rn = one / a;
        const double inv = 1.0 / (double)a;
        const double ulp = (double)nextafterf(rn, INFINITY) - (double)rn;
        float y = nextafterf(nextafterf(nextafterf(rn, 0.0f), 0.0f), 0.0f);
        for (int k = 0; k < 7; ++k, y = nextafterf(y, INFINITY)) {
            if (fabs((double)y - inv) > 2.0 * ulp) continue;
            ++recips;
            const float r = fmaf(fmaf(-a, y, 1.0f), y, y);
            if (memcmp(&r, &rn, 4) != 0) {
                if (rbad < 10) printf("reciprocal mismatch a=%a y=%a got=%a want=%a\n", a, y, r, rn);
                ++rbad;
            }
        }
    }
    printf("recips %llu recip_mismatches %llu\n", recips, rbad);
    for (uint32_t ab = 1; ab <= top; ++ab) {
        float a = is_bf16 ? bf16_to_f((uint16_t)ab) : fp16_to_f((uint16_t)ab);
        int block_fast = a >= a_lo && a <= a_hi;
        volatile float one = 1.0f;
        float r = one / a;
        float x_lo = ldexpf(a, X_REL_EXP);
        for (uint32_t xb = 0; xb <= ab; ++xb) {
            for (int sgn = 0; sgn < 2; ++sgn) {
                uint16_t pat = (uint16_t)(xb | (sgn ? 0x8000u : 0u));
                float x = is_bf16 ? bf16_to_f(pat) : fp16_to_f(pat);
                ++pairs;
                if (!block_fast || !(fabsf(x) >= x_lo)) continue;
                ++fast;
                float ref = x / a;
                float q0 = x * r;
                float e = fmaf(-q0, a, x);
                float q1 = fmaf(e, r, q0);
                if (memcmp(&q1, &ref, 4) != 0) {
                    if (bad < 10) printf("mismatch a=%a x=%a ref=%a got=%a\n", a, x, ref, q1);
                    ++bad;
                }
            }
        }
    }
    printf("pairs %llu fast %llu mismatches %llu\n", pairs, fast, bad);
    return bad != 0 || rbad != 0;
}
