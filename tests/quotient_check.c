/* Exhaustive host check of the INT8 quantizer's division shortcut.
 *
 * The quantizer defines code = clamp(round_half_even(x / scale), -127, 127)
 * with scale = amax / 127 and x / scale an IEEE fp32 division (glossary
 * monograph, section 5.1: Q = round(K / S); PagedKV-Fusion README,
 * "Overview": symmetric INT8 per (block, head)). The GPU kernel forms the
 * quotient without a division per element, with r = 1 / scale (IEEE):
 *     q0 = RN(x * r),  e = fma(-q0, scale, x),  q = fma(e, r, q0)
 * (a Markstein correction step), clamps q with a median-of-three to +-127 and
 * rounds to an integer by adding 1.5 * 2^23 (round half to even), keeping
 * the two's-complement code in the low byte. This program restates that
 * sequence in C (fmaf, IEEE single arithmetic) and compares, for every finite
 * fp16 amax > 0 and every fp16 x with |x| <= amax (both signs, zeros
 * included), the quotient with the IEEE division x / scale bit for bit and
 * the code with clamp(nearbyintf(x / scale)). It prints the number of pairs
 * checked and of mismatches of each kind.
 *
 * Build: gcc -O2 -mfma -ffp-contract=off -fopenmp quotient_check.c -o quotient_check
 * (x86-64 with SSE arithmetic: float operations round to single precision).
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float half_to_float(uint16_t h)
{
    const uint32_t sign = (uint32_t)(h >> 15) << 31;
    const uint32_t exp = (h >> 10) & 0x1F, man = h & 0x3FF;
    float v;
    if (exp == 0)
        v = ldexpf((float)man, -24); /* subnormal (exact) */
    else
        v = ldexpf((float)(man | 0x400), (int)exp - 25);
    uint32_t bits;
    memcpy(&bits, &v, 4);
    bits |= sign;
    memcpy(&v, &bits, 4);
    return v;
}

static uint32_t bits_of(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    return b;
}

int main(void)
{
    fesetround(FE_TONEAREST);
    long long pairs = 0, quot_bad = 0, code_bad = 0;
    /* amax runs over the positive finite fp16 values 0x0001 .. 0x7BFF */
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, quot_bad, code_bad)
    for (int ha = 1; ha <= 0x7BFF; ++ha) {
        const float amax = half_to_float((uint16_t)ha);
        const volatile float v127 = 127.0f;
        const float scale = amax / v127;
        const float r = 1.0f / scale;
        for (int hx = 0; hx <= ha; ++hx) {
            for (int sgn = 0; sgn < 2; ++sgn) {
                const float x = half_to_float((uint16_t)(hx | (sgn << 15)));
                /* the kernel's sequence */
                const float q0 = x * r;
                const float e = fmaf(-q0, scale, x);
                const float q = fmaf(e, r, q0);
                const float c = q < -127.0f ? -127.0f : (q > 127.0f ? 127.0f : q);
                const float shifted = c + 12582912.0f;
                const int8_t code = (int8_t)(bits_of(shifted) & 0xFF);
                /* the definition */
                const float want_q = x / scale;
                float want_c = nearbyintf(want_q);
                want_c = want_c < -127.0f ? -127.0f : (want_c > 127.0f ? 127.0f : want_c);
                /* equal quotients, zeros of either sign counted equal */
                if (bits_of(q) != bits_of(want_q) && !(q == 0.0f && want_q == 0.0f)) ++quot_bad;
                if ((int)code != (int)want_c) ++code_bad;
                ++pairs;
            }
        }
    }
    printf("pairs %lld quotient_mismatches %lld code_mismatches %lld\n", pairs, quot_bad, code_bad);
    return 0;
}
